"""ctypes binding of libalspec.so: argument marshalling only.

Every step of the speculative flash-decode path runs in the library's HIP
kernels; this module checks tensor shapes, dtypes and devices, packs the
parameter struct, and passes raw device pointers and stream handles.  There
is no fallback: if the library is not built, importing the package fails.
"""
import ctypes
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
IN_TREE_LIB = os.path.join(HERE, "libalspec.so")
# ALSPEC_LIB selects another build of the same library (e.g. a variant
# built with different compile-time options) for timing comparisons; the
# benchmark records the path it loaded.  The test suite always checks the
# in-tree build: under pytest a different path is refused.
LIB_PATH = os.environ.get("ALSPEC_LIB") or IN_TREE_LIB
if "pytest" in sys.modules and (os.path.realpath(LIB_PATH) !=
                                os.path.realpath(IN_TREE_LIB)):
    raise ImportError(f"ALSPEC_LIB={LIB_PATH} is not honoured under pytest: "
                      "the tests check the in-tree library")

KV_F32 = 0
KV_BF16 = 1
STATUS = {0: "ALSPEC_OK", 1: "ALSPEC_ERR_INVALID_ARG",
          2: "ALSPEC_ERR_UNSUPPORTED", 3: "ALSPEC_ERR_WORKSPACE",
          4: "ALSPEC_ERR_HIP"}
MAX_BATCH = 64
# ALSPEC_LAYERS_WS_RING: layers fewer than this apart in one
# spec_decode_layers call must not share a workspace
LAYERS_WS_RING = 3

# One HIP runtime per process: torch ships its own libamdhip64 (same SONAME
# as the system one).  Loading torch first makes this library bind to the
# runtime torch already holds instead of pulling in a second copy, which
# would not see the device that torch has opened.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c "
        "'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_i32 = ctypes.c_int32


class Params(ctypes.Structure):
    """Mirror of alspec_params."""
    _fields_ = [("batch", _i32), ("num_q_heads", _i32),
                ("num_kv_heads", _i32), ("head_dim", _i32),
                ("kv_capacity", _i32), ("seq_lens", ctypes.POINTER(_i32)),
                ("kv_dtype", _i32), ("sink", _i32), ("window", _i32),
                ("sm_scale", ctypes.c_float), ("lam", ctypes.c_float),
                ("split_tokens", _i32), ("window_split_tokens", _i32),
                ("overlap", _i32)]


class Events(ctypes.Structure):
    """Mirror of alspec_events (hipEvent_t handles, may be None)."""
    _fields_ = [("approx_begin", _P), ("approx_end", _P),
                ("exact_begin", _P), ("exact_end", _P), ("verify_end", _P)]


class Layer(ctypes.Structure):
    """Mirror of alspec_layer (device pointers)."""
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("o_approx", _P),
                ("lse_approx", _P), ("o_exact", _P), ("lse_exact", _P),
                ("ratio", _P), ("commit", _P), ("o_committed", _P),
                ("ws", _P), ("ws_bytes", ctypes.c_size_t)]


def _sig(name, *args):
    f = getattr(_lib, name)
    f.restype = ctypes.c_int
    f.argtypes = list(args)
    return f


_PP = ctypes.POINTER(Params)
_status_string = getattr(_lib, "alspec_status_string")
_status_string.restype = ctypes.c_char_p
_status_string.argtypes = [ctypes.c_int]
_last_error = getattr(_lib, "alspec_last_error")
_last_error.restype = ctypes.c_char_p
_last_error.argtypes = []
_version = getattr(_lib, "alspec_version")
_version.restype = _i32
_workspace_size = _sig("alspec_workspace_size", _PP,
                       ctypes.POINTER(ctypes.c_size_t))
_plan_splits = _sig("alspec_plan_splits", _PP, _i32, _P, _P, _P, _i32,
                    ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                    ctypes.POINTER(_i32))
_create = _sig("alspec_create", ctypes.c_int, ctypes.POINTER(_P))
_destroy = _sig("alspec_destroy", _P)
_sink_approx = _sig("alspec_sink_approx", _P, _PP, _P, _P, _P, _P, _P, _P,
                    ctypes.c_size_t, _P)
_flash_exact = _sig("alspec_flash_decode_exact", _P, _PP, _P, _P, _P, _i32,
                    _P, ctypes.c_size_t, _P)
_lse_combine = _sig("alspec_lse_combine", _P, _PP, _P, ctypes.c_size_t, _P,
                    _P, _P)
_verify = _sig("alspec_verify", _P, _PP, _P, _P, _P, _P, _P, _P)
_order_after_verify = _sig("alspec_order_after_verify", _P, _P)
_spec_decode_layers = _sig("alspec_spec_decode_layers", _P, _PP, _i32,
                           ctypes.POINTER(Layer), _P)
_spec_decode_noalloc = _sig("alspec_spec_decode_noalloc", _P, _PP, _P, _P,
                            _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                            ctypes.POINTER(Events))
NOALLOC_SCRATCH_BYTES = 16 << 20
_spec_decode = _sig("alspec_spec_decode", _P, _PP, _P, _P, _P, _P, _P, _P,
                    _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P,
                    ctypes.POINTER(Events))


class AlspecError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = f"{what}: {status_string(status)}"
        if int(status) == 4:               # ALSPEC_ERR_HIP
            msg += f" ({last_error()})"
        super().__init__(msg)


def last_error():
    """The HIP call and error behind this thread's last ALSPEC_ERR_HIP."""
    return _last_error().decode()


def status_string(st):
    return _status_string(int(st)).decode()


def version():
    return int(_version())


def _check(st, what):
    if st != 0:
        raise AlspecError(st, what)


def make_params(batch, num_q_heads, num_kv_heads, head_dim, kv_capacity,
                seq_lens, kv_dtype, sink, window, lam, sm_scale=None,
                split_tokens=0, window_split_tokens=0, overlap=0):
    """Build an alspec_params.  kv_dtype is "f32" or "bf16" (or 0/1).  The
    returned struct keeps its host seq_lens array alive."""
    if isinstance(kv_dtype, str):
        kv_dtype = {"f32": KV_F32, "bf16": KV_BF16}[kv_dtype]
    lens = (_i32 * max(1, len(seq_lens)))(*[int(x) for x in seq_lens])
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    p = Params(int(batch), int(num_q_heads), int(num_kv_heads),
               int(head_dim), int(kv_capacity),
               ctypes.cast(lens, ctypes.POINTER(_i32)), int(kv_dtype),
               int(sink), int(window), float(sm_scale), float(lam),
               int(split_tokens), int(window_split_tokens), int(overlap))
    p._lens = lens  # keep alive
    return p


def params_for(w, **kw):
    """alspec_params of a synthetic workload description (synth.gen)."""
    args = dict(split_tokens=0, window_split_tokens=0, lam=w.lam)
    args.update(kw)
    return make_params(w.B, w.Hq, w.Hkv, w.D, w.L_cap, w.seq_lens,
                       w.kv_dtype, w.S, w.W, **args)


def workspace_size(p):
    n = ctypes.c_size_t(0)
    _check(_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "alspec_workspace_size")
    return int(n.value)


def plan_splits(p, b):
    """[(kind, begin, end)] of batch entry b (kind 0 sink, 1 window, 2
    middle), plus the (middle, window) split lengths.  Every entry point
    takes this plan."""
    name = "alspec_plan_splits"
    cnt = _i32(0)
    t = _i32(0)
    tw = _i32(0)
    _check(_plan_splits(ctypes.byref(p), b, None, None, None, 0,
                        ctypes.byref(cnt), ctypes.byref(t), ctypes.byref(tw)),
           name)
    n = cnt.value
    kind = (_i32 * max(1, n))()
    beg = (_i32 * max(1, n))()
    end = (_i32 * max(1, n))()
    _check(_plan_splits(ctypes.byref(p), b, kind, beg, end, n,
                        ctypes.byref(cnt), None, None), name)
    return [(kind[i], beg[i], end[i]) for i in range(n)], (t.value, tw.value)


def symbols():
    """Names exported by the loaded library that the header declares."""
    return _lib


# ------------------------------------------------------------ device side ---

def _torch():
    import torch
    return torch


def _ptr(t, dtype, shape, name, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, want {shape}")
    del torch
    return t.data_ptr()


def _kv_torch_dtype(p):
    torch = _torch()
    return torch.bfloat16 if p.kv_dtype == KV_BF16 else torch.float32


_hip = None


def stream_is_capturing(s):
    """Whether torch stream `s` is recording into a HIP graph (asked of the
    HIP runtime torch loaded, reached by its soname)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipStreamIsCapturing.argtypes = [_P, ctypes.POINTER(ctypes.c_int)]
        _hip.hipStreamIsCapturing.restype = ctypes.c_int
    status = ctypes.c_int(0)
    err = _hip.hipStreamIsCapturing(_P(s.cuda_stream), ctypes.byref(status))
    if err != 0:
        raise RuntimeError(f"hipStreamIsCapturing failed ({err})")
    return status.value == 1        # hipStreamCaptureStatusActive


def _stream(s):
    torch = _torch()
    if s is None:
        s = torch.cuda.current_stream()
    return s.cuda_stream


class Handle:
    """alspec_handle bound to one device."""

    def __init__(self, device=0):
        h = _P()
        _check(_create(int(device), ctypes.byref(h)), "alspec_create")
        self._h = h
        self.device = device

    @property
    def ptr(self):
        if self._h is None:
            raise ValueError("handle is closed")
        return self._h

    def close(self):
        if self._h is not None:
            _destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def alloc_workspace(p, device="cuda"):
    """Zero-filled device workspace of the required size (256-aligned)."""
    torch = _torch()
    n = workspace_size(p)
    ws = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def alloc_outputs(p, device="cuda"):
    """Output tensors of one fused call."""
    torch = _torch()
    B, Hq, D = p.batch, p.num_q_heads, p.head_dim
    f = dict(dtype=torch.float32, device=device)
    return {
        "o_approx": torch.empty((B, Hq, D), **f),
        "lse_approx": torch.empty((B, Hq), **f),
        "o_exact": torch.empty((B, Hq, D), **f),
        "lse_exact": torch.empty((B, Hq), **f),
        "ratio": torch.empty((B,), **f),
        "commit": torch.empty((B,), dtype=torch.uint8, device=device),
        "o_committed": torch.empty((B, Hq, D), **f),
    }


def _qkv(p, q, k, v):
    torch = _torch()
    B, Hq, Hkv, D, L = (p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim,
                        p.kv_capacity)
    kd = _kv_torch_dtype(p)
    return (_ptr(q, torch.float32, (B, Hq, D), "q"),
            _ptr(k, kd, (B, Hkv, L, D), "k"),
            _ptr(v, kd, (B, Hkv, L, D), "v"))


def _ws(ws):
    torch = _torch()
    return _ptr(ws, torch.uint8, None, "ws"), ws.numel()


def sink_approx(h, p, q, k, v, o_approx, lse_approx, ws, stream=None):
    torch = _torch()
    qp, kp, vp = _qkv(p, q, k, v)
    B, Hq, D = p.batch, p.num_q_heads, p.head_dim
    wp, wn = _ws(ws)
    _check(_sink_approx(h.ptr, ctypes.byref(p), qp, kp, vp,
                        _ptr(o_approx, torch.float32, (B, Hq, D), "o_approx"),
                        _ptr(lse_approx, torch.float32, (B, Hq), "lse_approx",
                             True), wp, wn, _stream(stream)),
           "alspec_sink_approx")


def flash_decode_exact(h, p, q, k, v, include_sink_window, ws, stream=None):
    qp, kp, vp = _qkv(p, q, k, v)
    wp, wn = _ws(ws)
    _check(_flash_exact(h.ptr, ctypes.byref(p), qp, kp, vp,
                        int(include_sink_window), wp, wn, _stream(stream)),
           "alspec_flash_decode_exact")


def lse_combine(h, p, ws, o_exact, lse_exact, stream=None):
    torch = _torch()
    B, Hq, D = p.batch, p.num_q_heads, p.head_dim
    wp, wn = _ws(ws)
    _check(_lse_combine(h.ptr, ctypes.byref(p), wp, wn,
                        _ptr(o_exact, torch.float32, (B, Hq, D), "o_exact"),
                        _ptr(lse_exact, torch.float32, (B, Hq), "lse_exact",
                             True), _stream(stream)), "alspec_lse_combine")


def verify(h, p, o_approx, o_exact, ratio, commit, o_committed=None,
           stream=None):
    torch = _torch()
    B, Hq, D = p.batch, p.num_q_heads, p.head_dim
    _check(_verify(h.ptr, ctypes.byref(p),
                   _ptr(o_approx, torch.float32, (B, Hq, D), "o_approx"),
                   _ptr(o_exact, torch.float32, (B, Hq, D), "o_exact"),
                   _ptr(ratio, torch.float32, (B,), "ratio"),
                   _ptr(commit, torch.uint8, (B,), "commit"),
                   _ptr(o_committed, torch.float32, (B, Hq, D), "o_committed",
                        True), _stream(stream)), "alspec_verify")


def spec_decode(h, p, q, k, v, out, ws, stream_approx=None,
                stream_exact=None, events=None):
    """Fused step.  `out` is a dict as made by alloc_outputs (lse_* and
    o_committed may be None).  `events`: dict of torch.cuda.Event by
    alspec_events member name, or None; each event must have been recorded
    once already (torch creates the underlying hipEvent on first record)."""
    torch = _torch()
    qp, kp, vp = _qkv(p, q, k, v)
    B, Hq, D = p.batch, p.num_q_heads, p.head_dim
    wp, wn = _ws(ws)
    ev = None
    if events:
        ev = Events(*[events[n].cuda_event if events.get(n) is not None
                      else None for n in ("approx_begin", "approx_end",
                                          "exact_begin", "exact_end",
                                          "verify_end")])
    sa = _stream(stream_approx)
    se = _stream(stream_exact if stream_exact is not None else stream_approx)
    _check(_spec_decode(
        h.ptr, ctypes.byref(p), qp, kp, vp,
        _ptr(out["o_approx"], torch.float32, (B, Hq, D), "o_approx"),
        _ptr(out.get("lse_approx"), torch.float32, (B, Hq), "lse_approx",
             True),
        _ptr(out["o_exact"], torch.float32, (B, Hq, D), "o_exact"),
        _ptr(out.get("lse_exact"), torch.float32, (B, Hq), "lse_exact", True),
        _ptr(out["ratio"], torch.float32, (B,), "ratio"),
        _ptr(out["commit"], torch.uint8, (B,), "commit"),
        _ptr(out.get("o_committed"), torch.float32, (B, Hq, D),
             "o_committed", True),
        wp, wn, sa, se, ctypes.byref(ev) if ev is not None else None),
        "alspec_spec_decode")


def spec_decode_noalloc(h, p, q, k, v, out, stream_approx=None,
                        stream_exact=None):
    """The fused step with the library's static scratch as its workspace
    (alspec_spec_decode_noalloc): no workspace argument, nothing
    allocated.  Calls that overlap in time on one GPU race."""
    torch = _torch()
    qp, kp, vp = _qkv(p, q, k, v)
    B, Hq, D = p.batch, p.num_q_heads, p.head_dim
    sa = _stream(stream_approx)
    se = _stream(stream_exact if stream_exact is not None else stream_approx)
    _check(_spec_decode_noalloc(
        h.ptr, ctypes.byref(p), qp, kp, vp,
        _ptr(out["o_approx"], torch.float32, (B, Hq, D), "o_approx"),
        _ptr(out.get("lse_approx"), torch.float32, (B, Hq), "lse_approx",
             True),
        _ptr(out["o_exact"], torch.float32, (B, Hq, D), "o_exact"),
        _ptr(out.get("lse_exact"), torch.float32, (B, Hq), "lse_exact", True),
        _ptr(out["ratio"], torch.float32, (B,), "ratio"),
        _ptr(out["commit"], torch.uint8, (B,), "commit"),
        _ptr(out.get("o_committed"), torch.float32, (B, Hq, D),
             "o_committed", True), sa, se, None),
        "alspec_spec_decode_noalloc")


def layers_struct(p, layers):
    """ctypes array of alspec_layer from (q, k, v, out, ws) tuples (out as
    made by alloc_outputs); checks shapes and dtypes."""
    torch = _torch()
    B, Hq, D = p.batch, p.num_q_heads, p.head_dim
    arr = (Layer * len(layers))()
    for i, (q, k, v, out, ws) in enumerate(layers):
        qp, kp, vp = _qkv(p, q, k, v)
        wp, wn = _ws(ws)
        arr[i] = Layer(
            qp, kp, vp,
            _ptr(out["o_approx"], torch.float32, (B, Hq, D), "o_approx"),
            _ptr(out.get("lse_approx"), torch.float32, (B, Hq), "lse_approx",
                 True),
            _ptr(out["o_exact"], torch.float32, (B, Hq, D), "o_exact"),
            _ptr(out.get("lse_exact"), torch.float32, (B, Hq), "lse_exact",
                 True),
            _ptr(out["ratio"], torch.float32, (B,), "ratio"),
            _ptr(out["commit"], torch.uint8, (B,), "commit"),
            _ptr(out.get("o_committed"), torch.float32, (B, Hq, D),
                 "o_committed", True),
            wp, wn)
    return arr


def spec_decode_layers(h, p, layers, stream=None):
    """Layer-pipelined fused step over a chain of layers on one stream:
    `layers` is a list of (q, k, v, out, ws) tuples."""
    arr = layers_struct(p, layers)
    _check(_spec_decode_layers(h.ptr, ctypes.byref(p), len(layers), arr,
                               _stream(stream)),
           "alspec_spec_decode_layers")


def order_after_verify(h, stream=None):
    """Order `stream` (default: current) after the merge/verify work that
    pipelined calls on handle `h` have enqueued."""
    _check(_order_after_verify(h.ptr, _stream(stream)),
           "alspec_order_after_verify")


# ------------------------------------------------ post-attention operators ---

POST_MAX_BATCH = 8


class PostParams(ctypes.Structure):
    """Mirror of alspec_post_params."""
    _fields_ = [("batch", _i32), ("attn_dim", _i32), ("hidden", _i32),
                ("ffn", _i32), ("qkv_dim", _i32), ("eps", ctypes.c_float)]


class PostWeights(ctypes.Structure):
    """Mirror of alspec_post_weights (device pointers to bf16 weights)."""
    _fields_ = [("w_o", _P), ("norm_mlp", _P), ("w_gate", _P), ("w_up", _P),
                ("w_down", _P), ("norm_attn", _P), ("w_qkv", _P)]


POST_WEIGHT_NAMES = ("w_o", "norm_mlp", "w_gate", "w_up", "w_down",
                     "norm_attn", "w_qkv")

_post_workspace_size = _sig("alspec_post_workspace_size",
                            ctypes.POINTER(PostParams),
                            ctypes.POINTER(ctypes.c_size_t))
_post_attention = _sig("alspec_post_attention", _P,
                       ctypes.POINTER(PostParams),
                       ctypes.POINTER(PostWeights), _P, _P, _P, _P, _P, _P,
                       ctypes.c_size_t, _P)


def make_post_params(batch, attn_dim, hidden, ffn, qkv_dim, eps=1e-5):
    return PostParams(int(batch), int(attn_dim), int(hidden), int(ffn),
                      int(qkv_dim), float(eps))


def post_workspace_size(p):
    n = ctypes.c_size_t()
    _check(_post_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "alspec_post_workspace_size")
    return n.value


def alloc_post_workspace(p, device="cuda"):
    """Device workspace of alspec_post_attention (256-byte aligned)."""
    torch = _torch()
    n = post_workspace_size(p)
    ws = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def post_weights_struct(p, w):
    """alspec_post_weights from a dict of bf16 device tensors."""
    torch = _torch()
    shapes = {"w_o": (p.hidden, p.attn_dim), "norm_mlp": (p.hidden,),
              "w_gate": (p.ffn, p.hidden), "w_up": (p.ffn, p.hidden),
              "w_down": (p.hidden, p.ffn), "norm_attn": (p.hidden,),
              "w_qkv": (p.qkv_dim, p.hidden)}
    return PostWeights(*[_ptr(w[n], torch.bfloat16, shapes[n], n)
                         for n in POST_WEIGHT_NAMES])


def post_attention(h, p, w, o, h_in, h_out, qkv, ws, skip=None, stream=None):
    """Post-attention operators (alspec_post_attention); `w` is a dict of
    bf16 device tensors or a PostWeights struct."""
    torch = _torch()
    B = p.batch
    ws_struct = w if isinstance(w, PostWeights) else post_weights_struct(p, w)
    wp, wn = _ws(ws)
    _check(_post_attention(
        h.ptr, ctypes.byref(p), ctypes.byref(ws_struct),
        _ptr(o, torch.float32, (B, p.attn_dim), "o"),
        _ptr(h_in, torch.float32, (B, p.hidden), "h_in"),
        _ptr(h_out, torch.float32, (B, p.hidden), "h_out"),
        _ptr(qkv, torch.float32, (B, p.qkv_dim), "qkv"),
        _ptr(skip, torch.uint8, (B,), "skip", True), wp, wn, _stream(stream)),
        "alspec_post_attention")
