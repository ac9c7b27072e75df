"""Host-side checks of the C ABI (no GPU needed): every function that
include/alspec.h declares is exported by libalspec.so, parameters are
validated before any GPU work, and the split plan tiles every context
exactly into sink, window and middle ranges."""
import ctypes
import os
import re

import numpy as np
import pytest

import attention_level_speculation_amd as al
from attention_level_speculation_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "alspec.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(alspec_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("alspec_sink_approx", "alspec_flash_decode_exact",
              "alspec_lse_combine", "alspec_verify", "alspec_spec_decode",
              "alspec_workspace_size", "alspec_create", "alspec_destroy"):
        assert n in names


PAGE_CITATION = re.compile(
    r"Attention-Level Speculation|atlas\.scime\.ai|ICML 2025 poster")


def declarations_with_comments():
    """(name, first parameter, comment block just above) for every function
    the header declares."""
    text = open(HEADER).read()
    out = []
    for m in re.finditer(r"(/\*(?:(?!\*/).)*\*/)\s*(?:const\s+)?\w+\s*\*?\s*"
                         r"(alspec_[a-z_]+)\s*\(([^,)]*)", text, flags=re.S):
        out.append((m.group(2), m.group(3).strip(), m.group(1)))
    return out


def test_every_compute_call_cites_its_passage():
    """Each compute entry point (it takes a handle and enqueues GPU work)
    names the passage of the pages that defines its operation."""
    decls = declarations_with_comments()
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    takes_handle = set(re.findall(r"\b(alspec_[a-z_]+)\s*\(\s*alspec_handle",
                                  text))
    assert takes_handle <= {n for n, _, _ in decls} | {"alspec_destroy"}
    compute = [(n, c) for n, first, c in decls
               if first.startswith("alspec_handle")
               and n not in ("alspec_create", "alspec_destroy",
                             "alspec_order_after_verify")]
    assert len(compute) >= 7, [n for n, _ in compute]
    for n, comment in compute:
        if n.endswith("_noalloc"):
            # the allocation-free variant names the callers it serves
            assert "allocate" in comment, n
        else:
            assert PAGE_CITATION.search(comment), f"{n} cites no passage"


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(al.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings_and_version():
    for code, name in _binding.STATUS.items():
        assert al.status_string(code) == name
    assert al.status_string(99) == "ALSPEC_UNKNOWN_STATUS"
    assert al.version() == 100


def P(**kw):
    args = dict(batch=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                kv_capacity=1000, seq_lens=[1000], kv_dtype="bf16", sink=4,
                window=64, lam=0.1)
    args.update(kw)
    if "seq_lens" not in kw:
        args["seq_lens"] = [args["kv_capacity"]] * args["batch"]
    return al.make_params(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(num_q_heads=6, num_kv_heads=4), 1),
    (dict(seq_lens=[0]), 1), (dict(seq_lens=[1001]), 1),
    (dict(sink=0, window=0), 1), (dict(sink=-1), 1), (dict(window=-5), 1),
    (dict(lam=-0.5), 1), (dict(lam=float("nan")), 1),
    (dict(sm_scale=0.0), 1), (dict(sm_scale=float("inf")), 1),
    (dict(kv_dtype=7), 1), (dict(split_tokens=-1), 1), (dict(overlap=3), 1),
    (dict(head_dim=96), 2), (dict(num_q_heads=48, num_kv_heads=2), 2),
    (dict(batch=65, kv_capacity=10), 2), (dict(num_kv_heads=128,
                                              num_q_heads=128), 2),
])
def test_workspace_size_validates(kw, status):
    with pytest.raises(al.AlspecError) as e:
        al.workspace_size(P(**kw))
    assert e.value.status == status


def test_lambda_inf_is_accepted():
    assert al.workspace_size(P(lam=float("inf"))) > 0


def test_null_handle_and_pointers_rejected_before_gpu_work():
    p = P()
    f = _binding._spec_decode
    st = f(None, ctypes.byref(p), *([None] * 11), 0, None, None, None)
    assert st == 1
    assert _binding._sink_approx(None, ctypes.byref(p), None, None, None,
                                 None, None, None, 0, None) == 1
    assert _binding._verify(None, ctypes.byref(p), None, None, None, None,
                            None, None) == 1
    assert _binding._lse_combine(None, ctypes.byref(p), None, 0, None, None,
                                 None) == 1
    assert _binding._flash_exact(None, ctypes.byref(p), None, None, None, 0,
                                 None, 0, None) == 1
    n = ctypes.c_size_t()
    assert _binding._workspace_size(None, ctypes.byref(n)) == 1


def _check_tiling(p, b, L, S, W):
    splits, (T, Tw) = al.plan_splits(p, b)
    s_end = min(S, L)
    w_begin = max(s_end, L - W)
    kinds = [k for k, _, _ in splits]
    assert kinds == sorted(kinds), "slot order must be sink, window, middle"
    # every token of [0, L) exactly once
    cover = np.zeros(L, np.int32)
    for kd, t0, t1 in splits:
        assert 0 <= t0 < t1 <= L
        cover[t0:t1] += 1
        if kd == 0:
            assert (t0, t1) == (0, s_end)
        elif kd == 1:
            assert w_begin <= t0 and t1 <= L and t1 - t0 <= Tw
        else:
            assert s_end <= t0 and t1 <= w_begin and t1 - t0 <= T
    assert (cover == 1).all()
    assert sum(1 for k in kinds if k == 0) == (1 if s_end > 0 else 0)
    win = sorted((t0, t1) for kd, t0, t1 in splits if kd == 1)
    mid = sorted((t0, t1) for kd, t0, t1 in splits if kd == 2)
    if win:
        assert win[0][0] == w_begin and win[-1][1] == L
    if mid:
        assert mid[0][0] == s_end and mid[-1][1] == w_begin


@pytest.mark.parametrize("seed", range(25))
def test_split_plan_tiles_context(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    L_cap = int(rng.choice([1, 7, 64, 1000, 4097, 131072]))
    lens = [int(x) for x in rng.integers(1, L_cap + 1, size=B)]
    S = int(rng.integers(0, 9))
    W = int(rng.choice([0, 1, 63, 128, 2048, 5000]))
    if S + W == 0:
        W = 1
    split = int(rng.choice([0, 0, 64, 300, 1024]))
    wsplit = int(rng.choice([0, 0, 32, 100]))
    p = al.make_params(B, 8, 4, 64, L_cap, lens, "f32", S, W, 0.1,
                       split_tokens=split, window_split_tokens=wsplit)
    for b in range(B):
        _check_tiling(p, b, lens[b], S, W)
    assert al.workspace_size(p) > 0


def test_headline_plan_shape():
    """Context 131072, S 4, W 2048, 8 kv heads: one sink split, window cut
    into 16 pieces of 128, middle pieces of 4032 tokens: 32 per kv head,
    one per CU."""
    p = al.make_params(1, 32, 8, 128, 131072, [131072], "bf16", 4, 2048, 0.1)
    splits, (T, Tw) = al.plan_splits(p, 0)
    assert Tw == 128 and T == 4032
    assert sum(1 for s in splits if s[0] == 1) == 16
    assert sum(1 for s in splits if s[0] == 2) == 32
    _check_tiling(p, 0, 131072, 4, 2048)


def test_window_splits_tile_the_window():
    """The headline plan (16 window splits of 128 tokens per kv head) cuts
    the window into adjacent pieces; an explicit window split is taken as
    given."""
    p = al.make_params(1, 32, 8, 128, 131072, [131072], "bf16", 4, 2048, 0.1)
    s1, (T1, Tw1) = al.plan_splits(p, 0)
    assert (T1, Tw1) == (4032, 128)
    w1 = sorted((b, e) for k, b, e in s1 if k == 1)
    assert len(w1) == 16
    assert w1[0][0] == 131072 - 2048 and w1[-1][1] == 131072
    assert all(w1[i][1] == w1[i + 1][0] for i in range(len(w1) - 1))
    q = al.make_params(1, 32, 8, 128, 131072, [131072], "bf16", 4, 2048, 0.1,
                       window_split_tokens=96)
    assert al.plan_splits(q, 0)[1][1] == 96


@pytest.mark.parametrize("B,Hkv,W,tw", [
    (1, 8, 2048, 128),     # Llama-3-8B at 128K: 16 per kv head
    (4, 8, 4096, 1024),    # Llama-3-70B stack, 4 users: 4 each (cap)
    (1, 8, 1024, 64),      # Llama-3-8B at 32K
    (8, 8, 2048, 1024),    # 8 users: 2 per (user, kv head) (cap)
    (2, 8, 2048, 256),     # 2 users: 8 per (user, kv head)
    (64, 8, 2048, 1024),   # more pairs than splits: at most 1024
    (1, 8, 128, 64),       # short window: at least 64 tokens
])
def test_automatic_window_split_targets_a_split_count(B, Hkv, W, tw):
    """The automatic window split is the power of two (64 to 1024) at or
    below the longest window over (128 / pairs), pairs being the (entry, kv
    head) pairs with a window."""
    p = al.make_params(B, Hkv * 4, Hkv, 128, 131072, [131072] * B, "bf16",
                       4, W, 0.1)
    assert al.plan_splits(p, 0)[1][1] == tw
    n = sum(1 for s in al.plan_splits(p, 0)[0] if s[0] == 1) * B * Hkv
    assert n <= max(128, B * Hkv * -(-W // 1024))


@pytest.mark.parametrize("seed", range(30))
def test_middle_split_length_fills_the_cus_once(seed):
    """The default middle split length is the shortest whole number of
    64-token steps, at least 256, whose splits over all entries and kv heads
    number at most one per CU (256), or per round of 256 when the (entry,
    kv head) pairs with a middle outnumber the CUs."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 65))
    Hkv = int(rng.choice([1, 2, 4, 8, 16]))
    L_cap = int(rng.choice([3000, 20000, 131072]))
    lens = [int(x) for x in rng.integers(1, L_cap + 1, size=B)]
    S, W = 4, int(rng.choice([64, 2048]))
    p = al.make_params(B, Hkv * 4, Hkv, 128, L_cap, lens, "bf16", S, W, 0.1)
    T = al.plan_splits(p, 0)[1][0]
    mids = [max(0, max(min(S, L), L - W) - min(S, L)) for L in lens]

    def items(t):
        return Hkv * sum(-(-m // t) for m in mids if m > 0)
    pairs = Hkv * sum(1 for m in mids if m > 0)
    target = 256 * -(-pairs // 256)
    assert T % 64 == 0 and T >= 256
    if pairs:
        assert items(T) <= target
        if T > 256:
            assert items(T - 64) > target
    got = sum(1 for b in range(B) for s in al.plan_splits(p, b)[0]
              if s[0] == 2)
    assert got * Hkv == items(T)


def test_workspace_grows_with_splits():
    a = al.workspace_size(P(split_tokens=1024))
    b = al.workspace_size(P(split_tokens=64))
    assert b > a


def test_last_error_is_a_string():
    assert isinstance(al.last_error(), str)


def test_layers_chain_validation_before_gpu_work():
    """alspec_spec_decode_layers rejects bad arguments and workspaces shared
    by layers fewer than 3 apart before any HIP call (no GPU needed)."""
    p = P()
    f = _binding._spec_decode_layers
    fake_h = ctypes.c_void_p(0x1000)
    assert f(None, ctypes.byref(p), 1, None, None) == 1
    arr = (_binding.Layer * 4)()
    assert f(fake_h, ctypes.byref(p), 0, arr, None) == 1
    size = al.workspace_size(p)
    base = 1 << 40                        # aligned stand-in addresses
    for i in range(4):
        arr[i] = _binding.Layer(base, base, base, base, None, base, None,
                                base, base, None, base + (i << 30), size)
    arr[2].ws = arr[1].ws                 # layers 1 and 2 share
    assert f(fake_h, ctypes.byref(p), 4, arr, None) == 3
    arr[2].ws = base + (2 << 30)
    arr[3].ws = arr[1].ws                 # layers 1 and 3 share
    assert f(fake_h, ctypes.byref(p), 4, arr, None) == 3
    arr[3].ws = base + (3 << 30)
    arr[1].ws_bytes = size - 1            # too small
    assert f(fake_h, ctypes.byref(p), 4, arr, None) == 3
    arr[1].ws_bytes = size
    arr[2].q = base + 4                   # misaligned input
    assert f(fake_h, ctypes.byref(p), 4, arr, None) == 1


def test_verify_rejects_misaligned_outputs_before_gpu_work():
    """alspec_verify reads and writes its [B][Hq][D] arrays 16 bytes at a
    time: a misaligned o_approx, o_exact or o_committed is rejected before
    any HIP call (no GPU needed)."""
    p = P()
    f = _binding._verify
    fake_h = ctypes.c_void_p(0x1000)
    a = 1 << 40                           # aligned stand-in addresses
    assert f(fake_h, ctypes.byref(p), a + 4, a, a, a, a, None) == 1
    assert f(fake_h, ctypes.byref(p), a, a + 8, a, a, a, None) == 1
    assert f(fake_h, ctypes.byref(p), a, a, a, a, a + 12, None) == 1
    assert f(None, ctypes.byref(p), a, a, a, a, a, None) == 1
    assert f(fake_h, ctypes.byref(p), None, a, a, a, a, None) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(batch=9), 2), (dict(attn_dim=12), 1),
    (dict(hidden=4), 1), (dict(ffn=1001), 1), (dict(qkv_dim=0), 1),
    (dict(eps=0.0), 1), (dict(eps=float("nan")), 1),
    (dict(eps=float("inf")), 1)])
def test_post_workspace_size_validates(kw, status):
    args = dict(batch=1, attn_dim=64, hidden=64, ffn=128, qkv_dim=32,
                eps=1e-5)
    args.update(kw)
    with pytest.raises(al.AlspecError) as e:
        al.post_workspace_size(al.make_post_params(**args))
    assert e.value.status == status


def test_post_attention_rejects_before_gpu_work():
    """Null or misaligned pointers, aliasing outputs, skip flags with an
    in-place residual and a short workspace are refused before any HIP
    call (no GPU needed)."""
    p = al.make_post_params(2, 64, 64, 128, 32)
    need = al.post_workspace_size(p)
    assert need == 2 * 128 * 4 + (-(2 * 128 * 4)) % 256
    f = _binding._post_attention
    fake_h = ctypes.c_void_p(0x1000)
    base = 1 << 40
    w = _binding.PostWeights(*[base + (i << 24) for i in range(7)])
    o, hi, ho, q, sk, ws = (base + (i << 28) for i in range(8, 14))
    ok = (o, hi, ho, q, sk, ws, need, None)
    assert f(None, ctypes.byref(p), ctypes.byref(w), *ok) == 1
    assert f(fake_h, ctypes.byref(p), None, *ok) == 1
    assert f(fake_h, ctypes.byref(p), ctypes.byref(w),
             o + 4, hi, ho, q, sk, ws, need, None) == 1       # misaligned
    assert f(fake_h, ctypes.byref(p), ctypes.byref(w),
             o, hi, hi, q, sk, ws, need, None) == 1           # skip + in place
    assert f(fake_h, ctypes.byref(p), ctypes.byref(w),
             o, hi, q, q, None, ws, need, None) == 1          # h_out is qkv
    assert f(fake_h, ctypes.byref(p), ctypes.byref(w),
             o, hi, ho, q, sk, ws, need - 1, None) == 3       # short ws
    assert f(fake_h, ctypes.byref(p), ctypes.byref(w),
             o, hi, ho, q, sk, ws + 16, need, None) == 3      # misaligned ws
    w.w_up = None
    assert f(fake_h, ctypes.byref(p), ctypes.byref(w), *ok) == 1


def test_other_library_refused_under_pytest():
    """ALSPEC_LIB (a variant build for timing comparisons) is refused when
    pytest is loaded: the tests check the in-tree library."""
    import subprocess
    import sys
    env = dict(os.environ, ALSPEC_LIB="/nonexistent/libalspec.so")
    r = subprocess.run(
        [sys.executable, "-c",
         "import sys; sys.path.insert(0, %r); import pytest; "
         "import attention_level_speculation_amd" % ROOT],
        env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "not honoured under pytest" in r.stderr
