"""CPU oracle for the speculative flash-decode step of attention-level
speculation (ALSpec).

TEST INFRASTRUCTURE ONLY: this package is the plain double-precision
definition that the GPU library is checked against.  Only the tests, the
smoke check and the benchmark's CPU-baseline leg use it; the GPU library
never imports or calls it, and it shares no code with the GPU library.

The arithmetic lives in ``alspec_oracle.c`` (plain C, double); this module
only marshals numpy arrays through ctypes.  See that file's header for the
passages followed and the readings taken where the pages are silent.

Parity status of each function (what pins it, in ``tests/test_oracle_pins.py``):
  spec_decode  pinned: hand-worked closed forms, S+W>=L identity, shift
               invariance, uniform/one-hot limits, GQA==repeated MHA, affine
               in V, middle-permutation invariance, closed form of the error,
               window/sink boundary cases, high-precision brute force.
  partial, lse_merge  pinned: split-and-merge equals the one-pass softmax for
               random partitions including empty parts; brute force.
  verify       pinned: constructed outputs with known relative error,
               monotonicity in lambda, zero/NaN special cases.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_F = ctypes.POINTER(ctypes.c_float)
_I = ctypes.POINTER(ctypes.c_int32)
_U8 = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ALSPEC_ORACLE_LIB")  # planted-mistake tests only
    if not path:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_spec_decode.restype = ctypes.c_int
    lib.oracle_spec_decode.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _I, ctypes.c_int, _F, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
        ctypes.c_int, _D, _D, _D, _D, _D, _D, _U8, _D]
    lib.oracle_partial.restype = ctypes.c_int
    lib.oracle_partial.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, _F, ctypes.c_void_p,
        ctypes.c_void_p, _I, ctypes.c_int, ctypes.c_double, _D, _D, _D]
    lib.oracle_lse_merge.restype = ctypes.c_int
    lib.oracle_lse_merge.argtypes = [ctypes.c_int, ctypes.c_int, _D, _D, _D,
                                     _D, _D]
    lib.oracle_verify.restype = ctypes.c_int
    lib.oracle_verify.argtypes = [ctypes.c_int, ctypes.c_int, _D, _D,
                                  ctypes.c_double, _D, _U8]
    _lib = lib
    return lib


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _kv_array(x):
    """Return (contiguous array, is_bf16).  bf16 data is given as uint16 bit
    patterns (numpy has no bf16 type)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, 0
    if x.dtype in (np.uint16, np.int16):
        return x.view(np.uint16), 1
    raise TypeError(f"k/v must be float32 or uint16 (bf16 bits), got {x.dtype}")


def default_threads():
    return max(1, len(os.sched_getaffinity(0)))


def spec_decode(q, k, v, seq_lens, sink, window, lam, sm_scale=None,
                threads=None):
    """Exact and sink+window attention, relative-L2 verify and commit.

    q: float32 [B][Hq][D]; k, v: float32 or uint16 bf16 bits [B][Hkv][L_cap][D];
    seq_lens: int [B].  Returns a dict of float64 arrays (and uint8 commit).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k, kb = _kv_array(k)
    v, vb = _kv_array(v)
    if kb != vb or k.shape != v.shape:
        raise ValueError("k and v must share dtype and shape")
    B, Hq, D = q.shape
    Bk, Hkv, L_cap, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("shape mismatch between q and k/v")
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32).reshape(B)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    if threads is None:
        threads = default_threads()
    out = {
        "o_exact": np.empty((B, Hq, D)), "lse_exact": np.empty((B, Hq)),
        "o_approx": np.empty((B, Hq, D)), "lse_approx": np.empty((B, Hq)),
        "mass_A": np.empty((B, Hq)), "ratio": np.empty(B),
        "commit": np.empty(B, dtype=np.uint8),
        "o_committed": np.empty((B, Hq, D)),
    }
    rc = lib.oracle_spec_decode(
        B, Hq, Hkv, D, L_cap, _ptr(lens, _I), kb, _ptr(q, _F),
        k.ctypes.data, v.ctypes.data, int(sink), int(window), float(sm_scale),
        float(lam), int(threads), _ptr(out["o_exact"], _D),
        _ptr(out["lse_exact"], _D), _ptr(out["o_approx"], _D),
        _ptr(out["lse_approx"], _D), _ptr(out["mass_A"], _D),
        _ptr(out["ratio"], _D), _ptr(out["commit"], _U8),
        _ptr(out["o_committed"], _D))
    if rc != 0:
        raise ValueError(f"oracle_spec_decode rejected its arguments (rc={rc})")
    return out


def partial(q_head, k_head, v_head, tokens, sm_scale):
    """State (m, l, acc) of one query head over listed token positions."""
    lib = _load()
    q_head = np.ascontiguousarray(q_head, dtype=np.float32)
    k_head, kb = _kv_array(k_head)
    v_head, vb = _kv_array(v_head)
    L_cap, D = k_head.shape
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
    m = np.empty(1)
    l = np.empty(1)
    acc = np.empty(D)
    rc = lib.oracle_partial(D, L_cap, kb, _ptr(q_head, _F), k_head.ctypes.data,
                            v_head.ctypes.data, _ptr(tok, _I), tok.size,
                            float(sm_scale), _ptr(m, _D), _ptr(l, _D),
                            _ptr(acc, _D))
    if rc != 0:
        raise ValueError(f"oracle_partial rejected its arguments (rc={rc})")
    return float(m[0]), float(l[0]), acc


def lse_merge(m, l, acc):
    """Log-sum-exp merge of partial states -> (output [D], lse)."""
    lib = _load()
    m = np.ascontiguousarray(m, dtype=np.float64).reshape(-1)
    l = np.ascontiguousarray(l, dtype=np.float64).reshape(-1)
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    n, D = acc.shape
    out = np.empty(D)
    lse = np.empty(1)
    rc = lib.oracle_lse_merge(n, D, _ptr(m, _D), _ptr(l, _D), _ptr(acc, _D),
                              _ptr(out, _D), _ptr(lse, _D))
    if rc != 0:
        raise ValueError(f"oracle_lse_merge rejected its arguments (rc={rc})")
    return out, float(lse[0])


def verify(o_approx, o_exact, lam):
    """Per-batch-entry relative L2 error and commit flag."""
    lib = _load()
    a = np.ascontiguousarray(o_approx, dtype=np.float64)
    e = np.ascontiguousarray(o_exact, dtype=np.float64)
    if a.shape != e.shape:
        raise ValueError("shape mismatch")
    B = a.shape[0]
    n = int(np.prod(a.shape[1:]))
    ratio = np.empty(B)
    commit = np.empty(B, dtype=np.uint8)
    rc = lib.oracle_verify(B, n, _ptr(a, _D), _ptr(e, _D), float(lam),
                           _ptr(ratio, _D), _ptr(commit, _U8))
    if rc != 0:
        raise ValueError(f"oracle_verify rejected its arguments (rc={rc})")
    return ratio, commit
