"""Draw a workload layer straight into device memory.

ctypes front end of libalspec_synth.so, the device twin of gen.kv_slice.
The host computes each head's planted rows and direction with gen.head_plant
(so both sides share them exactly) and the kernel draws the bulk normals.
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build
from . import gen

_lib = None


def _load():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (bind to the HIP runtime torch loaded)
        if not os.path.exists(_build.LIB):
            raise RuntimeError(
                f"{_build.LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_build.LIB)
        lib.synth_kv_fill.restype = ctypes.c_int
        lib.synth_kv_fill.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
            ctypes.c_uint32, ctypes.c_uint32, ctypes.c_double, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        _lib = lib
    return _lib


def fill_kv(w: gen.Workload, layer: int, k, v, stream=None):
    """Fill torch device tensors k, v ([B][Hkv][L_cap][D], float32 for an
    f32 workload, bfloat16 for bf16) with the layer's keys and values."""
    import torch
    lib = _load()
    bf16 = 1 if w.kv_dtype == "bf16" else 0
    want = torch.bfloat16 if bf16 else torch.float32
    for t in (k, v):
        if (t.dtype != want or not t.is_contiguous() or
                tuple(t.shape) != (w.B, w.Hkv, w.L_cap, w.D)):
            raise ValueError("k/v tensor does not match the workload")
    if stream is None:
        stream = torch.cuda.current_stream()
    key = gen.layer_key(w.seed, layer)
    sqrt_d = math.sqrt(w.D)
    for b in range(w.B):
        for g in range(w.Hkv):
            p = gen.head_plant(w, layer, b, g)
            u = np.ascontiguousarray(p.u, dtype=np.float64)
            for tid, dst in ((gen.TENSOR_K, k), (gen.TENSOR_V, v)):
                if tid == gen.TENSOR_K:
                    rows = np.ascontiguousarray(p.bias_rows, dtype=np.int32)
                    coef = np.ascontiguousarray(p.bias_coef, dtype=np.float64)
                else:
                    rows = np.zeros(0, np.int32)
                    coef = np.zeros(0, np.float64)
                rc = lib.synth_kv_fill(
                    dst[b, g].data_ptr(), bf16, w.L_cap, w.D, key[0], key[1],
                    g, tid, b, sqrt_d, int(rows.size), rows.ctypes.data,
                    coef.ctypes.data, u.ctypes.data, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"synth_kv_fill failed: {rc}")


def layer_to_device(w: gen.Workload, layer: int, device="cuda"):
    """(q, k, v) torch tensors on the device for one layer."""
    import torch
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    k = torch.empty((w.B, w.Hkv, w.L_cap, w.D), dtype=dt, device=device)
    v = torch.empty_like(k)
    fill_kv(w, layer, k, v)
    q = torch.from_numpy(gen.q_all(w, layer)).to(device)
    return q, k, v


def _probe_lib():
    lib = _load()
    if not hasattr(lib, "_probe_sig"):
        lib.probe_read.restype = ctypes.c_int
        lib.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
        lib.probe_copy.restype = ctypes.c_int
        lib.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p]
        lib._probe_sig = True
    return lib


PROBE_READ_BLOCKS = (1024, 2048, 4096, 8192)
PROBE_READ_UNROLL = (1, 2, 4, 8)


def probe_bandwidth(nbytes=4 << 30, reps=10, blocks=256 * 16):
    """Achievable read and copy bandwidth (GB/s, 1e9 bytes) over `nbytes`
    buffers, timed with HIP events; each kernel averaged over `reps`.  The
    read is swept over grid sizes, loads in flight per thread and plain or
    nontemporal loads; "read" is the fastest of the sweep (its settings
    beside it), "read_simple" one nontemporal load per thread on `blocks`
    blocks; the copy runs on `blocks` blocks."""
    import torch
    lib = _probe_lib()
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(max(PROBE_READ_BLOCKS + (blocks,)), dtype=torch.int32,
                       device="cuda")
    s = torch.cuda.current_stream()

    def timed(launch, moved):
        launch()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            launch()
        e1.record(s)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        return {"bytes_per_launch": moved, "ms": ms,
                "GBps": moved / (ms * 1e-3) / 1e9}

    def read(nb, unroll, nt):
        def launch():
            rc = lib.probe_read(src.data_ptr(), nbytes, sink.data_ptr(), nb,
                                unroll, nt, s.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"probe_read failed: {rc}")
        r = timed(launch, nbytes)
        r.update(blocks=nb, loads_in_flight=unroll, nontemporal=bool(nt))
        return r

    def copy():
        rc = lib.probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks,
                            s.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe_copy failed: {rc}")
    sweep = [read(nb, u, nt) for nb in PROBE_READ_BLOCKS
             for u in PROBE_READ_UNROLL for nt in (0, 1)]
    res = {"read": max(sweep, key=lambda r: r["GBps"]),
           "read_simple": read(blocks, 1, 1),
           "copy": timed(copy, 2 * nbytes)}
    del src, dst, sink
    return res


def probe_read_sizes(sizes, blocks=(256, 512, 1024, 2048), reps=None,
                     pool_bytes=2 << 30):
    """Achievable read bandwidth (GB/s) for single launches of given sizes:
    for each size in `sizes` (bytes, multiples of 16), the fastest read-probe
    setting over `blocks` x loads in flight x plain/nontemporal, each
    setting timed with HIP events over back-to-back launches that walk
    distinct slices of a `pool_bytes` buffer (well above the 256 MB of
    last-level cache, so no launch re-reads cached bytes).  A short launch
    pays its ramp and tail as a kernel of the same size does, so the result
    is the ceiling such a kernel can be held to."""
    import torch
    lib = _probe_lib()
    src = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sink = torch.zeros(max(blocks), dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    base = src.data_ptr()
    out = {}
    for nb_ in sizes:
        if nb_ % 16 or nb_ > pool_bytes:
            raise ValueError(f"probe size {nb_} not usable")
        slices = pool_bytes // nb_
        n = reps or max(32, slices)

        def launch(i, nb, u, nt):
            rc = lib.probe_read(base + (i % slices) * nb_, nb_,
                                sink.data_ptr(), nb, u, nt, s.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"probe_read failed: {rc}")
        best = None
        for nb in blocks:
            for u in PROBE_READ_UNROLL:
                for nt in (0, 1):
                    for i in range(4):
                        launch(i, nb, u, nt)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(s)
                    for i in range(n):
                        launch(i, nb, u, nt)
                    e1.record(s)
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) * 1e3 / n
                    r = {"bytes": nb_, "us": us,
                         "GBps": nb_ / (us * 1e-6) / 1e9, "blocks": nb,
                         "loads_in_flight": u, "nontemporal": bool(nt)}
                    if best is None or r["GBps"] > best["GBps"]:
                        best = r
        out[nb_] = best
    del src, sink
    return out
