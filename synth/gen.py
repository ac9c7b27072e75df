"""Seeded synthetic decode-attention inputs with a planted sink and needles.

This module only draws inputs.  It holds none of the attention method's
arithmetic and is shared by the CPU oracle's tests and the GPU library's
tests and benchmark.  The numpy functions here are the definition; the HIP
kernel in ``synth_kernels.hip`` reproduces ``kv_slice`` on the device for the
large workloads (same counters, same double-precision formula, same
rounding), and a GPU test checks the two agree.

Structure (the pages evaluate on task suites and a synthetic
needle-in-a-haystack set that are not reproduced here; these inputs stand in
for their long-context attention structure):
  * base elements of q, k, v are N(0,1)/sqrt(D);
  * each (layer, user, kv head) has a random unit direction u; every query
    head of the group gets q += a*u;
  * planted sink: the first S keys get k += b_s*u, sized so that their
    logit rises by Delta_s = ln(H/S) + c_s + tau_s*xi (xi ~ N(0,1) per kv
    head, H = number of plain middle tokens);
  * planted needles: n keys at distinct uniform positions of the middle get
    k += b_n*u with logit boost Delta_n = ln(H) + c_n + tau_n*xi_i.
A logit boost Delta needs b = Delta*sqrt(D)/a, because the attention logit is
<q, k>/sqrt(D) and <a*u, b*u> = a*b.

Random numbers: Philox4x32-10, key from SplitMix64 of (seed, layer), counter
(group index, head, tensor id, user); each counter gives four uint32, turned
into four normals by the Box-Muller transform in double precision.  Values
are formed in double and rounded once to float32 (round to nearest even),
then, for bf16 storage, to bf16 (round to nearest even on the float32 bits).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence

import numpy as np

from .philox import philox4x32_10, splitmix64

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_AUX = 0, 1, 2, 3
TWO_PI = 6.283185307179586
TWO_M32 = 2.3283064365386963e-10  # 2**-32

# aux-stream counter ranges (x0) per (layer, user, kv head)
AUX_DIR = 0            # D normals for the direction u
AUX_SINK_XI = 1 << 20  # one normal for the sink boost jitter
AUX_NEEDLE_POS = 2 << 20
AUX_NEEDLE_XI = 3 << 20
AUX_USER = 4 << 20     # per-user draws of a workload (ragged lengths, needles)


@dataclass(frozen=True)
class Constants:
    a: float = 8.0       # query alignment with u
    c_s: float = 3.5     # sink boost offset (nats)
    tau_s: float = 1.0   # sink boost jitter (nats)
    c_n: float = -3.0    # needle boost offset (nats)
    tau_n: float = 1.0   # needle boost jitter (nats)


@dataclass
class Workload:
    """One decode step's attention inputs: B users, one layer at a time."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    L_cap: int
    seq_lens: List[int]
    kv_dtype: str            # "f32" or "bf16"
    S: int
    W: int
    lam: float
    needles: List[int]       # planted needles per kv head, per user
    n_layers: int = 1
    seed: int = 1
    const: Constants = field(default_factory=Constants)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def kv_bytes_per_token(self):
        return self.Hkv * self.D * 2 * (4 if self.kv_dtype == "f32" else 2)

    def kv_bytes(self):
        """Bytes of K and V that one decode step reads for all users."""
        return sum(self.seq_lens) * self.kv_bytes_per_token


# --------------------------------------------------------------- drawing ---

def layer_key(seed: int, layer: int):
    z = splitmix64((int(seed) * 0x9E3779B97F4A7C15 + int(layer) + 1)
                   & 0xFFFFFFFFFFFFFFFF)
    return z & 0xFFFFFFFF, z >> 32


def box_muller(r0, r1):
    """Two uint32 arrays -> two normal arrays (double)."""
    u1 = (r0.astype(np.float64) + 0.5) * TWO_M32
    u2 = (r1.astype(np.float64) + 0.5) * TWO_M32
    rad = np.sqrt(-2.0 * np.log(u1))
    th = TWO_PI * u2
    return rad * np.cos(th), rad * np.sin(th)


def normals(key, x1, x2, x3, first_group, n_groups):
    """4*n_groups normals from counters (first_group.., x1, x2, x3)."""
    c0 = np.arange(first_group, first_group + n_groups, dtype=np.uint64)
    r0, r1, r2, r3 = philox4x32_10(c0, x1, x2, x3, key[0], key[1])
    z0, z1 = box_muller(r0, r1)
    z2, z3 = box_muller(r2, r3)
    return np.stack([z0, z1, z2, z3], axis=-1).reshape(-1)


def uniform_u32(key, x1, x2, x3, first_group, n_groups):
    c0 = np.arange(first_group, first_group + n_groups, dtype=np.uint64)
    return philox4x32_10(c0, x1, x2, x3, key[0], key[1])[0]


def sets(L, S, W):
    """(sink end, window begin): sink [0, s_end), window [w_begin, L)."""
    s_end = min(S, L)
    return s_end, max(s_end, L - W)


@dataclass
class HeadPlant:
    u: np.ndarray            # [D] unit direction (double)
    bias_rows: np.ndarray    # int rows that get k += coef*u
    bias_coef: np.ndarray    # double coefficients for those rows
    needle_pos: np.ndarray
    delta_s: float


def head_plant(w: Workload, layer: int, b: int, g: int) -> HeadPlant:
    key = layer_key(w.seed, layer)
    D = w.D
    z = normals(key, g, TENSOR_AUX, b, AUX_DIR, (D + 3) // 4)[:D]
    u = z / math.sqrt(float(np.dot(z, z)))
    L = w.seq_lens[b]
    s_end, w_begin = sets(L, w.S, w.W)
    M = w_begin - s_end
    n = min(int(w.needles[b]), max(M, 0))
    pos: List[int] = []
    t = 0
    while len(pos) < n:
        r = int(uniform_u32(key, g, TENSOR_AUX, b, AUX_NEEDLE_POS + t, 1)[0])
        t += 1
        p = s_end + ((r * M) >> 32)
        if p not in pos:
            pos.append(p)
    H = max(1, M - n)
    sqrt_d = math.sqrt(D)
    c = w.const
    rows, coef = [], []
    delta_s = 0.0
    if s_end > 0:
        xi = normals(key, g, TENSOR_AUX, b, AUX_SINK_XI, 1)[0]
        delta_s = math.log(H / s_end) + c.c_s + c.tau_s * xi
        bs = delta_s * sqrt_d / c.a
        rows += list(range(s_end))
        coef += [bs] * s_end
    for i, p in enumerate(pos):
        xi = normals(key, g, TENSOR_AUX, b, AUX_NEEDLE_XI + i, 1)[0]
        dn = math.log(H) + c.c_n + c.tau_n * xi
        rows.append(p)
        coef.append(dn * sqrt_d / c.a)
    return HeadPlant(u=u, bias_rows=np.array(rows, dtype=np.int32),
                     bias_coef=np.array(coef, dtype=np.float64),
                     needle_pos=np.array(pos, dtype=np.int32),
                     delta_s=delta_s)


def to_f32(x64):
    return x64.astype(np.float32)


def f32_to_bf16_bits(f32):
    bits = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    r = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b16):
    return (np.asarray(b16, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def kv_slice(w: Workload, layer: int, b: int, g: int, tensor: int,
             plant: Optional[HeadPlant] = None, rows=None):
    """K or V of one (layer, user, kv head): [L_cap][D] float32 or uint16
    bf16 bits.  `rows` (a range) limits generation to those rows."""
    key = layer_key(w.seed, layer)
    D = w.D
    r0, r1 = (0, w.L_cap) if rows is None else (rows.start, rows.stop)
    assert (D % 4) == 0
    g0 = r0 * D // 4
    ng = (r1 - r0) * D // 4
    z = normals(key, g, tensor, b, g0, ng).reshape(r1 - r0, D)
    sqrt_d = math.sqrt(D)
    x = z / sqrt_d
    if tensor == TENSOR_K:
        if plant is None:
            plant = head_plant(w, layer, b, g)
        for row, cf in zip(plant.bias_rows, plant.bias_coef):
            if r0 <= row < r1:
                x[row - r0] = z[row - r0] / sqrt_d + cf * plant.u
    f = to_f32(x)
    return f if w.kv_dtype == "f32" else f32_to_bf16_bits(f)


def q_all(w: Workload, layer: int):
    """Q of one layer: float32 [B][Hq][D]."""
    key = layer_key(w.seed, layer)
    D = w.D
    q = np.empty((w.B, w.Hq, D), np.float32)
    sqrt_d = math.sqrt(D)
    for b in range(w.B):
        for g in range(w.Hkv):
            u = head_plant(w, layer, b, g).u
            for h in range(g * w.G, (g + 1) * w.G):
                z = normals(key, h, TENSOR_Q, b, 0, D // 4)
                q[b, h] = to_f32(z / sqrt_d + w.const.a * u)
    return q


def layer_inputs(w: Workload, layer: int, threads: Optional[int] = None):
    """Whole layer on the host: (q, k, v) with k, v [B][Hkv][L_cap][D].
    Slices are drawn on a thread pool (numpy releases the GIL); the values
    do not depend on the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    kt = np.float32 if w.kv_dtype == "f32" else np.uint16
    k = np.empty((w.B, w.Hkv, w.L_cap, w.D), kt)
    v = np.empty((w.B, w.Hkv, w.L_cap, w.D), kt)
    chunk = max(1, (1 << 22) // w.D)

    def job(b, g, t, r0):
        p = head_plant(w, layer, b, g)
        r1 = min(w.L_cap, r0 + chunk)
        dst = k if t == TENSOR_K else v
        dst[b, g, r0:r1] = kv_slice(w, layer, b, g, t, p, range(r0, r1))

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    jobs = [(b, g, t, r0) for b in range(w.B) for g in range(w.Hkv)
            for t in (TENSOR_K, TENSOR_V) for r0 in range(0, w.L_cap, chunk)]
    if threads <= 1:
        for j in jobs:
            job(*j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            for f in [ex.submit(job, *j) for j in jobs]:
                f.result()
    return q_all(w, layer), k, v


# ------------------------------------------------------------ workloads ----

def tiny_f32_1k(seed=1):
    """Tiny decode attention, fp32: 1 user, 8 q heads = 8 kv heads, D 64,
    context 1024, 2 needles per head, S 4, W 128, lambda 0.10, one layer."""
    return Workload("tiny_f32_1k", B=1, Hq=8, Hkv=8, D=64, L_cap=1024,
                    seq_lens=[1024], kv_dtype="f32", S=4, W=128, lam=0.10,
                    needles=[2], n_layers=1, seed=seed)


def llama8b_32k(seed=2):
    """Llama-3-8B-shaped decode layer: 32 q / 8 kv heads, D 128, bf16 KV,
    context 32768, 1 needle per 8K tokens, S 4, W 1024, 32 layers."""
    return Workload("llama8b_32k", B=1, Hq=32, Hkv=8, D=128, L_cap=32768,
                    seq_lens=[32768], kv_dtype="bf16", S=4, W=1024, lam=0.10,
                    needles=[4], n_layers=32, seed=seed)


HEADLINE_NEEDLES = (0, 1, 2, 4, 8, 16)


def llama8b_128k(needles=4, seed=3):
    """Headline long context: the 8B shape at context 131072, batch 1, bf16
    KV, S 4, W 2048, 32 layers; needle density swept over HEADLINE_NEEDLES."""
    return Workload(f"llama8b_128k_n{needles}", B=1, Hq=32, Hkv=8, D=128,
                    L_cap=131072, seq_lens=[131072], kv_dtype="bf16", S=4,
                    W=2048, lam=0.10, needles=[needles], n_layers=32,
                    seed=seed * 1000 + needles)


def multiuser_8b(lam=0.10, seed=4, B=8):
    """Multi-user decode: 8 users of the 8B shape, bf16 KV, per-user context
    uniform in [65536, 131072], per-user needles uniform in [0, 16], S 4,
    W 2048, lambda in {0.05, 0.10, 0.20}."""
    key = layer_key(seed, 0)
    r = uniform_u32(key, 0, TENSOR_AUX, 0, AUX_USER, 2 * B)
    lens = [65536 + int((int(x) * 65537) >> 32) for x in r[:B]]
    ndl = [int((int(x) * 17) >> 32) for x in r[B:]]
    return Workload("multiuser_8b", B=B, Hq=32, Hkv=8, D=128, L_cap=131072,
                    seq_lens=lens, kv_dtype="bf16", S=4, W=2048, lam=lam,
                    needles=ndl, n_layers=32, seed=seed)


def llama70b_128k(seed=5):
    """Llama-3-70B-shaped attention: 64 q / 8 kv heads (group 8), D 128,
    bf16 KV, 4 users at context 131072, S 4, W 4096, lambda 0.10, 80
    layers; 4 needles per head."""
    return Workload("llama70b_128k", B=4, Hq=64, Hkv=8, D=128, L_cap=131072,
                    seq_lens=[131072] * 4, kv_dtype="bf16", S=4, W=4096,
                    lam=0.10, needles=[4] * 4, n_layers=80, seed=seed)


def scaled(w: Workload, L: int, **kw):
    """Same structure at a smaller context (every user at length L unless
    seq_lens is given)."""
    lens = kw.pop("seq_lens", [L] * w.B)
    return replace(w, L_cap=max(lens), seq_lens=list(lens), **kw)
