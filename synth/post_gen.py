"""Seeded synthetic inputs of the post-attention operators: activations and
random bf16 weights of a Llama-shaped decoder layer.  Shared by the oracle's
and the GPU library's tests and by the benchmark; holds none of the
operators' arithmetic.

Weights are N(0, 1/fan_in) rounded to bf16 (so each product keeps unit
scale); the RMSNorm weights are 1 + 0.1 N(0, 1).  Activations are N(0, 1)
fp32.  Everything comes from one numpy Generator seeded with `seed`, in a
fixed order.  For a chain of layers, plant_query_direction points each
next query at the next layer's planted sink direction (see there).
"""
from dataclasses import dataclass

import numpy as np

from .gen import f32_to_bf16_bits

NAMES = ("w_o", "norm_mlp", "w_gate", "w_up", "w_down", "norm_attn", "w_qkv")


@dataclass
class PostShape:
    name: str
    B: int
    attn_dim: int
    hidden: int
    ffn: int
    qkv_dim: int
    eps: float = 1e-5
    seed: int = 11

    def shapes(self):
        return {"w_o": (self.hidden, self.attn_dim),
                "norm_mlp": (self.hidden,),
                "w_gate": (self.ffn, self.hidden),
                "w_up": (self.ffn, self.hidden),
                "w_down": (self.hidden, self.ffn),
                "norm_attn": (self.hidden,),
                "w_qkv": (self.qkv_dim, self.hidden)}

    def weight_bytes(self):
        return sum(int(np.prod(s)) * 2 for s in self.shapes().values())


def llama8b(B=1, seed=11):
    """Llama-3-8B decoder layer: 32 x 128 attention output, width 4096,
    MLP 14336, next QKV (32 + 8 + 8) x 128."""
    return PostShape("llama8b", B, 4096, 4096, 14336, 6144, 1e-5, seed)


def llama70b(B=4, seed=12):
    """Llama-3-70B decoder layer: 64 x 128, width 8192, MLP 28672, next QKV
    (64 + 8 + 8) x 128."""
    return PostShape("llama70b", B, 8192, 8192, 28672, 10240, 1e-5, seed)


def weights(s: PostShape):
    """dict name -> uint16 bf16 bit array of the layer's weights."""
    rng = np.random.default_rng(s.seed)
    out = {}
    for n, shape in s.shapes().items():
        if n.startswith("norm"):
            v = 1.0 + 0.1 * rng.standard_normal(shape, dtype=np.float32)
        else:
            v = rng.standard_normal(shape, dtype=np.float32)
            v *= np.float32(1.0 / np.sqrt(shape[1]))
        out[n] = f32_to_bf16_bits(v)
    return out


def activations(s: PostShape, step: int = 0):
    """(o [B][attn_dim], h_in [B][hidden]) fp32 for token `step`."""
    rng = np.random.default_rng((s.seed, 1000 + step))
    o = rng.standard_normal((s.B, s.attn_dim), dtype=np.float32)
    h = rng.standard_normal((s.B, s.hidden), dtype=np.float32)
    return o, h


# The chained decode step's residual stream: one coordinate far above the
# others, through which the next QKV's query rows are pointed at the next
# layer's planted sink direction (plant_query_direction).
MASSIVE_DIM = 1234
MASSIVE_VALUE = 2.0e3


def plant_query_direction(w_qkv, norm_attn, dirs, a, D, G, hidden,
                          dim=MASSIVE_DIM):
    """Make the query rows of a QKV weight point at planted directions.

    w_qkv: float tensor [qkv_dim][hidden] (query rows first, head-major),
    norm_attn: float tensor [hidden], both modified in place (torch tensors
    on any device, before rounding to bf16); dirs: one unit vector of D
    floats per kv head; a: the planted query component.  With a residual
    stream whose coordinate `dim` is far above the others, RMSNorm maps that
    coordinate to about sqrt(hidden) whatever the rest holds; the norm's
    weight is set to 1 there and the column `dim` of query head h (kv head
    h // G) to a * dirs[h // G] / sqrt(hidden), so the query carries
    a * dirs[g] plus the random product of the other coordinates, as the
    generator's queries carry a * u."""
    import torch
    norm_attn[dim] = 1.0
    scale = a / float(hidden) ** 0.5
    for g, u in enumerate(dirs):
        col = torch.as_tensor(u, dtype=torch.float32).to(w_qkv.device) * scale
        for hq in range(g * G, (g + 1) * G):
            w_qkv[hq * D:(hq + 1) * D, dim] = col
