"""CPU oracle of the post-attention operators of one decoder layer.

TEST INFRASTRUCTURE ONLY: the plain double-precision definition the GPU
library's post-attention kernels are checked against.  Only the tests and
the benchmark may use it; it shares no code with the GPU library.

The operators ("Attention-Level Speculation", research-map page, summary
and Approach: the post-attention ops that run speculatively on the
approximate attention output) follow the Llama decoder layer of the pages'
8B and 70B shapes:
  h1  = h_in + W_o o
  x   = rmsnorm(h1) * norm_mlp,  rmsnorm(v) = v / sqrt(mean(v^2) + eps)
  m   = silu(W_gate x) * (W_up x),  silu(t) = t / (1 + exp(-t))
  h2  = h1 + W_down m
  qkv = W_qkv (rmsnorm(h2) * norm_attn)
Each step is written as its definition, one matrix product at a time, in
float64 on the exact bf16 weight values and fp32 activations.

Parity status (tests/test_oracle_post.py): pinned by plain-loop brute force
on small shapes, the identity-projection closed form, the unit RMS of a
normed output, textbook values of silu, the scale invariance of RMSNorm and
the affinity of the residual in the attention output.
"""
import numpy as np


def bf16_bits_to_f64(bits):
    """Exact value of bf16 bit patterns: the high half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def rmsnorm(v, g, eps):
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * g


def silu(t):
    return t / (1.0 + np.exp(-t))


def post_attention(o, h_in, w, eps):
    """(h_out, qkv) in float64 for activations o [B][attn_dim], h_in
    [B][hidden] and a dict of bf16 weight bit arrays (see module doc)."""
    o = np.asarray(o, dtype=np.float64)
    h_in = np.asarray(h_in, dtype=np.float64)
    W = {n: bf16_bits_to_f64(v) for n, v in w.items()}
    h1 = h_in + o @ W["w_o"].T
    x = rmsnorm(h1, W["norm_mlp"], eps)
    m = silu(x @ W["w_gate"].T) * (x @ W["w_up"].T)
    h2 = h1 + m @ W["w_down"].T
    qkv = rmsnorm(h2, W["norm_attn"], eps) @ W["w_qkv"].T
    return h2, qkv
