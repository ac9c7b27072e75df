"""Chained decode of a stack of layers with the post-attention work run
speculatively on the approximate attention output and replayed on a
discard ("Attention-Level Speculation", research-map page, summary and
Approach: the post-attention ops run speculatively while exact attention
is computed, and a relative L2 check commits or discards them).

Scheduling only: every step is a call of the C ABI (the attention step,
alspec_spec_decode or its separate calls, and the post-attention
operators, alspec_post_attention), enqueued on HIP streams.  Whether a
layer's replay does any work is decided on the device: the replay kernels
read the layer's commit flag and end at once where it is set, so the
sequence of launches is static and the work dynamic.  The two-stream form
is issued eagerly only: its two streams wait on each other in turn, and
capturing that into a HIP graph ended in a host segmentation fault inside
hipStreamEndCapture with the HIP runtime torch loads, so model_step
refuses it (ValueError, nothing enqueued) while either stream is
capturing.  The one-stream form (one_stream=True) issues the same work in
dependency order on one stream, so the whole stack of layers captures
into one HIP graph.

Per layer l, with q_l the first Hq*D entries of the previous layer's QKV
projection (one decode token, batch 1):
  stream_exact:  alspec_spec_decode (sequential mode: approximation, exact
                 split-K pass, merge, verify and commit); it hands the
                 approximate output to stream_approx as soon as it exists
  stream_approx: post-attention on o_approx -> h_{l+1}, qkv_{l+1}
                 (speculative; runs beside the exact pass)
  stream_exact:  waits for it, then post-attention on o_exact with the
                 commit flag as skip flag -> overwrites h_{l+1}, qkv_{l+1}
                 only after a discard
so layer l+1 starts from the committed output of layer l: o_approx where
the verify committed it, else o_exact.  The result equals the plain
sequence "alspec_spec_decode, then post-attention on o_committed" bit for
bit (model_step with speculative=False).

The one-stream form, per layer on stream_exact: alspec_sink_approx, the
post-attention work on o_approx, alspec_flash_decode_exact over the middle
splits, alspec_lse_combine, alspec_verify, then the replay on o_exact with
the commit flag as skip flag.  The speculative work runs before the exact
pass instead of beside it (on one GPU both stream from the same HBM, so
running them side by side buys nothing), and the result is again the
committed output's post-attention work.
"""
from . import _binding as B_


class ModelLayer:
    """Device buffers of one layer of the chained step."""

    def __init__(self, k, v, weights, out, h_in, h_out, qkv_out):
        self.k, self.v = k, v
        self.weights = weights   # PostWeights struct (bf16 device pointers)
        self.out = out           # alloc_outputs dict of the attention step
        self.h_in, self.h_out, self.qkv_out = h_in, h_out, qkv_out


def q_view(p, qkv):
    """The query part of a QKV projection row as the attention input
    [1][Hq][D] (contiguous for batch 1)."""
    if p.batch != 1:
        raise ValueError("the chained step takes one decode token (batch 1)")
    return qkv[:, :p.num_q_heads * p.head_dim].view(1, p.num_q_heads,
                                                   p.head_dim)


def model_step(h, p, pp, q0, layers, ws_attn, ws_post_a, ws_post_b,
               stream_approx, stream_exact, speculative=True, exact_only=False,
               one_stream=False):
    """Enqueue one decode token through `layers` (list of ModelLayer).

    p: attention params (batch 1; p.overlap is ignored: the sequential mode
    is used); pp: PostParams; q0: the first layer's query [1][Hq][D];
    ws_attn: attention workspace; ws_post_a / ws_post_b: post-attention
    workspaces of the two streams.  speculative=False runs the same
    arithmetic as one sequence on stream_exact; exact_only=True runs exact
    attention (every split, no approximation or verify) and the
    post-attention work on its output, the non-speculative baseline;
    one_stream=True (with speculative) runs the speculative form on
    stream_exact alone, in an order a stream capture can record.  Layer l's
    query is layers[l-1].qkv_out's query part.  The two-stream speculative
    form raises ValueError, before enqueuing anything, if either stream is
    capturing into a HIP graph."""
    if p.batch != 1 or pp.batch != 1:
        raise ValueError("the chained step takes one decode token (batch 1)")
    if (speculative and not one_stream and not exact_only and
            (B_.stream_is_capturing(stream_approx) or
             B_.stream_is_capturing(stream_exact))):
        raise ValueError("the two-stream speculative step is not captured "
                         "(its capture crashed the HIP runtime's "
                         "hipStreamEndCapture); use one_stream=True under "
                         "stream capture")
    p0 = B_.Params.from_buffer_copy(p)
    p0.overlap = 0
    sa = stream_approx if speculative else stream_exact
    se = stream_exact
    q = q0
    for layer in layers:
        o = layer.out
        if exact_only:
            B_.flash_decode_exact(h, p0, q, layer.k, layer.v, 1, ws_attn, se)
            B_.lse_combine(h, p0, ws_attn, o["o_exact"], o["lse_exact"], se)
            B_.post_attention(h, pp, layer.weights, o["o_exact"].view(1, -1),
                              layer.h_in, layer.h_out, layer.qkv_out,
                              ws_post_b, stream=se)
        elif speculative and one_stream:
            B_.sink_approx(h, p0, q, layer.k, layer.v, o["o_approx"],
                           o["lse_approx"], ws_attn, se)
            B_.post_attention(h, pp, layer.weights, o["o_approx"].view(1, -1),
                              layer.h_in, layer.h_out, layer.qkv_out,
                              ws_post_a, stream=se)
            B_.flash_decode_exact(h, p0, q, layer.k, layer.v, 0, ws_attn, se)
            B_.lse_combine(h, p0, ws_attn, o["o_exact"], o["lse_exact"], se)
            B_.verify(h, p0, o["o_approx"], o["o_exact"], o["ratio"],
                      o["commit"], o["o_committed"], se)
            B_.post_attention(h, pp, layer.weights, o["o_exact"].view(1, -1),
                              layer.h_in, layer.h_out, layer.qkv_out,
                              ws_post_b, skip=o["commit"], stream=se)
        elif speculative:
            B_.spec_decode(h, p0, q, layer.k, layer.v, o, ws_attn,
                           stream_approx=sa, stream_exact=se)
            B_.post_attention(h, pp, layer.weights, o["o_approx"].view(1, -1),
                              layer.h_in, layer.h_out, layer.qkv_out,
                              ws_post_a, stream=sa)
            se.wait_stream(sa)
            B_.post_attention(h, pp, layer.weights, o["o_exact"].view(1, -1),
                              layer.h_in, layer.h_out, layer.qkv_out,
                              ws_post_b, skip=o["commit"], stream=se)
        else:
            B_.spec_decode(h, p0, q, layer.k, layer.v, o, ws_attn,
                           stream_approx=se, stream_exact=se)
            B_.post_attention(h, pp, layer.weights,
                              o["o_committed"].view(1, -1), layer.h_in,
                              layer.h_out, layer.qkv_out, ws_post_b,
                              stream=se)
        q = q_view(p, layer.qkv_out)

