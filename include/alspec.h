/*
 * alspec.h -- C ABI of the speculative flash-decode step of attention-level
 * speculation (ALSpec) on AMD Instinct MI355X (gfx950).
 *
 * The method, as the pages state it ("Attention-Level Speculation",
 * atlas.scime.ai summary, sections Summary and Approach; ICML 2025 poster
 * page, abstract): each layer's self-attention output is speculated with a
 * cheap attention-sink approximation, exact attention is computed while the
 * work after attention proceeds on the approximation, and the approximation
 * is then verified with a relative L2 threshold (lambda = 0.10 in the
 * evaluation, Key results) and committed or discarded.  The pages name a
 * speculative flash-decode kernel and flash decoding as its basis; this
 * library is a new gfx950 design of that step for one decode token.
 *
 * Notation.  B batch entries (one user's token through one layer each), Hq
 * query heads, Hkv kv heads, G = Hq / Hkv query heads per kv head (query
 * head h reads kv head h / G), head dimension D, per-entry context length
 * L_b <= L_cap.  With S' = min(S, L_b):
 *   sink   = tokens [0, S'),
 *   window = tokens [max(S', L_b - W), L_b),
 *   middle = tokens [S', max(S', L_b - W)).
 * The approximation is softmax attention over sink + window, renormalised
 * over that set; exact attention covers [0, L_b).  Logits are
 * sm_scale * <q, k>.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless marked "host".  Layouts are dense
 *    row-major with the last index fastest:
 *      q, o_*        : float32 [B][Hq][D]
 *      k, v          : [B][Hkv][L_cap][D] of the kv dtype (float32, or bf16
 *                      stored as 16-bit patterns), 16-byte aligned
 *      lse_*         : float32 [B][Hq] (natural log of the softmax
 *                      normaliser, logits included)
 *      ratio         : float32 [B];  commit : uint8 [B] (1 = commit)
 *    q, k, v and the o_* arrays must be 16-byte aligned.
 *  - The caller owns every buffer and stream.  The library allocates no
 *    device memory and keeps no pointer after a call returns.
 *  - Compute calls only enqueue work on the given stream(s); they do not
 *    synchronise.  Arguments are validated on the host first; on any
 *    validation failure nothing is enqueued and a status other than
 *    ALSPEC_OK is returned.  A HIP launch error is reported as
 *    ALSPEC_ERR_HIP.  No C++ exception crosses this interface.
 *  - Streams are hipStream_t values passed as void* (NULL = the legacy
 *    default stream); events are hipEvent_t passed as void*.
 *  - Workspace: size from alspec_workspace_size.  A new workspace must be
 *    zero-filled once before its first use; every call leaves the
 *    workspace's internal counters at zero again when its work completes.
 *    Calls whose work may overlap in time must not share a workspace.
 *    The pointer must be 256-byte aligned.
 *  - Handles: one handle may be used by one host thread at a time.
 */
#ifndef ALSPEC_H
#define ALSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ALSPEC_OK = 0,
  ALSPEC_ERR_INVALID_ARG = 1, /* null pointer, bad size, out-of-range value */
  ALSPEC_ERR_UNSUPPORTED = 2, /* valid, but outside the built shapes or
                                 not available in this context */
  ALSPEC_ERR_WORKSPACE = 3,   /* workspace too small or misaligned */
  ALSPEC_ERR_HIP = 4          /* the HIP runtime reported an error */
} alspec_status;

typedef enum { ALSPEC_KV_F32 = 0, ALSPEC_KV_BF16 = 1 } alspec_kv_dtype;

/* Shape and method parameters of one call (all fields host values). */
typedef struct {
  int32_t batch;        /* B, 1 .. ALSPEC_MAX_BATCH */
  int32_t num_q_heads;  /* Hq, multiple of num_kv_heads */
  int32_t num_kv_heads; /* Hkv, 1 .. ALSPEC_MAX_KV_HEADS */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t kv_capacity;  /* L_cap: token stride of k and v */
  const int32_t *seq_lens; /* host [B], 1 <= L_b <= L_cap */
  int32_t kv_dtype;     /* alspec_kv_dtype */
  int32_t sink;         /* S >= 0 */
  int32_t window;       /* W >= 0, S + W >= 1 */
  float sm_scale;       /* logit scale, > 0 and finite (normally 1/sqrt(D)) */
  float lambda;         /* verify threshold, >= 0 (+inf allowed, NaN not) */
  int32_t split_tokens;        /* middle split length; 0 = automatic: the
                                  shortest multiple of 64 tokens (at least
                                  256) giving at most one middle split per
                                  CU of an MI355X (256), or per round of
                                  256 when the (entry, kv head) pairs are
                                  more.  Results depend on the split plan
                                  only through rounding order. */
  int32_t window_split_tokens; /* window split length; 0 = automatic: the
                                  longest window over (128 / pairs),
                                  rounded down to a power of two from 64
                                  to 1024 tokens, pairs being the (entry,
                                  kv head) pairs with a window.  Every
                                  entry point takes the same plan, so the
                                  layered and single calls give the same
                                  bits. */
  int32_t overlap; /* 0 = sequential, 1 = overlapped, 2 = pipelined (see
                      alspec_spec_decode); alspec_spec_decode_layers: 0 or
                      2 = one launch per chain, 1 = one launch per layer */
} alspec_params;

#define ALSPEC_MAX_BATCH 64
#define ALSPEC_MAX_KV_HEADS 64
/* group sizes G = Hq / Hkv that are built: 1, 2, 4, 8 */

/* Optional timing events recorded around the fused call's kernels (any
 * member may be NULL; each a hipEvent_t created with timing enabled).
 * approx_* bracket the approximation's kernels, exact_begin/exact_end only
 * the middle split-K kernel, verify_end follows the merge and verify.  They
 * are recorded on the stream that runs those kernels: in overlap mode 0
 * all on stream_exact; in mode 1 approx_* on stream_approx; in mode 2 also
 * verify_end on the handle's verify stream.  Inside a stream capture they
 * are recorded with hipEventRecordExternal (timestamp nodes of the graph);
 * a HIP runtime without that support fails the call with ALSPEC_ERR_HIP,
 * so pass NULL events to calls that are captured. */
typedef struct {
  void *approx_begin, *approx_end;
  void *exact_begin, *exact_end;
  void *verify_end;
} alspec_events;

typedef struct alspec_handle alspec_handle;

/* Human-readable name of a status code (static string, never NULL). */
const char *alspec_status_string(alspec_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t alspec_version(void);

/* Text naming the HIP call and HIP error behind the most recent
 * ALSPEC_ERR_HIP returned on the calling thread, or the sizes behind an
 * ALSPEC_ERR_WORKSPACE of alspec_spec_decode_noalloc ("" if none yet).
 * The string is thread-local and stays valid until the thread's next
 * failing call. */
const char *alspec_last_error(void);

/* Bytes of workspace the compute calls need for these parameters.  Pure
 * host computation (no GPU needed); validates the parameters. */
alspec_status alspec_workspace_size(const alspec_params *p, size_t *bytes);

/* Inspection of the split plan (pure host): the splits of batch entry b in
 * slot order, as kind (0 sink, 1 window, 2 middle) and token range
 * [begin, end).  At most `cap` entries are written to the host arrays;
 * *count receives the number of splits.  Also reports the chosen middle
 * and window split lengths if the pointers are non-NULL. */
alspec_status alspec_plan_splits(const alspec_params *p, int32_t b,
                                 int32_t *kind, int32_t *begin, int32_t *end,
                                 int32_t cap, int32_t *count,
                                 int32_t *split_tokens,
                                 int32_t *window_split_tokens);

/* Create a handle bound to HIP device `device`: the events the fused call
 * uses for cross-stream ordering, a 16-entry table of workspace events and
 * the pipelined mode's verify stream (default priority).  *out is set on
 * success. */
alspec_status alspec_create(int device, alspec_handle **out);
alspec_status alspec_destroy(alspec_handle *h);

/*
 * Attention-sink approximation (the cheap speculative attention of
 * "Attention-Level Speculation", atlas.scime.ai research-map page, summary
 * and Approach): softmax attention of each query over
 * the sink and window tokens only, renormalised over that set.  Writes
 * o_approx [B][Hq][D] and, if non-NULL, lse_approx [B][Hq].  Also leaves in
 * `ws` the per-split states of the sink and window tokens and their merged
 * state, which alspec_lse_combine and the fused call reuse.
 */
alspec_status alspec_sink_approx(alspec_handle *h, const alspec_params *p,
                                 const float *q, const void *k, const void *v,
                                 float *o_approx, float *lse_approx, void *ws,
                                 size_t ws_bytes, void *stream);

/*
 * Split-K flash decoding over the KV cache (flash decoding, which the pages
 * list as a building block, atlas.scime.ai summary, "Builds on"): each
 * (batch entry, kv head, token split) produces the softmax state
 * (running max, normaliser, weighted value sum) of its G query heads, stored
 * in `ws`.  include_sink_window = 1 computes every split (sink, window and
 * middle); 0 computes the middle splits only, for use after
 * alspec_sink_approx on the same workspace.
 */
alspec_status alspec_flash_decode_exact(alspec_handle *h,
                                        const alspec_params *p,
                                        const float *q, const void *k,
                                        const void *v,
                                        int32_t include_sink_window, void *ws,
                                        size_t ws_bytes, void *stream);

/*
 * Log-sum-exp combine of split states into exact attention: flash
 * decoding's merge of per-range softmax states, which the pages name as a
 * building block ("Attention-Level Speculation", atlas.scime.ai summary,
 * "Builds on").  Every split state of the plan must be present in `ws`
 * (sink, window and middle splits: alspec_flash_decode_exact with
 * include_sink_window = 1, or alspec_sink_approx followed by
 * alspec_flash_decode_exact with 0).  Writes o_exact [B][Hq][D] and, if
 * non-NULL, lse_exact [B][Hq].
 *
 * `ws` is written as well as read: the call first merges the sink and
 * window states into the workspace's merged sink+window state (the same
 * state alspec_sink_approx leaves there, with the same bits), then merges
 * the middle states onto it.  So the call may not overlap in time with any
 * other call on the same workspace.
 */
alspec_status alspec_lse_combine(alspec_handle *h, const alspec_params *p,
                                 void *ws, size_t ws_bytes, float *o_exact,
                                 float *lse_exact, void *stream);

/*
 * Relative L2 verification (the check that decides commit or discard in
 * "Attention-Level Speculation", atlas.scime.ai research-map page, summary
 * and Approach): per batch entry b over its Hq*D outputs (16-byte aligned,
 * like o_committed), ratio = ||o_approx - o_exact||_2 / ||o_exact||_2
 * (0 if both norms are 0, +inf if only the exact norm is 0, NaN if any
 * input is NaN) and commit = (ratio <= lambda).  If o_committed is non-NULL
 * it receives o_approx for committed entries and o_exact otherwise.
 */
alspec_status alspec_verify(alspec_handle *h, const alspec_params *p,
                            const float *o_approx, const float *o_exact,
                            float *ratio, uint8_t *commit, float *o_committed,
                            void *stream);

/*
 * The whole speculative step (atlas.scime.ai summary, Approach; ICML poster
 * abstract: the approximation lets later work start early while exact
 * attention runs, then a verify commits or discards).  Writes o_approx
 * (and lse_approx if non-NULL), o_exact (and lse_exact if non-NULL), the
 * per-entry ratio and commit flag and, if non-NULL, o_committed.
 *
 * With p->overlap == 0 (default) every kernel runs on stream_exact: the
 * sink and window splits and their merge (o_approx), then the middle
 * splits, then the merge with the reused sink/window state, the verify and
 * the commit.  stream_approx is made to wait for the approximation only,
 * so work enqueued on stream_approx after this call may consume o_approx
 * while the exact pass runs.
 *
 * With p->overlap == 1 the approximation runs on stream_approx while the
 * middle splits run on stream_exact; the exact merge, verify and commit
 * follow on stream_exact once both are done.  Successive calls (under
 * speculation, the layers of one decode step, each exact pass ordered by
 * the caller after the approximation that produced its q) pipeline when
 * each approximation needs to wait only for an earlier verify on its own
 * workspace.  This mode may be captured into a HIP graph.
 *
 * With p->overlap == 2 (pipelined) stream_exact
 * carries only the middle splits, so successive calls' exact passes run
 * back to back; the approximation runs on stream_approx (o_approx,
 * lse_approx complete in its order), and the merge, verify and commit run
 * on a stream owned by the handle once both are done, overlapping the next
 * call's exact pass; alspec_order_after_verify orders a caller's stream
 * after them.  Under stream capture the verify stream joins the capture;
 * the capture must then call alspec_order_after_verify on a capturing
 * stream before it ends, which joins it back.
 *
 * Workspace ordering: for uncaptured calls the handle remembers, for the
 * 16 most recently used workspaces, the event after the last fused call's
 * verify on it, and orders a later fused call on that workspace after it
 * (an overlap-1 call on a workspace with no such record first orders
 * stream_approx after all work queued on stream_exact).  Under stream
 * capture the library adds no workspace ordering: captured calls that
 * share a workspace, graph launches and uncaptured calls that share one,
 * and the standalone calls are ordered by the caller (for a captured
 * overlap-1 pipeline, simplest by giving each call its own workspace).
 * Ordering the exact pass after whatever produced q is the caller's task,
 * as for any input.
 *
 * Results are identical in all modes.  The two streams may be the same
 * stream; two distinct streams must both be outside any stream capture or
 * in the same one (else ALSPEC_ERR_INVALID_ARG, nothing enqueued).  `ev`
 * may be NULL.  Buffers written by a call must not be read by
 * the caller's own work until it is ordered after the call's completion on
 * the stream named above.
 */
alspec_status alspec_spec_decode(alspec_handle *h, const alspec_params *p,
                                 const float *q, const void *k, const void *v,
                                 float *o_approx, float *lse_approx,
                                 float *o_exact, float *lse_exact,
                                 float *ratio, uint8_t *commit,
                                 float *o_committed, void *ws,
                                 size_t ws_bytes, void *stream_approx,
                                 void *stream_exact, const alspec_events *ev);

/* Size of the static scratch of alspec_spec_decode_noalloc, per GPU. */
#define ALSPEC_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * For callers that cannot allocate device memory (work recorded under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * alspec_spec_decode with no workspace argument.  The workspace is a
 * static device array of ALSPEC_NOALLOC_SCRATCH_BYTES (16 MiB) inside the
 * library, one per GPU, set up by alspec_create (its device address looked
 * up and its counters cleared, once per device and process) and held until
 * the process ends.  The call allocates nothing; the caller still passes
 * every input and output, as to alspec_spec_decode, whose kernels and bits
 * it shares.
 *
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents: calls whose work overlaps in time on the same GPU race,
 * from any handle or thread.  Uncaptured calls through one handle are
 * ordered by its workspace table as alspec_spec_decode's are; calls through
 * different handles, and captured calls, are ordered by the caller.
 * Parameters whose workspace (alspec_workspace_size) exceeds the array
 * return ALSPEC_ERR_WORKSPACE with nothing enqueued, and alspec_last_error
 * then names both sizes.  A handle on a device past index 63 has no array
 * (ALSPEC_ERR_UNSUPPORTED).
 */
alspec_status alspec_spec_decode_noalloc(
    alspec_handle *h, const alspec_params *p, const float *q, const void *k,
    const void *v, float *o_approx, float *lse_approx, float *o_exact,
    float *lse_exact, float *ratio, uint8_t *commit, float *o_committed,
    void *stream_approx, void *stream_exact, const alspec_events *ev);

/* One layer's buffers for alspec_spec_decode_layers: as the arguments of
 * alspec_spec_decode (device pointers; lse_approx, lse_exact and
 * o_committed may be NULL). */
typedef struct {
  const float *q;
  const void *k, *v;
  float *o_approx, *lse_approx, *o_exact, *lse_exact, *ratio;
  uint8_t *commit;
  float *o_committed;
  void *ws;
  size_t ws_bytes;
} alspec_layer;

/* Workspaces of alspec_spec_decode_layers: layers fewer than this many
 * apart in one call must not share a workspace (either form), so a ring of
 * this many workspaces serves any chain. */
#define ALSPEC_LAYERS_WS_RING 3

/*
 * The fused step for a chain of n_layers layers of one decode step, on one
 * stream, layer-pipelined: the speculative order of "Attention-Level
 * Speculation" (atlas.scime.ai research-map page, summary and Approach:
 * downstream work starts on the approximation while exact attention is
 * still running), for layers whose queries are all given (independent
 * layers).  Each layer's outputs equal those of alspec_spec_decode (any
 * mode) on its inputs, bit for bit.
 *
 * p->overlap == 0 (default; 2 is taken as 0), one launch: a small kernel first
 * writes the table of the layers' buffers into the first layer's workspace;
 * then one launch runs the whole chain, its blocks taking work items, one
 * each, from a queue in that workspace: the first layer's sink and window
 * splits, then for each layer j in turn the merge of layer j's sink and window
 * states into its approximate output, layer j+1's sink and window splits,
 * layer j's middle splits and layer j-1's exact merge, verify and commit, and
 * last the last layer's verify.  A block takes the next item when it starts,
 * so faster compute units take more items, one layer's slowest blocks do not
 * delay the next layer's, and the launch's tail is paid once per call.  Items
 * that need others' results wait on per-layer completion counts, and a layer's
 * splits wait for the verify of the latest earlier layer on the same
 * workspace; every wait is bounded (one that runs out leaves that layer's
 * outputs wrong and counts itself in the workspace; it does not hang).  Chains
 * longer than 256 layers take one such pair of launches per 256 layers.
 *
 * p->overlap == 1, one launch per layer: launch j computes, in disjoint
 * block ranges of one grid, layer j's middle splits (dispatched first),
 * layer j+1's sink and window splits, the merge of layer j's sink and
 * window states (for j >= 1), and layer j-1's exact merge, verify and
 * commit; a last launch verifies layer n-1.  Stream order alone carries
 * the dependencies.
 *
 * A stack whose next query is computed from the approximate output runs
 * through the single-layer calls instead.  `layers` is a host array of
 * n_layers entries (>= 1), each validated as the arguments of
 * alspec_spec_decode; layers fewer than ALSPEC_LAYERS_WS_RING apart that
 * share a workspace return ALSPEC_ERR_WORKSPACE with nothing enqueued.
 * Calls sharing a workspace with other calls are ordered by the caller.
 * May be captured into a HIP graph.
 */
alspec_status alspec_spec_decode_layers(alspec_handle *h,
                                        const alspec_params *p,
                                        int32_t n_layers,
                                        const alspec_layer *layers,
                                        void *stream);

/* Orders `stream` after all merge, verify and commit work that pipelined
 * calls (p->overlap == 2) on this handle have enqueued so far.  Under
 * stream capture: joins the handle's verify stream back into the capture
 * of `stream` (OK and no work if no pipelined call was captured);
 * ALSPEC_ERR_UNSUPPORTED if the verify stream is part of another capture
 * or `stream` is not capturing while it is. */
alspec_status alspec_order_after_verify(alspec_handle *h, void *stream);

/* ---------------------------------------------------------------------
 * Post-attention operators of one decoder layer ("Attention-Level
 * Speculation", research-map page, summary and Approach: the work that the
 * method runs speculatively on the approximate attention output while the
 * exact attention is computed, and runs again on the exact output after a
 * discard).  They follow the Llama decoder layer of the pages' 8B and 70B
 * shapes, with weights the caller supplies (random here):
 *   h_out = h1 + W_down (silu(W_gate x) * (W_up x)),
 *           h1 = h_in + W_o o,  x = rmsnorm(h1) * norm_mlp
 *   qkv   = W_qkv (rmsnorm(h_out) * norm_attn)
 * with rmsnorm(v) = v / sqrt(mean(v^2) + eps), per batch entry.  Rotary
 * position embedding and the new token's K/V append are not applied: the
 * caller owns the cache (the attention calls take K/V that already hold
 * the current token).
 */
#define ALSPEC_POST_MAX_BATCH 8

typedef struct {
  int32_t batch;    /* B, 1 .. ALSPEC_POST_MAX_BATCH */
  int32_t attn_dim; /* width of the attention output (Hq * D), multiple of 8 */
  int32_t hidden;   /* model width, multiple of 8 */
  int32_t ffn;      /* MLP width, multiple of 8 */
  int32_t qkv_dim;  /* rows of the next layer's QKV projection, >= 1 */
  float eps;        /* RMSNorm epsilon, > 0 and finite */
} alspec_post_params;

/* Device pointers to bf16 weights (bit patterns, row-major, 16-byte
 * aligned); none may be NULL. */
typedef struct {
  const void *w_o;       /* [hidden][attn_dim] */
  const void *norm_mlp;  /* [hidden] */
  const void *w_gate;    /* [ffn][hidden] */
  const void *w_up;      /* [ffn][hidden] */
  const void *w_down;    /* [hidden][ffn] */
  const void *norm_attn; /* [hidden], the next layer's input norm */
  const void *w_qkv;     /* [qkv_dim][hidden], the next layer's projection */
} alspec_post_weights;

/* Workspace bytes of alspec_post_attention (the MLP activations,
 * B x ffn floats).  Pure host computation; validates the parameters. */
alspec_status alspec_post_workspace_size(const alspec_post_params *p,
                                         size_t *bytes);

/* The post-attention operators ("Attention-Level Speculation",
 * atlas.scime.ai summary, Approach: the work run speculatively on the
 * approximate output) for B entries, four kernel launches on `stream`, in
 * fp32 arithmetic on bf16 weights.
 *   o      fp32 [B][attn_dim] attention output (device)
 *   h_in   fp32 [B][hidden] residual stream in (device)
 *   h_out  fp32 [B][hidden] residual stream out (device; may equal h_in)
 *   qkv    fp32 [B][qkv_dim] next layer's projection (device)
 *   skip   uint8 [B] (device) or NULL: entries whose flag is nonzero are
 *          left untouched (h_out and qkv not written) -- with the commit
 *          flags of alspec_spec_decode this replays the operators on the
 *          exact output only where the speculation was discarded; the
 *          kernels read the flags on the device and end at once when every
 *          entry is skipped, so such a call can sit in a captured graph.
 *   ws     workspace of alspec_post_workspace_size bytes, 256-byte aligned
 * The caller owns every buffer; nothing is allocated or synchronised.
 * Pointers must be 16-byte aligned (ALSPEC_ERR_INVALID_ARG otherwise).
 * Results are deterministic: each output is summed in a fixed order.
 * h_out must not overlap o or qkv; with skip flags, h_out must not be
 * h_in (a skipped entry keeps its previous h_out). */
alspec_status alspec_post_attention(alspec_handle *h,
                                    const alspec_post_params *p,
                                    const alspec_post_weights *w,
                                    const float *o, const float *h_in,
                                    float *h_out, float *qkv,
                                    const uint8_t *skip, void *ws,
                                    size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ALSPEC_H */
