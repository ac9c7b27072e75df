// Launchers of the gfx950 kernels (host functions defined in
// alspec_kernels.hip).  Each enqueues its kernel(s) on `s` and returns the
// HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "alspec_plan.h"

namespace alspec {

struct WsPtrs {
  unsigned *counters;
  float2 *part_ml;   // [slots][Hq] (m, l), m in log2 units
  float *part_acc;   // [slots][Hq][D]
  float2 *stA_ml;    // [B][Hq] merged sink+window state
  float *stA_acc;    // [B][Hq][D]
  float2 *headnd;    // [B][Hq] per-head (num, den) of the verify
};

WsPtrs ws_ptrs(void *ws, const Workspace &wl);

// Output buffers of the merging kernel modes (any may be null where a
// mode does not write it; lse_* and o_committed are always optional).
struct Outs {
  float *o_approx, *lse_approx, *o_exact, *lse_exact, *ratio;
  uint8_t *commit;
  float *o_committed;
  float lambda;
};

// Which splits a partials launch computes.
enum PartialsSet { kPartialsMiddle = 0, kPartialsApprox = 1, kPartialsAll = 2 };

// Split states over the sink and window splits, the middle splits, or all
// of them (one launch), into the workspace slots.
hipError_t launch_partials(const PlanArgs &pa, int kv_dtype, PartialsSet set,
                           const float *q, const void *k, const void *v,
                           float sm_log2, const WsPtrs &w, hipStream_t s);

// The whole approximation in one launch (split states, then the merge by
// the last block of each (entry, kv head)): o.o_approx, o.lse_approx and the
// reusable merged state.
hipError_t launch_approx_fused(const PlanArgs &pa, int kv_dtype,
                               const float *q, const void *k, const void *v,
                               float sm_log2, const WsPtrs &w, const Outs &o,
                               hipStream_t s);

// Merge of the sink+window states (written by an earlier launch) into
// o.o_approx, o.lse_approx and the reusable merged state.
hipError_t launch_approx_combine(const PlanArgs &pa, const WsPtrs &w,
                                 const Outs &o, hipStream_t s);

// Exact merge of the stored sink+window state with the middle splits, then
// the relative L2 verify, the commit flag and the committed output (o.*).
hipError_t launch_merge_verify(const PlanArgs &pa, const WsPtrs &w,
                               const Outs &o, hipStream_t s);

// Exact merge of every split state of the plan.
hipError_t launch_lse_combine(const PlanArgs &pa, const WsPtrs &w,
                              float *o_exact, float *lse_exact, hipStream_t s);

// One layer's inputs, workspace and outputs in a layer-pipelined launch.
struct ChainLayer {
  const float *q;
  const void *k, *v;
  WsPtrs w;
  Outs o;
};

// One layer-pipelined launch in one grid: the merge of `mid`'s sink and
// window states (split by an earlier launch) if `merge_mid`, the middle
// splits of `mid`, the sink and window splits of `app`, and the exact
// merge, verify and commit of `ver` (each layer may be null).
hipError_t launch_chain(const PlanArgs &pa, int kv_dtype,
                        const ChainLayer *mid, const ChainLayer *app,
                        const ChainLayer *ver, bool merge_mid, float sm_log2,
                        hipStream_t s);

// One layer of the one-launch chain, as its entry in the layer table: its
// inputs, the base of its workspace (the layout is the plan's), its
// outputs, and the latest earlier layer of the chain on the same workspace
// (-1 if none).
struct ChainEntry {
  const float *q;
  const void *k, *v;
  char *ws;
  float *o_approx, *lse_approx, *o_exact, *lse_exact, *ratio;
  uint8_t *commit;
  float *o_committed;
  int prev;
  int unused;
};
static_assert(sizeof(ChainEntry) == kChainEntryBytes, "table entry");

// The one-launch chain over the n layers of `table` (device), with its
// control block at `ctl` (device, zero when the launch starts; zero again
// when it ends).
struct OneChainArgs {
  int n;
  float lambda;
  char *ctl;
  const ChainEntry *table;
  unsigned off_counters, off_part_ml, off_part_acc, off_stA_ml, off_stA_acc,
      off_headnd;
};

// Copies n host-side entries into the device table at dst (kernel
// arguments, so no host memory needs to stay valid after the call).
hipError_t launch_chain_table(const ChainEntry *src, int n, ChainEntry *dst,
                              hipStream_t s);

// The launch itself: one block per queue item.
hipError_t launch_one_chain(const PlanArgs &pa, int kv_dtype,
                            const OneChainArgs &ca, float sm_log2,
                            hipStream_t s);

// Length of the one-launch chain's queue (host): the first layer's sink and
// window splits, then per layer s of n: its merge of sink and window
// states, the next layer's sink and window splits (but after the last
// layer), its middle splits and the verify of the layer before (but for
// the first layer); then the last layer's verify.
inline int one_chain_items(const PlanArgs &pa, int n) {
  const int nG = pa.B * pa.Hkv, nA = pa.itemA_pre[pa.B];
  const int nM = pa.itemM_pre[pa.B], nV = pa.B * pa.Hq / pa.NHv;
  return nA + n * (nG + nM) + (n - 1) * (nA + nV) + nV;
}

// Standalone verify of two output buffers.
hipError_t launch_verify(const PlanArgs &pa, const float *o_approx,
                         const float *o_exact, float *ratio, uint8_t *commit,
                         float *o_committed, float lambda, hipStream_t s);

// Shape of the post-attention operators (validated by the caller).
struct PostShape {
  int batch, attn_dim, hidden, ffn, qkv_dim;
  float eps;
};

// Buffers of the post-attention operators: bf16 weights (uint16 bits),
// fp32 activations, optional skip flags ([batch], nonzero: leave that
// entry's outputs untouched).
struct PostPtrs {
  const uint16_t *w_o, *norm_mlp, *w_gate, *w_up, *w_down, *norm_attn, *w_qkv;
  const float *o, *h_in;
  float *h_out, *qkv, *m;  // m: [batch][ffn] scratch
  const uint8_t *skip;
};

// Output projection with residual, RMSNorm + gated MLP, down projection
// with residual, RMSNorm + next layer's QKV: four launches on `s`.
hipError_t launch_post_attention(const PostShape &sh, const PostPtrs &p,
                                 hipStream_t s);

}  // namespace alspec
