// Split plan and workspace layout of the speculative flash-decode step.
// Host-side C++ shared by the C ABI and the kernel launchers.  Holds no GPU
// code.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "alspec.h"

namespace alspec {

constexpr int kMaxBatch = ALSPEC_MAX_BATCH;
constexpr int kMaxKvHeads = ALSPEC_MAX_KV_HEADS;
constexpr size_t kWsAlign = 256;
// counters at the start of every workspace, independent of the shape, so a
// workspace reused for another shape still finds them at zero.  Each counter
// has a 128-byte line of its own (kCounterStride words), so the arrivals of
// different groups do not queue on one line's atomics:
//   kUserCounters + b * kCounterStride      heads done (exact merge), per b
//   kApproxCounters + (b * Hkv + g) * kCounterStride
//                                       sink/window splits done (one-launch
//                                       approximation), per (b, kv head)
constexpr int kCounterStride = 32;
constexpr int kUserCounters = 0;
constexpr int kApproxCounters = kUserCounters + kMaxBatch * kCounterStride;
constexpr int kNumCounters =
    kApproxCounters + kMaxBatch * kMaxKvHeads * kCounterStride;
// The one-launch chain (alspec_spec_decode_layers) keeps a control block in
// the workspace of the chain's first layer (every workspace has room for
// one): the queue, finished and error counters (a 128-byte line each), one
// line per layer with its counts of finished sink/window splits, middle
// splits, merges and verifies (words 0, 8, 16 and 24 of the line), and the
// table of the layers' buffers.  One launch covers up to kChainMaxLayers
// layers.
constexpr int kChainMaxLayers = 256;
constexpr size_t kChainCtlBytes = (size_t)(3 + kChainMaxLayers) * 128;
constexpr size_t kCounterBytes = (kNumCounters * 4 + 255) / 256 * 256;

// Everything a kernel needs to map a block index to its work; passed by
// value as a kernel argument.
struct PlanArgs {
  int B, Hq, Hkv, G, D, L_cap;
  int T;   // middle split length (tokens)
  int Tw;  // window split length (tokens)
  int NHv; // query heads per exact-merge block (1, 2 or 4)
  int total_slots;
  int L[kMaxBatch];
  int s_end[kMaxBatch];    // sink = [0, s_end)
  int w_begin[kMaxBatch];  // window = [w_begin, L), middle = [s_end, w_begin)
  int nsink[kMaxBatch];    // 0 or 1 sink split
  int nwin[kMaxBatch];     // window splits
  int nmid[kMaxBatch];     // middle splits
  int slot_base[kMaxBatch];       // first slot of user b: sink, window, middle
  int itemA_pre[kMaxBatch + 1];   // prefix of (nsink + nwin) * Hkv
  int itemM_pre[kMaxBatch + 1];   // prefix of nmid * Hkv
};

struct Workspace {
  size_t off_counters, off_part_ml, off_part_acc, off_stA_ml, off_stA_acc,
      off_headnd, off_chain_ctl, off_chain_table, total;
};

// Bytes of one entry of the one-launch chain's layer table.
constexpr size_t kChainEntryBytes = 96;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Nominal compute-unit count of an MI355X; the automatic split length aims
// at a few work items per CU.  The plan depends on the parameters only, so
// the workspace size needs no device.
constexpr int kNominalCUs = 256;

// Validate `p` and fill the plan (the same for every entry point).  Returns
// ALSPEC_OK or the status to report.
alspec_status make_plan(const alspec_params *p, PlanArgs *pa, Workspace *ws);

}  // namespace alspec
