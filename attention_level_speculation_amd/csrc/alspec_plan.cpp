// Split plan: validation of the parameters, the sink / window / middle sets
// of every batch entry, their split into work items, and the workspace
// layout.  Host C++ only.
#include "alspec_plan.h"

#include <math.h>
#include <string.h>

namespace alspec {

namespace {

int ceil_div(int a, int b) { return (a + b - 1) / b; }

int pow2_floor(int x) {
  int r = 1;
  while (r * 2 <= x) r *= 2;
  return r;
}

}  // namespace

alspec_status make_plan(const alspec_params *p, PlanArgs *pa, Workspace *ws) {
  if (!p || !pa || !ws) return ALSPEC_ERR_INVALID_ARG;
  const int B = p->batch, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
  const int D = p->head_dim;
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || p->kv_capacity < 1)
    return ALSPEC_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ALSPEC_ERR_INVALID_ARG;
  if (!p->seq_lens) return ALSPEC_ERR_INVALID_ARG;
  if (p->sink < 0 || p->window < 0 ||
      (int64_t)p->sink + (int64_t)p->window < 1)
    return ALSPEC_ERR_INVALID_ARG;
  if (!(p->sm_scale > 0.f) || isinf(p->sm_scale)) return ALSPEC_ERR_INVALID_ARG;
  if (!(p->lambda >= 0.f)) return ALSPEC_ERR_INVALID_ARG;  // NaN, negative
  if (p->kv_dtype != ALSPEC_KV_F32 && p->kv_dtype != ALSPEC_KV_BF16)
    return ALSPEC_ERR_INVALID_ARG;
  if (p->split_tokens < 0 || p->window_split_tokens < 0)
    return ALSPEC_ERR_INVALID_ARG;
  if (p->overlap < 0 || p->overlap > 2) return ALSPEC_ERR_INVALID_ARG;
  for (int b = 0; b < B && b < kMaxBatch; ++b)
    if (p->seq_lens[b] < 1 || p->seq_lens[b] > p->kv_capacity)
      return ALSPEC_ERR_INVALID_ARG;
  const int G = Hq / Hkv;
  if (B > kMaxBatch || Hkv > kMaxKvHeads) return ALSPEC_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ALSPEC_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return ALSPEC_ERR_UNSUPPORTED;

  memset(pa, 0, sizeof *pa);
  pa->B = B;
  pa->Hq = Hq;
  pa->Hkv = Hkv;
  pa->G = G;
  pa->D = D;
  pa->L_cap = p->kv_capacity;

  // Sets of every entry.
  int max_win = 0;
  for (int b = 0; b < B; ++b) {
    const int L = p->seq_lens[b];
    const int s_end = p->sink < L ? p->sink : L;
    int64_t wb = (int64_t)L - (int64_t)p->window;
    if (wb < s_end) wb = s_end;
    pa->L[b] = L;
    pa->s_end[b] = s_end;
    pa->w_begin[b] = (int)wb;
    if (L - (int)wb > max_win) max_win = L - (int)wb;
  }

  // Middle split length: the shortest whole number of 64-token steps (at
  // least 256 tokens) whose splits number no more than one per CU, or one
  // per CU-round when the (entry, kv head) pairs alone outnumber the CUs.
  // With one split per CU every CU streams from start to end; with two or
  // more per CU the block dispatched first runs ahead of the others (the
  // wave arbiter favours older waves) and the CU streams its last stretch
  // with fewer loads in flight.
  int T = p->split_tokens;
  if (T == 0) {
    int pairs = 0, max_mid = 0;
    for (int b = 0; b < B; ++b) {
      const int m = pa->w_begin[b] - pa->s_end[b];
      if (m > 0) pairs += Hkv;
      if (m > max_mid) max_mid = m;
    }
    const int64_t target =
        (int64_t)kNominalCUs * ((pairs + kNominalCUs - 1) / kNominalCUs);
    auto items = [&](int64_t t) {
      int64_t n = 0;
      for (int b = 0; b < B; ++b) {
        const int64_t m = pa->w_begin[b] - pa->s_end[b];
        if (m > 0) n += Hkv * ((m + t - 1) / t);
      }
      return n;
    };
    int64_t lo = 4, hi = (max_mid + 63) / 64;  // in 64-token steps
    if (hi < lo) hi = lo;
    while (lo < hi) {                          // smallest fitting length
      const int64_t mid = (lo + hi) / 2;
      if (items(mid * 64) <= target) hi = mid; else lo = mid + 1;
    }
    T = (int)(lo * 64);
  }
  // Window split length: the windows of all (entry, kv head) pairs are cut
  // into about 128 splits in all, which run side by side on half the CUs.
  // In a single step every split ends in a device-scope hand-off to the
  // merge, and those queue per XCD, so more splits cost more than they
  // save; the layer-pipelined launch has no hand-off (its merge runs in the
  // next launch) and was fastest at the same count.  A power of two from 64
  // to 1024 tokens: a longer split streams for long on one CU.
  int Tw = p->window_split_tokens;
  if (Tw == 0) {
    int pairs = 0;
    for (int b = 0; b < B; ++b)
      if (pa->L[b] > pa->w_begin[b]) pairs += Hkv;
    const int target = 128;
    const int pieces = pairs > 0 && pairs < target ? target / pairs : 1;
    Tw = max_win / pieces;
    if (Tw < 64) Tw = 64;
    if (Tw > 1024) Tw = 1024;
    Tw = pow2_floor(Tw);
  }
  pa->T = T;
  pa->Tw = Tw;

  int slots = 0;
  pa->itemA_pre[0] = 0;
  pa->itemM_pre[0] = 0;
  for (int b = 0; b < B; ++b) {
    const int L = pa->L[b], s_end = pa->s_end[b], wb = pa->w_begin[b];
    pa->nsink[b] = s_end > 0 ? 1 : 0;
    pa->nwin[b] = ceil_div(L - wb, Tw);
    pa->nmid[b] = ceil_div(wb - s_end, T);
    pa->slot_base[b] = slots;
    slots += pa->nsink[b] + pa->nwin[b] + pa->nmid[b];
    pa->itemA_pre[b + 1] =
        pa->itemA_pre[b] + (pa->nsink[b] + pa->nwin[b]) * Hkv;
    pa->itemM_pre[b + 1] = pa->itemM_pre[b] + pa->nmid[b] * Hkv;
  }
  pa->total_slots = slots;
  // Query heads per exact-merge block: the most of 4, 2 and 1 for which
  // every head's middle states still fit one memory round of the merge
  // (8192 / (NH D) slots), 4 only where there are many (entry, head)
  // pairs.  Fewer blocks then take the verify's device-scope hand-off.  The
  // choice sets the merge's summation order, so every merging kernel takes
  // it from here.
  int max_mid = 0;
  for (int b = 0; b < B; ++b)
    if (pa->nmid[b] > max_mid) max_mid = pa->nmid[b];
  pa->NHv = (Hq % 4 == 0 && B * Hq >= 128 && max_mid <= 2048 / D) ? 4
            : (Hq % 2 == 0 && max_mid <= 4096 / D)                  ? 2
                                                                    : 1;

  size_t off = 0;
  ws->off_counters = off;
  off += kCounterBytes;
  ws->off_part_ml = off;
  off = align_up(off + (size_t)slots * Hq * 8, kWsAlign);
  ws->off_part_acc = off;
  off = align_up(off + (size_t)slots * Hq * D * 4, kWsAlign);
  ws->off_stA_ml = off;
  off = align_up(off + (size_t)B * Hq * 8, kWsAlign);
  ws->off_stA_acc = off;
  off = align_up(off + (size_t)B * Hq * D * 4, kWsAlign);
  ws->off_headnd = off;
  off = align_up(off + (size_t)B * Hq * 8, kWsAlign);
  ws->off_chain_ctl = off;
  off = align_up(off + kChainCtlBytes, kWsAlign);
  ws->off_chain_table = off;
  off = align_up(off + kChainMaxLayers * kChainEntryBytes, kWsAlign);
  ws->total = off;
  return ALSPEC_OK;
}

}  // namespace alspec
