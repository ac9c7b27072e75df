// gfx950 kernels of the speculative flash-decode step.
//
// Flash decoding (named by the pages as a building block: "Attention-Level
// Speculation", atlas.scime.ai summary, "Builds on") splits each context
// into token ranges, computes a softmax state (running max m, normaliser l,
// weighted value sum acc) per range and merges the states with log-sum-exp
// weights.  Here every work item is one (batch entry, kv head, token range);
// its block streams the range's K and V rows once from HBM and serves all G
// query heads of that kv head, so each KV byte is read once per step.  The
// sink and window ranges are computed first (the approximation, "a cheap
// attention-sink approximation", Approach) and their merged state is reused
// by the exact merge, so the approximation costs no extra KV traffic.
//
// Logits are kept in log2 units: q is pre-scaled by sm_scale * log2(e) and
// exponentials are exp2, which maps to the hardware v_exp_f32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "alspec_kernels.h"

namespace alspec {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Reference point for exponentials: the running max, or 0 while no token has
// been seen (keeps exp2(-inf - ref) = 0 instead of NaN).
__device__ __forceinline__ float exp_ref(float m) {
  return m == neg_inf() ? 0.f : m;
}

// ---------------------------------------------------------------- types ---

struct KvF32 {
  using elem = float;
  static constexpr int EPL = 4;  // elements per 16-byte load
  static __device__ __forceinline__ void unpack(const uint4 r, float *f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
};

struct KvBf16 {
  using elem = uint16_t;  // bf16 bit pattern
  static constexpr int EPL = 8;
  static __device__ __forceinline__ void unpack(const uint4 r, float *f) {
    // A bf16 is the high half of the float32 with the same value.
    f[0] = __uint_as_float(r.x << 16);
    f[1] = __uint_as_float(r.x & 0xffff0000u);
    f[2] = __uint_as_float(r.y << 16);
    f[3] = __uint_as_float(r.y & 0xffff0000u);
    f[4] = __uint_as_float(r.z << 16);
    f[5] = __uint_as_float(r.z & 0xffff0000u);
    f[6] = __uint_as_float(r.w << 16);
    f[7] = __uint_as_float(r.w & 0xffff0000u);
  }
};

// ------------------------------------------------------- lane reductions ---

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of
// a group ends with the same bits (each step adds a value to its partner's,
// and IEEE addition is commutative).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// ------------------------------------------------- one split of one head ---

// Softmax state of the G query heads of one kv head over tokens [t0, t1).
// The block's 4 waves each own one contiguous quarter of every block-step of
// tokens; inside a wave, LPR lanes hold one K/V row (16 bytes each), so one
// load instruction covers RPI consecutive rows.  Every lane group keeps an
// independent online softmax; the groups and waves are merged at the end.
// Writes (m, l) to out_ml[h * ml_stride] and acc to out_acc[h * D + d].
template <class KV, int D, int G>
__device__ void split_state(const float *__restrict__ qg,
                            const typename KV::elem *__restrict__ kb,
                            const typename KV::elem *__restrict__ vb, int t0,
                            int t1, float sm_log2, float2 *__restrict__ out_ml,
                            float *__restrict__ out_acc) {
  constexpr int EPL = KV::EPL;
  constexpr int LPR = D / EPL;
  constexpr int RPI = 64 / LPR;
  constexpr int U = 4;
  constexpr int STEP = kWaves * RPI * U;

  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;
  const int c = lane % LPR;

  float qf[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      qf[h][i] = qg[h * D + c * EPL + i] * sm_log2;

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = neg_inf();
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[h][i] = 0.f;
  }

  for (int blk = t0; blk < t1; blk += STEP) {
    const int row0 = blk + wave * (RPI * U) + r;
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tok = row0 + u * RPI;
      valid[u] = tok < t1;
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (valid[u]) {
        kr[u] = *(const uint4 *)(kb + (size_t)tok * D + c * EPL);
        vr[u] = *(const uint4 *)(vb + (size_t)tok * D + c * EPL);
      }
    }
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
      KV::unpack(kr[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) a += qf[h][i] * kf[i];
        s[u][h] = group_sum<LPR>(a);
      }
    }
    float p[U][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = neg_inf();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!valid[u]) s[u][h] = neg_inf();
        mx = fmaxf(mx, s[u][h]);
      }
      const float mnew = fmaxf(m[h], mx);
      const float ref = exp_ref(mnew);
      const float sc = fast_exp2(m[h] - ref);
      m[h] = mnew;
      float ls = l[h] * sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u][h] = fast_exp2(s[u][h] - ref);
        ls += p[u][h];
      }
      l[h] = ls;
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[h][i] *= sc;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      KV::unpack(vr[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[h][i] += p[u][h] * vf[i];
    }
  }

  // Merge the RPI row groups of the wave (lanes with the same c).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float ref = exp_ref(mn);
      const float sa = fast_exp2(m[h] - ref);
      const float sb = fast_exp2(mo - ref);
      l[h] = l[h] * sa + lo * sb;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const float ao = __shfl_xor(acc[h][i], off);
        acc[h][i] = acc[h][i] * sa + ao * sb;
      }
      m[h] = mn;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) s_acc[wave][h][c * EPL + i] = acc[h][i];
      if (c == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  // Merge the waves.
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    const float ref = exp_ref(M);
    float ls = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sw = fast_exp2(s_m[w][h] - ref);
      ls += s_l[w][h] * sw;
      a += s_acc[w][h][d] * sw;
    }
    out_acc[h * D + d] = a;
    if (d == 0) out_ml[h] = make_float2(M, ls);
  }
}

// ------------------------------------------------------- merge of splits ---

// Merge the states of query head h of one batch entry: an optional prior
// state, then slots [slot0, slot0 + n) (stride Hq in ml, Hq * D in acc).
// All threads of the block take part.  On return res_acc[0..D) (shared),
// *res_m and *res_l (shared) hold the merged state.  The sum order is a
// fixed function of n, so equal inputs give equal bits.
template <int D>
__device__ void merge_head(const float2 *__restrict__ ml,
                           const float *__restrict__ acc, int slot0, int n,
                           int Hq, int h, bool has_prior, float2 prior_ml,
                           const float *__restrict__ prior_acc,
                           float *res_acc, float *res_m, float *res_l) {
  constexpr int CH = D / 4;            // float4 chunks of a row
  constexpr int NSG = kThreads / CH;   // slot groups
  __shared__ float s_red[kWaves];
  __shared__ float s_pl[NSG];
  __shared__ float4 s_pacc[NSG][CH];

  const int t = threadIdx.x;
  // global max
  float mx = has_prior ? prior_ml.x : neg_inf();
  for (int i = t; i < n; i += kThreads)
    mx = fmaxf(mx, ml[(size_t)(slot0 + i) * Hq + h].x);
  mx = wave_max(mx);
  if ((t & 63) == 0) s_red[t >> 6] = mx;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_red[w]);
  const float ref = exp_ref(M);

  const int c = t % CH, sg = t / CH;
  float ls = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = sg; i < n; i += NSG) {
    const size_t sl = (size_t)(slot0 + i) * Hq + h;
    const float2 mli = ml[sl];
    const float4 ai = ((const float4 *)(acc + sl * D))[c];
    const float w = fast_exp2(mli.x - ref);
    ls += mli.y * w;
    a.x += ai.x * w;
    a.y += ai.y * w;
    a.z += ai.z * w;
    a.w += ai.w * w;
  }
  s_pacc[sg][c] = a;
  if (c == 0) s_pl[sg] = ls;
  __syncthreads();
  if (t < D) {
    float tot = 0.f;
    if (has_prior) tot = prior_acc[t] * fast_exp2(prior_ml.x - ref);
#pragma unroll
    for (int g = 0; g < NSG; ++g) tot += ((const float *)&s_pacc[g][0])[t];
    res_acc[t] = tot;
  }
  if (t == 0) {
    float tl = has_prior ? prior_ml.y * fast_exp2(prior_ml.x - ref) : 0.f;
#pragma unroll
    for (int g = 0; g < NSG; ++g) tl += s_pl[g];
    *res_l = tl;
    *res_m = M;
  }
  __syncthreads();
}

__device__ __forceinline__ float normalise(float acc, float l) {
  return acc / l;
}

__device__ __forceinline__ float lse_nat(float m_log2, float l) {
  return (m_log2 + __builtin_log2f(l)) * kLn2;
}

// Block sum with a fixed order (wave shuffles, then waves in order).
__device__ float block_sum(float x, float *s_red) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  float tot = s_red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) tot += s_red[w];
  return tot;
}

__device__ __forceinline__ float ratio_of(float num, float den) {
  if (isnan(num) || isnan(den)) return __builtin_nanf("");
  if (den > 0.f) return sqrtf(num / den);
  return num == 0.f ? 0.f : __builtin_huge_valf();
}

// Returns true in every thread of the block for the last block to arrive at
// `cnt` out of `total`; that block also resets the counter to zero.  Release
// of this block's global writes before the arrival and acquire of the
// others' after it use device-scope fences.
__device__ bool arrive_last(unsigned *cnt, unsigned total) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = atomicAdd(cnt, 1u);
    s_last = (old == total - 1) ? 1 : 0;
    if (s_last) atomicExch(cnt, 0u);
  }
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

// ---------------------------------------------------------------- kernels ---

struct Item {
  int b, g, slot, t0, t1;
};

// Block index -> (entry, kv head, slot, token range).
__device__ __forceinline__ Item decode_item(const PlanArgs &pa,
                                            bool approx_set, int idx) {
  const int *pre = approx_set ? pa.itemA_pre : pa.itemM_pre;
  int b = 0;
  while (b + 1 < pa.B && pre[b + 1] <= idx) ++b;
  const int local = idx - pre[b];
  Item it;
  it.b = b;
  if (approx_set) {
    const int n = pa.nsink[b] + pa.nwin[b];
    it.g = local / n;
    const int a = local - it.g * n;
    it.slot = pa.slot_base[b] + a;
    if (a < pa.nsink[b]) {
      it.t0 = 0;
      it.t1 = pa.s_end[b];
    } else {
      const int w = a - pa.nsink[b];
      it.t0 = pa.w_begin[b] + w * pa.Tw;
      it.t1 = min(pa.L[b], it.t0 + pa.Tw);
    }
  } else {
    const int n = pa.nmid[b];
    it.g = local / n;
    const int mi = local - it.g * n;
    it.slot = pa.slot_base[b] + pa.nsink[b] + pa.nwin[b] + mi;
    it.t0 = pa.s_end[b] + mi * pa.T;
    it.t1 = min(pa.w_begin[b], it.t0 + pa.T);
  }
  return it;
}

template <class KV, int D, int G>
__global__ __launch_bounds__(kThreads) void partials_kernel(
    PlanArgs pa, bool approx_set, bool combine, const float *__restrict__ q,
    const typename KV::elem *__restrict__ k,
    const typename KV::elem *__restrict__ v, float sm_log2, WsPtrs w,
    float *__restrict__ o_approx, float *__restrict__ lse_approx) {
  const Item it = decode_item(pa, approx_set, blockIdx.x);
  const int Hq = pa.Hq;
  const size_t kv_off = ((size_t)it.b * pa.Hkv + it.g) * pa.L_cap * D;
  const int h0 = it.g * G;
  split_state<KV, D, G>(q + ((size_t)it.b * Hq + h0) * D, k + kv_off,
                        v + kv_off, it.t0, it.t1, sm_log2,
                        w.part_ml + (size_t)it.slot * Hq + h0,
                        w.part_acc + ((size_t)it.slot * Hq + h0) * D);
  if (!combine) return;

  // Last block of this (entry, kv head): merge its sink + window states.
  const int nA = pa.nsink[it.b] + pa.nwin[it.b];
  if (!arrive_last(w.counters + it.b * kMaxKvHeads + it.g, (unsigned)nA))
    return;
  __shared__ float r_acc[D];
  __shared__ float r_m, r_l;
  for (int hh = 0; hh < G; ++hh) {
    const int h = h0 + hh;
    merge_head<D>(w.part_ml, w.part_acc, pa.slot_base[it.b], nA, Hq, h, false,
                  make_float2(0.f, 0.f), nullptr, r_acc, &r_m, &r_l);
    const size_t bh = (size_t)it.b * Hq + h;
    for (int d = threadIdx.x; d < D; d += kThreads) {
      w.stA_acc[bh * D + d] = r_acc[d];
      o_approx[bh * D + d] = normalise(r_acc[d], r_l);
    }
    if (threadIdx.x == 0) {
      w.stA_ml[bh] = make_float2(r_m, r_l);
      if (lse_approx) lse_approx[bh] = lse_nat(r_m, r_l);
    }
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_verify_kernel(
    PlanArgs pa, WsPtrs w, const float *__restrict__ o_approx,
    float *__restrict__ o_exact, float *__restrict__ lse_exact,
    float *__restrict__ ratio, uint8_t *__restrict__ commit,
    float *__restrict__ o_committed, float lambda) {
  __shared__ float r_acc[D];
  __shared__ float r_m, r_l;
  __shared__ float s_red[kWaves];
  const int Hq = pa.Hq;
  const int b = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const size_t bh = (size_t)b * Hq + h;
  const int nA = pa.nsink[b] + pa.nwin[b];
  merge_head<D>(w.part_ml, w.part_acc, pa.slot_base[b] + nA, pa.nmid[b], Hq,
                h, true, w.stA_ml[bh], w.stA_acc + bh * D, r_acc, &r_m, &r_l);
  float num = 0.f, den = 0.f;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    const float e = normalise(r_acc[d], r_l);
    o_exact[bh * D + d] = e;
    const float diff = o_approx[bh * D + d] - e;
    num += diff * diff;
    den += e * e;
  }
  num = block_sum(num, s_red);
  den = block_sum(den, s_red);
  if (threadIdx.x == 0) {
    w.headnd[bh] = make_float2(num, den);
    if (lse_exact) lse_exact[bh] = lse_nat(r_m, r_l);
  }
  if (!arrive_last(w.counters + kApproxCounters + b, (unsigned)Hq)) return;

  // Last head of entry b: per-entry ratio over all heads, in head order.
  __shared__ int s_commit;
  if (threadIdx.x == 0) {
    float tn = 0.f, td = 0.f;
    for (int hh = 0; hh < Hq; ++hh) {
      const float2 nd = w.headnd[(size_t)b * Hq + hh];
      tn += nd.x;
      td += nd.y;
    }
    const float rt = ratio_of(tn, td);
    const int cm = rt <= lambda ? 1 : 0;
    ratio[b] = rt;
    commit[b] = (uint8_t)cm;
    s_commit = cm;
  }
  __syncthreads();
  if (o_committed) {
    const float *src = s_commit ? o_approx : o_exact;
    const size_t base = (size_t)b * Hq * D;
    for (int i = threadIdx.x; i < Hq * D; i += kThreads)
      o_committed[base + i] = src[base + i];
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void lse_combine_kernel(
    PlanArgs pa, WsPtrs w, float *__restrict__ o_exact,
    float *__restrict__ lse_exact) {
  __shared__ float r_acc[D];
  __shared__ float r_m, r_l;
  const int Hq = pa.Hq;
  const int b = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const size_t bh = (size_t)b * Hq + h;
  const int n = pa.nsink[b] + pa.nwin[b] + pa.nmid[b];
  merge_head<D>(w.part_ml, w.part_acc, pa.slot_base[b], n, Hq, h, false,
                make_float2(0.f, 0.f), nullptr, r_acc, &r_m, &r_l);
  for (int d = threadIdx.x; d < D; d += kThreads)
    o_exact[bh * D + d] = normalise(r_acc[d], r_l);
  if (threadIdx.x == 0 && lse_exact) lse_exact[bh] = lse_nat(r_m, r_l);
}

__global__ __launch_bounds__(kThreads) void verify_kernel(
    int n_per_entry, const float *__restrict__ o_approx,
    const float *__restrict__ o_exact, float *__restrict__ ratio,
    uint8_t *__restrict__ commit, float *__restrict__ o_committed,
    float lambda) {
  __shared__ float s_red[kWaves];
  __shared__ int s_commit;
  const int b = blockIdx.x;
  const size_t base = (size_t)b * n_per_entry;
  float num = 0.f, den = 0.f;
  for (int i = threadIdx.x; i < n_per_entry; i += kThreads) {
    const float e = o_exact[base + i];
    const float diff = o_approx[base + i] - e;
    num += diff * diff;
    den += e * e;
  }
  num = block_sum(num, s_red);
  den = block_sum(den, s_red);
  if (threadIdx.x == 0) {
    const float rt = ratio_of(num, den);
    ratio[b] = rt;
    s_commit = rt <= lambda ? 1 : 0;
    commit[b] = (uint8_t)s_commit;
  }
  __syncthreads();
  if (o_committed) {
    const float *src = s_commit ? o_approx : o_exact;
    for (int i = threadIdx.x; i < n_per_entry; i += kThreads)
      o_committed[base + i] = src[base + i];
  }
}

// ------------------------------------------------------------- dispatch ---

template <class KV, int D>
hipError_t partials_g(const PlanArgs &pa, bool approx_set, bool combine,
                      const float *q, const void *k, const void *v,
                      float sm_log2, const WsPtrs &w, float *o_approx,
                      float *lse_approx, hipStream_t s) {
  const int items = approx_set ? pa.itemA_pre[pa.B] : pa.itemM_pre[pa.B];
  if (items == 0) return hipSuccess;
  using E = typename KV::elem;
  const E *kk = (const E *)k;
  const E *vv = (const E *)v;
  dim3 grid(items), block(kThreads);
  switch (pa.G) {
    case 1:
      hipLaunchKernelGGL((partials_kernel<KV, D, 1>), grid, block, 0, s, pa,
                         approx_set, combine, q, kk, vv, sm_log2, w, o_approx,
                         lse_approx);
      break;
    case 2:
      hipLaunchKernelGGL((partials_kernel<KV, D, 2>), grid, block, 0, s, pa,
                         approx_set, combine, q, kk, vv, sm_log2, w, o_approx,
                         lse_approx);
      break;
    case 4:
      hipLaunchKernelGGL((partials_kernel<KV, D, 4>), grid, block, 0, s, pa,
                         approx_set, combine, q, kk, vv, sm_log2, w, o_approx,
                         lse_approx);
      break;
    case 8:
      hipLaunchKernelGGL((partials_kernel<KV, D, 8>), grid, block, 0, s, pa,
                         approx_set, combine, q, kk, vv, sm_log2, w, o_approx,
                         lse_approx);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

WsPtrs ws_ptrs(void *ws, const Workspace &wl) {
  char *base = (char *)ws;
  WsPtrs w;
  w.counters = (unsigned *)(base + wl.off_counters);
  w.part_ml = (float2 *)(base + wl.off_part_ml);
  w.part_acc = (float *)(base + wl.off_part_acc);
  w.stA_ml = (float2 *)(base + wl.off_stA_ml);
  w.stA_acc = (float *)(base + wl.off_stA_acc);
  w.headnd = (float2 *)(base + wl.off_headnd);
  return w;
}

hipError_t launch_partials(const PlanArgs &pa, int kv_dtype, bool approx_set,
                           bool combine, const float *q, const void *k,
                           const void *v, float sm_log2, const WsPtrs &w,
                           float *o_approx, float *lse_approx, hipStream_t s) {
  if (kv_dtype == ALSPEC_KV_BF16) {
    if (pa.D == 128)
      return partials_g<KvBf16, 128>(pa, approx_set, combine, q, k, v,
                                     sm_log2, w, o_approx, lse_approx, s);
    return partials_g<KvBf16, 64>(pa, approx_set, combine, q, k, v, sm_log2,
                                  w, o_approx, lse_approx, s);
  }
  if (pa.D == 128)
    return partials_g<KvF32, 128>(pa, approx_set, combine, q, k, v, sm_log2,
                                  w, o_approx, lse_approx, s);
  return partials_g<KvF32, 64>(pa, approx_set, combine, q, k, v, sm_log2, w,
                               o_approx, lse_approx, s);
}

hipError_t launch_merge_verify(const PlanArgs &pa, const WsPtrs &w,
                               const float *o_approx, float *o_exact,
                               float *lse_exact, float *ratio, uint8_t *commit,
                               float *o_committed, float lambda,
                               hipStream_t s) {
  dim3 grid(pa.B * pa.Hq), block(kThreads);
  if (pa.D == 128)
    hipLaunchKernelGGL(merge_verify_kernel<128>, grid, block, 0, s, pa, w,
                       o_approx, o_exact, lse_exact, ratio, commit,
                       o_committed, lambda);
  else
    hipLaunchKernelGGL(merge_verify_kernel<64>, grid, block, 0, s, pa, w,
                       o_approx, o_exact, lse_exact, ratio, commit,
                       o_committed, lambda);
  return hipGetLastError();
}

hipError_t launch_lse_combine(const PlanArgs &pa, const WsPtrs &w,
                              float *o_exact, float *lse_exact,
                              hipStream_t s) {
  dim3 grid(pa.B * pa.Hq), block(kThreads);
  if (pa.D == 128)
    hipLaunchKernelGGL(lse_combine_kernel<128>, grid, block, 0, s, pa, w,
                       o_exact, lse_exact);
  else
    hipLaunchKernelGGL(lse_combine_kernel<64>, grid, block, 0, s, pa, w,
                       o_exact, lse_exact);
  return hipGetLastError();
}

hipError_t launch_verify(const PlanArgs &pa, const float *o_approx,
                         const float *o_exact, float *ratio, uint8_t *commit,
                         float *o_committed, float lambda, hipStream_t s) {
  hipLaunchKernelGGL(verify_kernel, dim3(pa.B), dim3(kThreads), 0, s,
                     pa.Hq * pa.D, o_approx, o_exact, ratio, commit,
                     o_committed, lambda);
  return hipGetLastError();
}

}  // namespace alspec
