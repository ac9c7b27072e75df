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

#include <tuple>
#include <type_traits>

#include "alspec_kernels.h"

// Floating-point contraction only within one expression: a result's rounding
// then follows from the source alone, the same in every kernel that inlines
// a shared step.
#pragma clang fp contract(on)

namespace alspec {

namespace {

constexpr int kThreads = 256;
// Register sets for K/V tiles per wave in the MFMA split loop (the tiles in
// flight while one is computed are one fewer).
constexpr int kPrefetchSets = 2;
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

// Stores of split states.  With CO (a state handed to another block of the
// same launch) they are agent-scope relaxed atomic stores: coherent across
// the XCDs' L2 caches as they are written, so the hand-off needs no release
// fence (an L2 write-back of the whole XCD, which stalls every block on
// it); the writer waits for their completion before arriving.
template <bool CO>
__device__ __forceinline__ void put_f(float *p, float v) {
  if constexpr (CO)
    __hip_atomic_store((unsigned *)p, __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool CO>
__device__ __forceinline__ void put_f2(float2 *p, float2 v) {
  if constexpr (CO)
    __hip_atomic_store((unsigned long long *)p,
                       __builtin_bit_cast(unsigned long long, v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// Loads of values another block of the same launch stored with put_f /
// put_f2 (CO): agent-scope relaxed atomic loads, which read the coherent
// copy, so the reader needs no acquire fence (an invalidation of its whole
// L2, which disturbs every block streaming through it).
template <bool CO>
__device__ __forceinline__ float get_f(const float *p) {
  if constexpr (CO)
    return __uint_as_float(__hip_atomic_load(
        (const unsigned *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  else
    return *p;
}
template <bool CO>
__device__ __forceinline__ float2 get_f2(const float2 *p) {
  if constexpr (CO)
    return __builtin_bit_cast(
        float2, __hip_atomic_load((const unsigned long long *)p,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  else
    return *p;
}
template <bool CO>
__device__ __forceinline__ float4 get_f4(const float4 *p) {
  if constexpr (CO) {
    const float2 a = get_f2<true>((const float2 *)p);
    const float2 b = get_f2<true>((const float2 *)p + 1);
    return make_float4(a.x, a.y, b.x, b.y);
  } else {
    return *p;
  }
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

// Butterfly steps across 16- and 32-lane rows on the VALU (gfx950 row
// swaps): lane l gets op(x[l], x[l ^ 16]) or op(x[l], x[l ^ 32]).  Swapping
// a register with itself leaves rows (0, 0, 2, 2) in one result and
// (1, 1, 3, 3) in the other (for 32: low half twice, high half twice), so
// the two results hold each lane's pair.  Sum and max are commutative, so
// the bits equal those of the same step done with a shuffle.  All 64 lanes
// must be active.
__device__ __forceinline__ float xor16_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Lane H of each 16-lane row, broadcast to the whole row (DPP
// row_newbcast, gfx90a and later).
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(H >= 0 && H < 16, "row lane");
  return dpp_mov<0x150 + H>(x);
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
  if constexpr (N >= 32) x = xor16_sum(x);
  if constexpr (N >= 64) x = xor32_sum(x);
  return x;
}

// Max over aligned groups of N lanes (N a power of two <= 64), in every
// lane of the group.
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_mov<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_mov<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_mov<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_mov<0x140>(x));
  if constexpr (N >= 32) x = xor16_max(x);
  if constexpr (N >= 64) x = xor32_max(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) { return group_max<64>(x); }

// ------------------------------------------------- one split of one head ---

// Softmax state of the G query heads of one kv head over tokens [t0, t1).
// The block's 4 waves each own one contiguous quarter of every block-step of
// tokens; inside a wave, LPR lanes hold one K/V row (16 bytes each), so one
// load instruction covers RPI consecutive rows.  Every lane group keeps an
// independent online softmax; the groups and waves are merged at the end.
// Writes (m, l) to out_ml[h * ml_stride] and acc to out_acc[h * D + d].
template <class KV, int D, int G, bool CO = false>
__device__ __forceinline__ void split_state(const float *__restrict__ qg,
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
    put_f<CO>(&out_acc[h * D + d], a);
    if (d == 0) put_f2<CO>(&out_ml[h], make_float2(M, ls));
  }
}

// --------------------------------------- one split of one head, MFMA QK ---

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef float f32x8 __attribute__((ext_vector_type(8)));

// x = hi + mid + lo with each part a bf16: every step takes the exact fp32
// residual of the previous one, so the three parts carry x to within
// 2^-24 |x|, the precision of x itself.  The conversions are gfx950's
// hardware float32 -> bf16 conversion, which rounds to nearest even (a NaN
// stays a NaN), and bf16 -> float32 is exact.
__device__ __forceinline__ void split3(const float *x, bf16x8 &hi,
                                       bf16x8 &mid, bf16x8 &lo) {
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  hi = __builtin_convertvector(v, bf16x8);
  const f32x8 r1 = v - __builtin_convertvector(hi, f32x8);
  mid = __builtin_convertvector(r1, bf16x8);
  const f32x8 r2 = r1 - __builtin_convertvector(mid, f32x8);
  lo = __builtin_convertvector(r2, bf16x8);
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Shared and per-wave state of the MFMA split computation below, and its
// steps (q preparation, one tile, the split's end).
template <int G>
struct MfmaShared {
  float p[kWaves][4][4][G];  // [wave][c][j][head] (LDS form of P*V)
  float m[kWaves][G];
  float l[kWaves][G];
  union {
    struct {
      float acc[kWaves][G][128];
      bf16x8 q[3][4][64];    // split q (LDS form)
    };
    // per wave, one K tile on its way into the MFMA operand layout (short
    // splits with q in registers, which leave q unused; acc is written only
    // after every wave's last tile)
    uint4 kt[kWaves][256];
  };
};

template <int G>
struct MfmaWave {
  static constexpr int D = 128;
  static constexpr int TILE = 16;
  static constexpr int STEP = kWaves * TILE;
  static_assert(kWaves == 4, "one wave per 32-wide slice of q");
  int lane, wave, r, c;
  float m_lane;  // running max of head r (same in all 4 rows)
  float l_lane;  // this lane's share of head r's normaliser
  float acc[G][8];

  __device__ __forceinline__ void init() {
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    r = lane & 15;
    c = lane >> 4;
    reset();
  }
  __device__ __forceinline__ void reset() {
    m_lane = neg_inf();
    l_lane = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  }

  // K and V of this wave's tile at row tb.  Rows past `last` are clamped to
  // it (a row of the same range, so no address outside it is formed);
  // their logits are masked to -inf in tile(), so they carry no weight.
  // Unconditional loads keep the memory pipeline free of branches.
  // Every load instruction for V covers four whole rows, so V is loaded
  // nontemporal (read once): the middle pass went from 88.1 to 84.3 us at
  // 128K, the same bits.  Here a K instruction covers 16-byte pieces of 16
  // rows (the MFMA operand layout), the rest of each line coming from the
  // wave's next three instructions, and nontemporal K loads were far
  // slower; load_rows brings K in whole rows as well (nontemporal), for
  // transpose_k to rearrange.
  __device__ __forceinline__ void load(const uint16_t *__restrict__ kb,
                                       const uint16_t *__restrict__ vb, int tb,
                                       int last, u32x4 (&kk)[4],
                                       u32x4 (&vv)[4]) const {
    const int krow = min(tb + r, last);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kk[s] = *(const u32x4 *)(kb + (size_t)krow * D + 32 * c + 8 * s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vrow = min(tb + 4 * c + j, last);
      vv[j] = __builtin_nontemporal_load(
          (const u32x4 *)(vb + (size_t)vrow * D + 8 * r));
    }
  }

  // The same tile with K loaded as V is: instruction i brings whole rows
  // 4i .. 4i + 3 (lane l: row 4i + l / 16, bytes 16 (l % 16) ..), so both
  // are loaded nontemporal; transpose_k then rearranges K for the MFMA.
  __device__ __forceinline__ void load_rows(const uint16_t *__restrict__ kb,
                                            const uint16_t *__restrict__ vb,
                                            int tb, int last, u32x4 (&kk)[4],
                                            u32x4 (&vv)[4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int krow = min(tb + 4 * i + c, last);
      kk[i] = __builtin_nontemporal_load(
          (const u32x4 *)(kb + (size_t)krow * D + 8 * r));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vrow = min(tb + 4 * c + j, last);
      vv[j] = __builtin_nontemporal_load(
          (const u32x4 *)(vb + (size_t)vrow * D + 8 * r));
    }
  }

  // K of load_rows into the MFMA operand layout of load() through this
  // wave's LDS buffer: row t, 16-byte piece j is stored at 16 t + (j ^ t),
  // so that neither the stores (one row per 16 lanes) nor the loads (one
  // piece of 16 rows per 16 lanes) meet in a bank.  LDS operations of one
  // wave complete in order, so no wait separates the stores, the loads and
  // the next tile's stores.
  __device__ __forceinline__ void transpose_k(const u32x4 (&kr)[4],
                                              u32x4 (&kx)[4],
                                              uint4 *buf) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + c;
      buf[row * 16 + (r ^ row)] = __builtin_bit_cast(uint4, kr[i]);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kx[s] = __builtin_bit_cast(u32x4, buf[r * 16 + ((4 * c + s) ^ r)]);
    __builtin_amdgcn_wave_barrier();
  }

  // q of head r, D slice s = wave (each of the four waves takes one 32-wide
  // slice; columns r >= G are padding: a valid row is read, and zeroed in
  // prepare_q, so the loads need no branch and go out together).
  __device__ __forceinline__ void load_q(const float *__restrict__ qg,
                                         float4 (&qv)[2]) const {
    const float4 *qr =
        (const float4 *)(qg + (size_t)(r < G ? r : G - 1) * D + 32 * c);
    qv[0] = qr[2 * wave];
    qv[1] = qr[2 * wave + 1];
  }

  // This wave's slice of q, scaled and split, into the shared operands.
  // The caller synchronises the block.
  __device__ __forceinline__ void prepare_q(const float4 (&qv)[2],
                                            float sm_log2,
                                            MfmaShared<G> &sh) const {
    const float qs = r < G ? sm_log2 : 0.f;
    const float x[8] = {qv[0].x * qs, qv[0].y * qs, qv[0].z * qs,
                        qv[0].w * qs, qv[1].x * qs, qv[1].y * qs,
                        qv[1].z * qs, qv[1].w * qs};
    bf16x8 qh, qm, ql;
    split3(x, qh, qm, ql);
    sh.q[0][wave][lane] = qh;
    sh.q[1][wave][lane] = qm;
    sh.q[2][wave][lane] = ql;
  }

  // One 16-token tile of this wave (rows from tb, range end t1): logits on
  // MFMA, online softmax, P*V.
  __device__ __forceinline__ void tile(int tb, int t1, const u32x4 (&kr)[4],
                                       const u32x4 (&vr)[4],
                                       MfmaShared<G> &sh) {
    // logits: lane holds tokens 4c + j of the tile for head r
    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 kk = __builtin_bit_cast(bf16x8, kr[s]);
      a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, sh.q[0][s][lane], a4,
                                                   0, 0, 0);
      a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, sh.q[1][s][lane], a4,
                                                   0, 0, 0);
      a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, sh.q[2][s][lane], a4,
                                                   0, 0, 0);
    }
    float sv[4];
    float mx = neg_inf();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = (tb + 4 * c + j < t1) ? a4[j] : neg_inf();
      mx = fmaxf(mx, sv[j]);
    }
    mx = xor32_max(xor16_max(mx));
    const float mnew = fmaxf(m_lane, mx);
    const float ref = exp_ref(mnew);
    const float sc = fast_exp2(m_lane - ref);
    m_lane = mnew;
    float ls = l_lane * sc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pj = fast_exp2(sv[j] - ref);
      ls += pj;
      if (r < G) sh.p[wave][c][j][r] = pj;
    }
    l_lane = ls;
    // rescale: head h's factor is uniform, held by lane h
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float shh = readlane_f(sc, h);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] *= shh;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float vf[8];
      KvBf16::unpack(__builtin_bit_cast(uint4, vr[j]), vf);
      float pv[G];
#pragma unroll
      for (int h4 = 0; h4 < G; h4 += 4) {
        const float4 p4 = *(const float4 *)&sh.p[wave][c][j][h4];
        pv[h4] = p4.x;
        pv[h4 + 1] = p4.y;
        pv[h4 + 2] = p4.z;
        pv[h4 + 3] = p4.w;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] += pv[h] * vf[i];
    }
    __builtin_amdgcn_wave_barrier();
  }

  // This lane's 32 elements of q for head r (columns r >= G read a valid
  // row and are zeroed by split_q_regs): d = 32c .. 32c + 31, all four
  // slices of the MFMA B operand.
  __device__ __forceinline__ void load_q_full(const float *__restrict__ qg,
                                              float4 (&qv)[8]) const {
    const float4 *qr =
        (const float4 *)(qg + (size_t)(r < G ? r : G - 1) * D + 32 * c);
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = qr[i];
  }

  // The scaled q (sm_scale log2(e); padding columns r >= G zeroed) split
  // into its three bf16 parts, per slice, in registers: the B operands of
  // the logits' MFMAs.
  __device__ __forceinline__ void split_q_regs(const float4 (&qv)[8],
                                               float sm_log2,
                                               bf16x8 (&qp)[3][4]) const {
    const float qs = r < G ? sm_log2 : 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float4 a = qv[2 * s], b = qv[2 * s + 1];
      const float x[8] = {a.x * qs, a.y * qs, a.z * qs, a.w * qs,
                          b.x * qs, b.y * qs, b.z * qs, b.w * qs};
      split3(x, qp[0][s], qp[1][s], qp[2][s]);
    }
  }

  // One 16-token tile of this wave (rows from tb, range end t1): logits on
  // MFMA from the split q in registers, online softmax, P*V on the VALU
  // with the probabilities passed between lanes by row broadcasts: no LDS
  // round trip inside the tile.
  __device__ __forceinline__ void tile_regs(int tb, int t1,
                                            const u32x4 (&kr)[4],
                                            const u32x4 (&vr)[4],
                                            const bf16x8 (&qp)[3][4]) {
    f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 kk = __builtin_bit_cast(bf16x8, kr[s]);
      a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qp[0][s], a4, 0, 0, 0);
      a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qp[1][s], a4, 0, 0, 0);
      a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qp[2][s], a4, 0, 0, 0);
    }
    float sv[4];
    float mx = neg_inf();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = (tb + 4 * c + j < t1) ? a4[j] : neg_inf();
      mx = fmaxf(mx, sv[j]);
    }
    mx = xor32_max(xor16_max(mx));
    const float mnew = fmaxf(m_lane, mx);
    const float ref = exp_ref(mnew);
    const float sc = fast_exp2(m_lane - ref);
    m_lane = mnew;
    float ls = l_lane * sc;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = fast_exp2(sv[j] - ref);
      ls += p[j];
    }
    l_lane = ls;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float shh = readlane_f(sc, h);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] *= shh;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float vf[8];
      KvBf16::unpack(__builtin_bit_cast(uint4, vr[j]), vf);
      // row c's lane h holds head h's probability of token 4c + j
      float pv[G];
      pv[0] = row_bcast<0>(p[j]);
      if constexpr (G > 1) pv[1] = row_bcast<1>(p[j]);
      if constexpr (G > 2) pv[2] = row_bcast<2>(p[j]);
      if constexpr (G > 3) pv[3] = row_bcast<3>(p[j]);
      if constexpr (G > 4) {
        pv[4] = row_bcast<4>(p[j]);
        pv[5] = row_bcast<5>(p[j]);
        pv[6] = row_bcast<6>(p[j]);
        pv[7] = row_bcast<7>(p[j]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] += pv[h] * vf[i];
    }
  }

  // The split's state: the four row groups summed (same running max in
  // every row), then the waves merged through LDS and written out.  All
  // threads of the block take part; on return the shared state arrays may
  // be reused.
  template <bool CO>
  __device__ __forceinline__ void finish(MfmaShared<G> &sh,
                                         float2 *__restrict__ out_ml,
                                         float *__restrict__ out_acc) {
    l_lane = xor32_sum(xor16_sum(l_lane));
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = xor32_sum(xor16_sum(acc[h][i]));
    if (c == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) sh.acc[wave][h][8 * r + i] = acc[h][i];
      if (r < G) {
        sh.m[wave][r] = m_lane;
        sh.l[wave][r] = l_lane;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
      const int h = idx / D, d = idx % D;
      float M = neg_inf();
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh.m[w][h]);
      const float ref = exp_ref(M);
      float ls = 0.f, a = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sw = fast_exp2(sh.m[w][h] - ref);
        ls += sh.l[w][h] * sw;
        a += sh.acc[w][h][d] * sw;
      }
      put_f<CO>(&out_acc[h * D + d], a);
      if (d == 0) put_f2<CO>(&out_ml[h], make_float2(M, ls));
    }
  }
};

// Softmax state of the G (4 or 8) query heads of one kv head over tokens
// [t0, t1), bf16 K/V with D = 128.  The logit block S^T = K_tile Q^T of a
// 16-token tile is one 16x16 output of v_mfma_f32_16x16x32_bf16 per
// 32-wide slice of D (K rows are the A operand, the query heads the B
// operand, padded to 16 columns, in registers for G = 4 and in LDS for
// G = 8).  q is split into three bf16 parts whose products accumulate in
// fp32, so the logits keep fp32 accuracy.  In the A operand lane l
// (r = l % 16, c = l / 16) holds bytes [64c, 64c + 64) of tile row r
// (loaded so for G = 8, moved there through LDS for G = 4), and both
// operands map slice s, element j to d = 32c + 8s + j.  The output gives lane l the logits of tokens
// 4c + j (j = 0..3) for head r.  P*V runs on the VALU: lane l owns
// d = 8r..8r+7 of V rows 4c + j and takes the G probabilities of its rows
// from the lanes of its row (row broadcasts for G = 4, LDS for G = 8).
// Wave w takes tile w of every 64-token step of the range and
// keeps NS register sets for K and V in turn: the loads of the next NS - 1
// tiles are in flight while one is computed, and no set is copied into
// another, so a wait covers only the loads of the tile about to be used.
// Each wave keeps its own online softmax; the waves are merged at the end.
template <int G, int NS, bool CO = false>
__device__ __forceinline__ void split_state_mfma(const float *__restrict__ qg,
                                 const uint16_t *__restrict__ kb,
                                 const uint16_t *__restrict__ vb, int t0,
                                 int t1, float sm_log2,
                                 float2 *__restrict__ out_ml,
                                 float *__restrict__ out_acc) {
  static_assert(G == 4 || G == 8, "MFMA path serves groups of 4 or 8");
  static_assert(NS >= 2, "at least one tile in flight");
  using W = MfmaWave<G>;
  constexpr int TILE = W::TILE, STEP = W::STEP;
  __shared__ MfmaShared<G> sh;
  W wv;
  wv.init();
  const int last = t1 - 1;
  const int ta0 = t0 + wv.wave * TILE;  // this wave's tile i is at ta0 + i*STEP

  // q is requested first and the first NS - 1 tiles after it, so the wait
  // for q leaves the tiles in flight.  For G = 4 each wave keeps all of q's
  // three bf16 parts in registers and passes the probabilities from lane to
  // lane by row broadcasts (tile_regs), so no tile waits on LDS (0.7 %
  // faster at the 8B shape).  For G = 8 that form needs 188 VGPRs and ran
  // 12 % slower at the 70B shape, so there each wave splits one 32-wide
  // slice of q into LDS and the probabilities go through LDS (tile); both
  // forms give the same bits.  The register form also loads K in whole
  // rows, nontemporal, and transposes it through LDS (the middle pass at
  // 128K: 84.1 against 87.5 us; 170 VGPRs, occupancy 2, against 152 and
  // 3).  Rows past the range are clamped to its last row.
  constexpr bool kRegs = G == 4;
  u32x4 kr[NS][4], vr[NS][4];
  float4 qv[kRegs ? 8 : 2];
  if constexpr (kRegs)
    wv.load_q_full(qg, qv);
  else
    wv.load_q(qg, qv);
  auto load = [&](int ta, u32x4 (&k)[4], u32x4 (&v)[4]) {
    if constexpr (kRegs)
      wv.load_rows(kb, vb, ta, last, k, v);
    else
      wv.load(kb, vb, ta, last, k, v);
  };
  if (t0 < t1) {
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) load(ta0 + i * STEP, kr[i], vr[i]);
  }
  bf16x8 qp[3][4];
  if constexpr (kRegs) {
    wv.split_q_regs(qv, sm_log2, qp);
  } else {
    wv.prepare_q(qv, sm_log2, sh);
    __syncthreads();
  }
  auto tile = [&](int ta, const u32x4 (&k)[4], const u32x4 (&v)[4]) {
    if constexpr (kRegs) {
      u32x4 kx[4];
      wv.transpose_k(k, kx, sh.kt[wv.wave]);
      wv.tile_regs(ta, t1, kx, v, qp);
    } else {
      wv.tile(ta, t1, k, v, sh);
    }
  };

  if constexpr (NS == 2) {
    // spelled out: the compiler keeps this form in fewer VGPRs
    for (int blk = t0; blk < t1; blk += 2 * STEP) {
      const int ta = blk + wv.wave * TILE;
      load(ta + STEP, kr[1], vr[1]);
      tile(ta, kr[0], vr[0]);
      if (blk + STEP >= t1) break;
      load(ta + 2 * STEP, kr[0], vr[0]);
      tile(ta + STEP, kr[1], vr[1]);
    }
  } else {
    for (int blk = t0; blk < t1; blk += NS * STEP) {
      const int ta = blk + wv.wave * TILE;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        load(ta + (i + NS - 1) * STEP, kr[(i + NS - 1) % NS],
             vr[(i + NS - 1) % NS]);
        tile(ta + i * STEP, kr[i], vr[i]);
        if (i + 1 < NS && blk + (i + 1) * STEP >= t1) break;
      }
    }
  }
  if constexpr (kRegs) __syncthreads();  // K buffers share LDS with acc
  wv.template finish<CO>(sh, out_ml, out_acc);
}

// split_state_mfma for a range of at most NT 64-token steps (the sink and
// window splits): each wave requests q and all its NT tiles at once, so the
// split costs one memory round trip.  The same tiles, arithmetic and order
// as split_state_mfma, so the same bits.  The range must be nonempty
// (every split of the plan is).
template <int G, int NT, bool CO>
__device__ __forceinline__ void split_state_mfma_short(const float *__restrict__ qg,
                                       const uint16_t *__restrict__ kb,
                                       const uint16_t *__restrict__ vb,
                                       int t0, int t1, float sm_log2,
                                       float2 *__restrict__ out_ml,
                                       float *__restrict__ out_acc) {
  static_assert(G == 4 || G == 8, "MFMA path serves groups of 4 or 8");
  using W = MfmaWave<G>;
  constexpr int TILE = W::TILE, STEP = W::STEP;
  __shared__ MfmaShared<G> sh;
  W wv;
  wv.init();
  const int last = t1 - 1;
  const int ta0 = t0 + wv.wave * TILE;
  float4 qv[8];
  wv.load_q_full(qg, qv);
  u32x4 kr[NT][4], vr[NT][4];
#pragma unroll
  for (int i = 0; i < NT; ++i)
    wv.load_rows(kb, vb, ta0 + i * STEP, last, kr[i], vr[i]);
  bf16x8 qp[3][4];
  wv.split_q_regs(qv, sm_log2, qp);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    u32x4 kx[4];
    wv.transpose_k(kr[i], kx, sh.kt[wv.wave]);
    wv.tile_regs(ta0 + i * STEP, t1, kx, vr[i], qp);
  }
  __syncthreads();  // the K buffers share LDS with finish's acc
  wv.template finish<CO>(sh, out_ml, out_acc);
}

// ------------------------------------------------------- merge of splits ---

// Merge the states of NH consecutive query heads h0.. of one batch entry:
// an optional prior state per head, then slots [slot0, slot0 + n) (stride
// Hq in ml, Hq * D in acc).  The block's threads split into NH heads x NSG
// slot groups x D/4 float4 chunks; slot i goes to group i % NSG, each group
// sums its slots in increasing order, and the groups are then added in
// order after the prior, so the bits depend only on (n, NH, D).  prior_ml
// and prior_acc must be valid addresses even when has_prior is false.  Up to
// NSG * R slots are merged in one memory round: every thread issues all
// its loads (which also cover every slot's max) before using any.  Larger
// n takes a max pass and then rounds of NSG * R slots.  On return
// res_acc[NH][D], res_m[NH], res_l[NH] (shared) hold the merged states.
template <int D, int NH, int R, bool CO = false>
__device__ void merge_heads(const float2 *__restrict__ ml,
                            const float *__restrict__ acc, int slot0, int n,
                            int Hq, int h0, bool has_prior,
                            const float2 *__restrict__ prior_ml,
                            const float *__restrict__ prior_acc,
                            float *res_acc, float *res_m, float *res_l) {
  constexpr int CH = D / 4;
  constexpr int TPH = kThreads / NH;  // threads per head
  constexpr int NSG = TPH / CH;       // slot groups per head
  static_assert(NSG >= 1 && NSG * CH * NH == kThreads, "thread split");
  constexpr int WPH = TPH >= 64 ? TPH / 64 : 1;  // waves per head
  __shared__ float s_mx[NH][WPH];
  __shared__ float4 s_pacc[NH][NSG][CH];
  __shared__ float s_pl[NH][NSG];

  const int t = threadIdx.x;
  const int hh = t / TPH, u = t % TPH;
  const int h = h0 + hh;
  const int c = u % CH, sg = u / CH;
  const bool one_round = n <= NSG * R;

  // All loads of the round are issued before any is used: indices past n
  // are clamped to a valid slot and their terms dropped, and the prior is
  // read whether or not it is used, so no load sits behind a branch.
  float2 mv[R];
  float4 av[R];
  const float2 pml_raw = get_f2<CO>(&prior_ml[has_prior ? hh : 0]);
  const float pacc_raw = get_f<CO>(&prior_acc[has_prior && t < NH * D ? t : 0]);
  const float2 pml = has_prior ? pml_raw : make_float2(neg_inf(), 0.f);
  const float pacc = has_prior ? pacc_raw : 0.f;
  float mx = pml.x;
  if (one_round && n > 0) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = min(sg + k * NSG, n - 1);
      const size_t sl = (size_t)(slot0 + i) * Hq + h;
      mv[k] = get_f2<CO>(&ml[sl]);
      av[k] = get_f4<CO>((const float4 *)(acc + sl * D) + c);
    }
#pragma unroll
    for (int k = 0; k < R; ++k)
      if (sg + k * NSG < n) mx = fmaxf(mx, mv[k].x);
  } else if (!one_round) {
    for (int i = u; i < n; i += TPH)
      mx = fmaxf(mx, get_f2<CO>(&ml[(size_t)(slot0 + i) * Hq + h]).x);
  }
  mx = group_max<(TPH < 64 ? TPH : 64)>(mx);
  if (TPH >= 64) {
    if ((u & 63) == 0) s_mx[hh][u >> 6] = mx;
  } else if (u == 0) {
    s_mx[hh][0] = mx;
  }
  __syncthreads();
  float M = s_mx[hh][0];
#pragma unroll
  for (int w = 1; w < WPH; ++w) M = fmaxf(M, s_mx[hh][w]);
  const float ref = exp_ref(M);

  float ls = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int base = sg; base < n; base += NSG * R) {
    if (!one_round) {
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int i = base + k * NSG;
        if (i < n) {
          const size_t sl = (size_t)(slot0 + i) * Hq + h;
          mv[k] = get_f2<CO>(&ml[sl]);
          av[k] = get_f4<CO>((const float4 *)(acc + sl * D) + c);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (base + k * NSG < n) {
        const float w = fast_exp2(mv[k].x - ref);
        ls += mv[k].y * w;
        a.x += av[k].x * w;
        a.y += av[k].y * w;
        a.z += av[k].z * w;
        a.w += av[k].w * w;
      }
    }
  }
  s_pacc[hh][sg][c] = a;
  if (c == 0) s_pl[hh][sg] = ls;
  __syncthreads();
  // thread t < NH * D owns (head t / D, element t % D) of the result
  for (int idx = t; idx < NH * D; idx += kThreads) {
    const int h2 = idx / D, d = idx % D;
    float Mh = s_mx[h2][0];
#pragma unroll
    for (int w = 1; w < WPH; ++w) Mh = fmaxf(Mh, s_mx[h2][w]);
    float tot = 0.f;
    if (has_prior) {
      const float pa = (idx == t) ? pacc : get_f<CO>(&prior_acc[idx]);
      tot = pa * fast_exp2(get_f2<CO>(&prior_ml[h2]).x - exp_ref(Mh));
    }
#pragma unroll
    for (int g = 0; g < NSG; ++g) tot += ((const float *)&s_pacc[h2][g][0])[d];
    res_acc[idx] = tot;
  }
  if (t < NH) {
    float Mh = s_mx[t][0];
#pragma unroll
    for (int w = 1; w < WPH; ++w) Mh = fmaxf(Mh, s_mx[t][w]);
    float tl = 0.f;
    if (has_prior) {
      const float2 pm = get_f2<CO>(&prior_ml[t]);
      tl = pm.y * fast_exp2(pm.x - exp_ref(Mh));
    }
#pragma unroll
    for (int g = 0; g < NSG; ++g) tl += s_pl[t][g];
    res_l[t] = tl;
    res_m[t] = Mh;
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

// Arrival counters (each on its own line): exact-merge heads of entry b,
// and sink/window splits of (entry b, kv head g).
__device__ __forceinline__ unsigned *user_counter(const WsPtrs &w, int b) {
  return w.counters + kUserCounters + b * kCounterStride;
}
__device__ __forceinline__ unsigned *approx_counter(const WsPtrs &w, int b,
                                                    int Hkv, int g) {
  return w.counters + kApproxCounters + (b * Hkv + g) * kCounterStride;
}

// Returns true in every thread of the block for the last block to arrive at
// `cnt` out of `total`; that block also resets the counter to zero.  The
// block barrier orders all of this block's global writes before thread 0's
// device-scope release fence and arrival; only the last block's thread 0
// then takes the device-scope acquire fence (which invalidates the L2 lines
// other blocks may have written) before the barrier that lets its threads
// read.  Keeping the acquire to one block per merge spares concurrently
// streaming kernels from repeated cache invalidation.
__device__ bool arrive_last(unsigned *cnt, unsigned total) {
  __shared__ int s_last;
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == total - 1) ? 1 : 0;
    if (last) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

// arrive_last for blocks that stored their state with agent-scope atomic
// stores (CO): each thread waits until its own stores have completed (been
// acknowledged at the agent-scope coherence point: s_waitcnt with every
// counter at zero; the workgroup-scope release before it keeps the stores
// ahead of it), then thread 0 arrives.  No cache write-back is needed, as
// nothing of the state sits in a non-coherent cache.  The last block's
// thread 0 takes the device-scope acquire (invalidating stale copies this
// CU and its L2 may hold) before the barrier that lets the block read the
// states with ordinary loads.
template <bool ACQ = true>
__device__ bool arrive_last_coherent(unsigned *cnt, unsigned total) {
  __shared__ int s_last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == total - 1) ? 1 : 0;
    if (last) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ACQ) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
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

// Slots merged per thread per memory round in the merges of the sink and
// window states.  A single call's automatic plan gives one entry with 8 kv
// heads (the Llama-3 shapes) 16 window splits plus one sink split, and the
// merge's two slot groups per head take up to 18 in one round (at 8, the
// 17th slot would add a separate max pass and a second round, each a
// dependent round trip).
constexpr int kMergeRoundA = 9;

// ... and in the exact merges (many middle splits).
constexpr int kMergeRoundM = 8;

template <class KV, int D, int G, bool CO = false, bool SHORT = false>
__device__ __forceinline__ void split_any(const float *qg,
                                          const typename KV::elem *kb,
                                          const typename KV::elem *vb, int t0,
                                          int t1, float sm_log2,
                                          float2 *out_ml, float *out_acc) {
  if constexpr (std::is_same<KV, KvBf16>::value && D == 128 &&
                (G == 4 || G == 8)) {
    constexpr int STEP = MfmaWave<G>::STEP;
    if (SHORT && t1 - t0 <= STEP)
      split_state_mfma_short<G, 1, CO>(qg, kb, vb, t0, t1, sm_log2, out_ml,
                                       out_acc);
    else if (SHORT && t1 - t0 <= 2 * STEP)
      split_state_mfma_short<G, 2, CO>(qg, kb, vb, t0, t1, sm_log2, out_ml,
                                       out_acc);
    else
      split_state_mfma<G, kPrefetchSets, CO>(qg, kb, vb, t0, t1, sm_log2,
                                             out_ml, out_acc);
  }
  else
    split_state<KV, D, G, CO>(qg, kb, vb, t0, t1, sm_log2, out_ml, out_acc);
}

// Per-head sums of the relative L2 test over a block's G x D outputs, kept
// in fixed order: each wave sums one head's slice of a pass, then the
// waves of a head are added in order.
template <int D, int G, bool CO = false>
__device__ void group_num_den(const float *e, const float *a, float *num,
                              float *den) {
  constexpr int WPH = D / 64;          // waves per head in one pass
  constexpr int HPP = kWaves / WPH;    // heads per pass
  constexpr int PASSES = (G + HPP - 1) / HPP;
  __shared__ float s_n[PASSES][kWaves], s_d[PASSES][kWaves];
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int idx = p * kThreads + threadIdx.x;
    float n = 0.f, d2 = 0.f;
    if (idx < G * D) {
      const float diff = get_f<CO>(&a[idx]) - e[idx];
      n = diff * diff;
      d2 = e[idx] * e[idx];
    }
    for (int off = 32; off >= 1; off >>= 1) {
      n += __shfl_xor(n, off);
      d2 += __shfl_xor(d2, off);
    }
    if ((threadIdx.x & 63) == 0) {
      s_n[p][wave] = n;
      s_d[p][wave] = d2;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int hh = threadIdx.x, p = hh / HPP, w0 = (hh % HPP) * WPH;
    float n = s_n[p][w0], d2 = s_d[p][w0];
#pragma unroll
    for (int w = 1; w < WPH; ++w) {
      n += s_n[p][w0 + w];
      d2 += s_d[p][w0 + w];
    }
    num[hh] = n;
    den[hh] = d2;
  }
}

// Exact output of NH consecutive query heads h0.. of entry b: the stored
// sink+window state merged with the middle slots, normalised into o_exact
// (and lse_exact); each head's (num, den) of the verify goes to the
// workspace.
template <int D, int NH, bool VERIFY = true, bool CO = false>
__device__ void exact_heads(const PlanArgs &pa, const WsPtrs &w, int b,
                            int h0, const float *__restrict__ o_approx,
                            float *__restrict__ o_exact,
                            float *__restrict__ lse_exact) {
  __shared__ float r_acc[NH * D];
  __shared__ float r_m[NH], r_l[NH];
  __shared__ float s_num[NH], s_den[NH];
  const int Hq = pa.Hq;
  const size_t bh0 = (size_t)b * Hq + h0;
  const int nA = pa.nsink[b] + pa.nwin[b];
  merge_heads<D, NH, kMergeRoundM, CO>(w.part_ml, w.part_acc,
                                       pa.slot_base[b] + nA, pa.nmid[b], Hq,
                                       h0, true, w.stA_ml + bh0,
                                       w.stA_acc + bh0 * D, r_acc, r_m, r_l);
  for (int idx = threadIdx.x; idx < NH * D; idx += kThreads) {
    const float e = normalise(r_acc[idx], r_l[idx / D]);
    r_acc[idx] = e;
    put_f<CO>(&o_exact[bh0 * D + idx], e);
  }
  __syncthreads();
  if constexpr (VERIFY) {
    group_num_den<D, NH, CO>(r_acc, o_approx + bh0 * D, s_num, s_den);
    __syncthreads();
  }
  if (threadIdx.x < NH) {
    const int hh = threadIdx.x;
    if constexpr (VERIFY)
      put_f2<CO>(&w.headnd[bh0 + hh], make_float2(s_num[hh], s_den[hh]));
    if (lse_exact) lse_exact[bh0 + hh] = lse_nat(r_m[hh], r_l[hh]);
  }
}

// Per-entry verdict once every head of entry b has stored its (num, den): ratio over all heads (summed in head order), commit flag,
// committed output.
template <int D, bool CO = false>
__device__ void finalize_entry(const PlanArgs &pa, const WsPtrs &w, int b,
                               const float *__restrict__ o_approx,
                               const float *__restrict__ o_exact,
                               float *__restrict__ ratio,
                               uint8_t *__restrict__ commit,
                               float *__restrict__ o_committed, float lambda) {
  __shared__ float s_red[kWaves];
  __shared__ int s_commit;
  const int Hq = pa.Hq;
  float n = 0.f, d2 = 0.f;
  for (int h = threadIdx.x; h < Hq; h += kThreads) {
    const float2 nd = get_f2<CO>(&w.headnd[(size_t)b * Hq + h]);
    n += nd.x;
    d2 += nd.y;
  }
  n = block_sum(n, s_red);
  d2 = block_sum(d2, s_red);
  if (threadIdx.x == 0) {
    const float rt = ratio_of(n, d2);
    const int cm = rt <= lambda ? 1 : 0;
    ratio[b] = rt;
    commit[b] = (uint8_t)cm;
    s_commit = cm;
  }
  __syncthreads();
  if (o_committed) {
    // float4 copy, four per thread per round, loads issued before stores
    const float4 *src = (const float4 *)((s_commit ? o_approx : o_exact) +
                                         (size_t)b * Hq * D);
    float4 *dst = (float4 *)(o_committed + (size_t)b * Hq * D);
    const int n4 = Hq * D / 4;
    for (int base = threadIdx.x; base < n4; base += 4 * kThreads) {
      float4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[k] = get_f4<CO>(&src[min(base + k * kThreads, n4 - 1)]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (base + k * kThreads < n4) dst[base + k * kThreads] = v[k];
    }
  }
}

// One block per work item (sink and window items when APPROX, else middle
// items): the split state of the item's G query heads over its token range.
// The long middle splits prefetch the next tile; the short sink and window
// splits keep a footprint that fits beside a running middle pass.
template <class KV, int D, int G, bool APPROX>
__global__ __launch_bounds__(kThreads) void partials_kernel(
    PlanArgs pa, const float *__restrict__ q,
    const typename KV::elem *__restrict__ k,
    const typename KV::elem *__restrict__ v, float sm_log2, WsPtrs w) {
  const Item it = decode_item(pa, APPROX, blockIdx.x);
  const int Hq = pa.Hq;
  const size_t kv_off = ((size_t)it.b * pa.Hkv + it.g) * pa.L_cap * D;
  const int h0 = it.g * G;
  split_any<KV, D, G>(q + ((size_t)it.b * Hq + h0) * D, k + kv_off,
                            v + kv_off, it.t0, it.t1, sm_log2,
                            w.part_ml + (size_t)it.slot * Hq + h0,
                            w.part_acc + ((size_t)it.slot * Hq + h0) * D);
}

// Every split of the plan (sink, window and middle) in one launch: the
// first blocks take the long middle splits, one per CU, and the short sink
// and window splits fill the slots left (dispatched first, the short ones
// could take the slots of middle splits, which would then start late or
// share a CU: 512 against 376 µs per layer at the 70B stack's shape).
template <class KV, int D, int G>
__global__ __launch_bounds__(kThreads) void partials_all_kernel(
    PlanArgs pa, const float *__restrict__ q,
    const typename KV::elem *__restrict__ k,
    const typename KV::elem *__restrict__ v, float sm_log2, WsPtrs w) {
  const int nM = pa.itemM_pre[pa.B];
  const int idx = blockIdx.x;
  const Item it =
      idx < nM ? decode_item(pa, false, idx) : decode_item(pa, true, idx - nM);
  const int Hq = pa.Hq;
  const size_t kv_off = ((size_t)it.b * pa.Hkv + it.g) * pa.L_cap * D;
  const int h0 = it.g * G;
  split_any<KV, D, G>(q + ((size_t)it.b * Hq + h0) * D, k + kv_off,
                            v + kv_off, it.t0, it.t1, sm_log2,
                            w.part_ml + (size_t)it.slot * Hq + h0,
                            w.part_acc + ((size_t)it.slot * Hq + h0) * D);
}

// Merge of the sink and window states of entry b, kv head g into the
// reusable merged state and (each if non-null) o_approx / lse_approx.  The
// exact combines start from that state, so with an empty middle they give
// the approximation's bits.
template <int D, int G, bool CO = false>
__device__ void approx_merge(const PlanArgs &pa, const WsPtrs &w,
                             const Outs &o, int b, int g) {
  __shared__ float r_acc[G * D];
  __shared__ float r_m[G], r_l[G];
  const int Hq = pa.Hq;
  const int h0 = g * G;
  const int nA = pa.nsink[b] + pa.nwin[b];
  const size_t bh0 = (size_t)b * Hq + h0;
  // no prior state; the stored-state slots only serve as valid addresses
  merge_heads<D, G, kMergeRoundA, CO>(w.part_ml, w.part_acc,
                                      pa.slot_base[b], nA, Hq, h0, false,
                                      w.stA_ml + bh0, w.stA_acc + bh0 * D,
                                      r_acc, r_m, r_l);
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int hh = idx / D;
    put_f<CO>(&w.stA_acc[bh0 * D + idx], r_acc[idx]);
    if (o.o_approx)
      put_f<CO>(&o.o_approx[bh0 * D + idx], normalise(r_acc[idx], r_l[hh]));
  }
  if (threadIdx.x < G) {
    const int hh = threadIdx.x;
    put_f2<CO>(&w.stA_ml[bh0 + hh], make_float2(r_m[hh], r_l[hh]));
    if (o.lse_approx) put_f<CO>(&o.lse_approx[bh0 + hh], lse_nat(r_m[hh], r_l[hh]));
  }
}

// The whole approximation in one launch: each block computes one sink or
// window split, and the last block of an (entry, kv head) to finish merges
// the group's states.  Saves the second launch on the approximation's
// latency path.  The states pass between blocks through agent-scope
// atomic stores, so no block writes back its cache.  Splits of up to two
// 64-token steps take the short form (all tiles requested with q, no LDS
// round trip inside a tile); its extra registers are free here, where one
// block runs per CU.
template <class KV, int D, int G>
__device__ __forceinline__ void approx_fused_body(
    const PlanArgs &pa, const Item &it, const float *__restrict__ q,
    const typename KV::elem *__restrict__ k,
    const typename KV::elem *__restrict__ v, int L_cap, int Hq,
    float sm_log2, const WsPtrs &w, const Outs &o) {
  const size_t kv_off = ((size_t)it.b * pa.Hkv + it.g) * L_cap * D;
  const int h0 = it.g * G;
  split_any<KV, D, G, true, true>(q + ((size_t)it.b * Hq + h0) * D,
                                  k + kv_off, v + kv_off, it.t0, it.t1,
                                  sm_log2, w.part_ml + (size_t)it.slot * Hq + h0,
                                  w.part_acc + ((size_t)it.slot * Hq + h0) * D);
  const unsigned n = (unsigned)(pa.nsink[it.b] + pa.nwin[it.b]);
  if (!arrive_last_coherent(approx_counter(w, it.b, pa.Hkv, it.g), n))
    return;
  approx_merge<D, G>(pa, w, o, it.b, it.g);
}

template <class KV, int D, int G>
__global__ __launch_bounds__(kThreads) void approx_fused_kernel(
    PlanArgs pa, const float *__restrict__ q,
    const typename KV::elem *__restrict__ k,
    const typename KV::elem *__restrict__ v, float sm_log2, WsPtrs w,
    Outs o) {
  const Item it = decode_item(pa, true, blockIdx.x);
  approx_fused_body<KV, D, G>(pa, it, q, k, v, pa.L_cap, pa.Hq, sm_log2, w,
                              o);
}

// The same for a launch over batch entry 0 alone.  The leading scalar
// arguments are all that the first memory requests and the addresses
// computed before them depend on (the item's kv head and token range, the
// cache stride, the head count of the state slots and the q, K and V
// bases: 14 dwords, as many as the hardware preloads); the library is built
// to preload the leading kernel arguments into scalar registers at wave
// launch, so those requests leave without waiting for a kernel-argument
// fetch (with the head count read from the plan they waited for one, which
// measured within noise of this form).  The plan has a sink split exactly
// when the sink is nonempty.
template <class KV, int D, int G>
__global__ __launch_bounds__(kThreads) void approx_fused_one_kernel(
    int n_split, int s_end, int w_begin, int Tw, int L, int L_cap, int Hq,
    const float *__restrict__ q, const typename KV::elem *__restrict__ k,
    const typename KV::elem *__restrict__ v, PlanArgs pa, float sm_log2,
    WsPtrs w, Outs o) {
  Item it;
  it.b = 0;
  it.g = blockIdx.x / n_split;
  const int a = blockIdx.x - it.g * n_split;
  it.slot = a;  // entry 0's slots start at 0
  const int nsink = s_end > 0 ? 1 : 0;
  if (a < nsink) {
    it.t0 = 0;
    it.t1 = s_end;
  } else {
    it.t0 = w_begin + (a - nsink) * Tw;
    it.t1 = min(L, it.t0 + Tw);
  }
  approx_fused_body<KV, D, G>(pa, it, q, k, v, L_cap, Hq, sm_log2, w, o);
}

// Merge of one head group's sink and window states (one block per
// (entry, kv head)).  The split states come from an earlier kernel, so no
// fence is needed.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void approx_combine_kernel(PlanArgs pa,
                                                                  WsPtrs w,
                                                                  Outs o) {
  approx_merge<D, G>(pa, w, o, blockIdx.x / pa.Hkv, blockIdx.x % pa.Hkv);
}

// Exact merge of NH query heads (the plan's NHv) of one entry, verify and
// commit: the block merges each head's stored sink+window state with its
// middle splits in one memory round; the last block of the entry to finish
// issues the verdict.  Shared by the fused call and the layer-pipelined
// launch, so both give the same bits.
template <int D, int NH>
__device__ void verify_block(const PlanArgs &pa, const WsPtrs &w,
                             const Outs &o, int idx) {
  const int per = pa.Hq / NH;
  const int b = idx / per, h0 = (idx % per) * NH;
  exact_heads<D, NH>(pa, w, b, h0, o.o_approx, o.o_exact, o.lse_exact);
  if (!arrive_last(user_counter(w, b), (unsigned)per)) return;
  finalize_entry<D>(pa, w, b, o.o_approx, o.o_exact, o.ratio, o.commit,
                    o.o_committed, o.lambda);
}

template <int D, int NH>
__global__ __launch_bounds__(kThreads) void merge_verify_kernel(PlanArgs pa,
                                                                WsPtrs w,
                                                                Outs o) {
  verify_block<D, NH>(pa, w, o, blockIdx.x);
}

// Layer-pipelined launch: one grid holds four disjoint block ranges, all
// resident at once (two 4-wave blocks fit a CU):
//   [0, nM)              the middle splits of layer j, dispatched first,
//   [nM, nM + nA)        the sink and window splits of layer j+1,
//   [.., + nG)           the merge of layer j's sink and window states
//                        (written by the launch before) into its
//                        approximate output, one block per (entry, kv
//                        head),
//   [.., ...)            merge, verify and commit of layer j-1.
// The middle blocks come first so that on each CU the middle split is the
// older block, whose waves the arbiter favours: the short blocks beside it
// then take the issue slots it leaves (the steady launch at 128K: 82.05
// against 82.5-82.7 us with the merges and splits dispatched first).
// Launch order alone then carries every dependency of the chain: a
// layer's merge follows its splits by one launch, its middle splits need
// nothing of the approximation, and layer j-1's verify follows its
// middle splits and merged approximation.  No block of the launch hands
// data to another, so none takes a device-scope fence: merging each
// group's splits in the same launch (a release per split block, the last
// one merging) cost about 4 us of a 95 us launch, because the L2
// write-backs stall the XCDs' streaming blocks.
template <class KV, int D, int G>
__global__ __launch_bounds__(kThreads) void chain_kernel(
    PlanArgs pa, ChainLayer mid, ChainLayer app, ChainLayer ver, int nG,
    int nM, int nA, float sm_log2) {
  using E = typename KV::elem;
  const int Hq = pa.Hq;
  int idx = blockIdx.x;
  if (idx >= nM + nA) {
    idx -= nM + nA;
    if (idx < nG) {
      approx_merge<D, G>(pa, mid.w, mid.o, idx / pa.Hkv, idx % pa.Hkv);
      return;
    }
    idx -= nG;
    if (pa.NHv == 4)
      verify_block<D, 4>(pa, ver.w, ver.o, idx);
    else if (pa.NHv == 2)
      verify_block<D, 2>(pa, ver.w, ver.o, idx);
    else
      verify_block<D, 1>(pa, ver.w, ver.o, idx);
    return;
  }
  const bool approx = idx >= nM;
  const ChainLayer &L = approx ? app : mid;
  const Item it = decode_item(pa, approx, approx ? idx - nM : idx);
  const size_t kv_off = ((size_t)it.b * pa.Hkv + it.g) * pa.L_cap * D;
  const int h0 = it.g * G;
  split_any<KV, D, G>(L.q + ((size_t)it.b * Hq + h0) * D,
                            (const E *)L.k + kv_off, (const E *)L.v + kv_off,
                            it.t0, it.t1, sm_log2,
                            L.w.part_ml + (size_t)it.slot * Hq + h0,
                            L.w.part_acc + ((size_t)it.slot * Hq + h0) * D);
}

// --------------------------------------------------- one-launch chain ---

// Waits of one block for another's items poll at most this often, about
// 1.7 us apart (about a second in all); a wait that runs out counts itself
// in the launch's error counter and goes on, so no wave ever waits without
// end.  The waits last tens of microseconds; polling less often keeps the
// waiting blocks' loads of one counter line off the memory system that the
// streaming blocks use.
constexpr unsigned kChainSpinLimit = 1u << 19;

// Thread 0 waits until *cnt reaches target; the barrier then lets the block
// read what the counted items stored, with agent-scope loads (no acquire
// fence: its L2 invalidation would disturb the blocks streaming beside).
__device__ void chain_wait(unsigned *cnt, unsigned target, unsigned *err) {
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           target) {
      __builtin_amdgcn_s_sleep(64);
      if (++spins > kChainSpinLimit) {
        __hip_atomic_fetch_add(err, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// Counts one finished item whose results the block stored with agent-scope
// atomic stores: every thread waits for its stores' completion, then
// thread 0 adds one.
__device__ void chain_signal(unsigned *cnt) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// verify_block for a launch whose other blocks run the same layer's items:
// the exact outputs and per-head sums go out as agent-scope atomic stores
// and the entry's last block takes them over without a cache write-back.
template <int D, int NH>
__device__ void verify_block_co(const PlanArgs &pa, const WsPtrs &w,
                                const Outs &o, int idx) {
  const int per = pa.Hq / NH;
  const int b = idx / per, h0 = (idx % per) * NH;
  exact_heads<D, NH, true, true>(pa, w, b, h0, o.o_approx, o.o_exact,
                                 o.lse_exact);
  if (!arrive_last_coherent<false>(user_counter(w, b), (unsigned)per))
    return;
  finalize_entry<D, true>(pa, w, b, o.o_approx, o.o_exact, o.ratio, o.commit,
                          o.o_committed, o.lambda);
}

__device__ __forceinline__ WsPtrs chain_ws(const OneChainArgs &ca,
                                           char *base) {
  WsPtrs w;
  w.counters = (unsigned *)(base + ca.off_counters);
  w.part_ml = (float2 *)(base + ca.off_part_ml);
  w.part_acc = (float *)(base + ca.off_part_acc);
  w.stA_ml = (float2 *)(base + ca.off_stA_ml);
  w.stA_acc = (float *)(base + ca.off_stA_acc);
  w.headnd = (float2 *)(base + ca.off_headnd);
  return w;
}

// Control block: queue (line 0), finished blocks (line 1), errors (line 2),
// then per layer j one line with its finished sink/window splits, middle
// splits, merges and verifies.
__device__ __forceinline__ unsigned *chain_line(const OneChainArgs &ca,
                                                int line) {
  return (unsigned *)ca.ctl + line * kCounterStride;
}
enum ChainCount { kCntA = 0, kCntM = 8, kCntG = 16, kCntV = 24 };
__device__ __forceinline__ unsigned *chain_count(const OneChainArgs &ca,
                                                 int layer, ChainCount c) {
  return chain_line(ca, 3 + layer) + c;
}

// A chain of independent layers in one launch, one block per item of the
// queue (one_chain_items):
//   the sink and window splits of layer 0, then for each layer s:
//     the merge of layer s's sink and window states   (waits: its splits)
//     the sink and window splits of layer s+1          (waits: see below)
//     the middle splits of layer s                     (waits: see below)
//     the exact merge, verify and commit of layer s-1  (waits: its middle
//                                                       splits and merge)
//   then the verify of the last layer.
// A block takes the next item with one atomic add when it starts, not the
// item of its index, so the XCDs whose blocks stream faster take more of
// the items, and no layer's slowest blocks hold up the next layer's middle
// splits: the launch ends once, after the last layer.  (The hardware deals
// block indices to the XCDs in turn, so items fixed by index would keep
// each XCD's share fixed.)  A layer's splits first wait until the latest
// earlier layer on the same workspace has finished its verify.  Every wait
// is for items earlier in the queue, so for blocks already running, and is
// bounded.  Every item runs the same code as in the per-layer launches, so
// the bits are the same.  The last block to finish resets the control
// block (but the error count, kept for inspection).
template <class KV, int D, int G>
__global__ __launch_bounds__(kThreads) void one_chain_kernel(PlanArgs pa,
                                                             OneChainArgs ca,
                                                             float sm_log2) {
  using E = typename KV::elem;
  __shared__ int s_item;
  unsigned *err = chain_line(ca, 2);
  const int nG = pa.B * pa.Hkv;
  const int nA = pa.itemA_pre[pa.B];
  const int nM = pa.itemM_pre[pa.B];
  const int nV = pa.B * pa.Hq / pa.NHv;
  const int n = ca.n;
  const int Hq = pa.Hq;
  if (threadIdx.x == 0)
    s_item = (int)__hip_atomic_fetch_add(chain_line(ca, 0), 1u,
                                         __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // the item is the same for the whole block: keep it (and every index and
  // branch derived from it) scalar
  int k = __builtin_amdgcn_readfirstlane(s_item);
  // kind: 0 merge, 1 sink/window split, 2 middle split, 3 verify; layer
  int kind, layer;
  if (k < nA) {
    kind = 1;
    layer = 0;
  } else {
    k -= nA;
    int s = 0;
    kind = 3;
    layer = n - 1;  // past every segment: the last layer's verify
    for (; s < n; ++s) {
      const int a = s + 1 < n ? nA : 0;
      const int v = s > 0 ? nV : 0;
      if (k < nG) {
        kind = 0;
        layer = s;
        break;
      }
      k -= nG;
      if (k < a) {
        kind = 1;
        layer = s + 1;
        break;
      }
      k -= a;
      if (k < nM) {
        kind = 2;
        layer = s;
        break;
      }
      k -= nM;
      if (k < v) {
        kind = 3;
        layer = s - 1;
        break;
      }
      k -= v;
    }
  }
  const ChainEntry &L = ca.table[layer];
  char *base = L.ws;
  const WsPtrs w = chain_ws(ca, base);
  const Outs o{L.o_approx, L.lse_approx, L.o_exact, L.lse_exact, L.ratio,
               L.commit,   L.o_committed, ca.lambda};
  if (kind == 0) {
    chain_wait(chain_count(ca, layer, kCntA), nA, err);
    approx_merge<D, G, true>(pa, w, o, k / pa.Hkv, k % pa.Hkv);
    chain_signal(chain_count(ca, layer, kCntG));
  } else if (kind != 3) {
    // the layer's workspace is free once the layer before on it is done
    if (L.prev >= 0) chain_wait(chain_count(ca, L.prev, kCntV), nV, err);
    const bool approx = kind == 1;
    const Item it = decode_item(pa, approx, k);
    const size_t kv_off = ((size_t)it.b * pa.Hkv + it.g) * pa.L_cap * D;
    const int h0 = it.g * G;
    split_any<KV, D, G, true>(L.q + ((size_t)it.b * Hq + h0) * D,
                              (const E *)L.k + kv_off,
                              (const E *)L.v + kv_off, it.t0, it.t1, sm_log2,
                              w.part_ml + (size_t)it.slot * Hq + h0,
                              w.part_acc + ((size_t)it.slot * Hq + h0) * D);
    chain_signal(chain_count(ca, layer, approx ? kCntA : kCntM));
  } else {
    chain_wait(chain_count(ca, layer, kCntM), nM, err);
    chain_wait(chain_count(ca, layer, kCntG), nG, err);
    if (pa.NHv == 4)
      verify_block_co<D, 4>(pa, w, o, k);
    else if (pa.NHv == 2)
      verify_block_co<D, 2>(pa, w, o, k);
    else
      verify_block_co<D, 1>(pa, w, o, k);
    chain_signal(chain_count(ca, layer, kCntV));
  }
  // The last block to finish resets the control block.  Every block has
  // taken its item (and left its waits) by then.
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(
        chain_line(ca, 1), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      __hip_atomic_store(chain_line(ca, 0), 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(chain_line(ca, 1), 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      for (int j = 0; j < n; ++j)
        for (int c = 0; c < 32; c += 8)
          __hip_atomic_store(chain_line(ca, 3 + j) + c, 0u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Entries of the layer table per launch of the table writer (kernel
// arguments).
constexpr int kChainTableChunk = 40;
struct ChainTableChunk {
  ChainEntry *dst;
  int n;
  ChainEntry e[kChainTableChunk];
};

__global__ void chain_table_kernel(ChainTableChunk c) {
  if ((int)threadIdx.x < c.n) c.dst[threadIdx.x] = c.e[threadIdx.x];
}

// Second stage of the exact output from every split state of the plan:
// one block per NH query heads of an entry (the plan's NHv) merges each
// head's middle states onto the merged sink+window state, as the fused
// call's exact merge does (so both give the same bits).
template <int D, int NH>
__global__ __launch_bounds__(kThreads) void lse_middle_kernel(
    PlanArgs pa, WsPtrs w, float *__restrict__ o_exact,
    float *__restrict__ lse_exact) {
  const int per = pa.Hq / NH;
  exact_heads<D, NH, false>(pa, w, blockIdx.x / per,
                            (blockIdx.x % per) * NH, nullptr, o_exact,
                            lse_exact);
}

// Standalone verify, one block per entry: num and den over the entry's
// Hq * D outputs, read 16 bytes at a time with a thread's loads all in
// flight, summed per wave in a fixed butterfly order and then in wave
// order.  Entries of up to kVerifyRegs * 4 * kThreads floats stay in
// registers, and the committed output is written from them.
constexpr int kVerifyRegs = 8;
__global__ __launch_bounds__(kThreads) void verify_kernel(
    int n_per_entry, const float *__restrict__ o_approx,
    const float *__restrict__ o_exact, float *__restrict__ ratio,
    uint8_t *__restrict__ commit, float *__restrict__ o_committed,
    float lambda) {
  __shared__ float s_n[kWaves], s_d[kWaves];
  __shared__ int s_commit;
  const int b = blockIdx.x, t = threadIdx.x;
  const size_t base = (size_t)b * n_per_entry;
  const float4 *a4 = (const float4 *)(o_approx + base);
  const float4 *e4 = (const float4 *)(o_exact + base);
  const int n4 = n_per_entry >> 2;
  float4 av[kVerifyRegs], ev[kVerifyRegs];
  float num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < n4; c0 += kVerifyRegs * kThreads) {
#pragma unroll
    for (int k = 0; k < kVerifyRegs; ++k) {
      const int i = c0 + k * kThreads + t;
      if (i < n4) {
        av[k] = a4[i];
        ev[k] = e4[i];
      }
    }
#pragma unroll
    for (int k = 0; k < kVerifyRegs; ++k) {
      if (c0 + k * kThreads + t < n4) {
        const float4 e = ev[k], a = av[k];
        const float dx = a.x - e.x, dy = a.y - e.y, dz = a.z - e.z,
                    dw = a.w - e.w;
        num += dx * dx;
        num += dy * dy;
        num += dz * dz;
        num += dw * dw;
        den += e.x * e.x;
        den += e.y * e.y;
        den += e.z * e.z;
        den += e.w * e.w;
      }
    }
  }
  num = group_sum<64>(num);
  den = group_sum<64>(den);
  if ((t & 63) == 0) {
    s_n[t >> 6] = num;
    s_d[t >> 6] = den;
  }
  __syncthreads();
  if (t == 0) {
    float tn = s_n[0], td = s_d[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      tn += s_n[w];
      td += s_d[w];
    }
    const float rt = ratio_of(tn, td);
    ratio[b] = rt;
    s_commit = rt <= lambda ? 1 : 0;
    commit[b] = (uint8_t)s_commit;
  }
  __syncthreads();
  if (o_committed) {
    float4 *o4 = (float4 *)(o_committed + base);
    if (n4 <= kVerifyRegs * kThreads) {
#pragma unroll
      for (int k = 0; k < kVerifyRegs; ++k) {
        const int i = k * kThreads + t;
        if (i < n4) o4[i] = s_commit ? av[k] : ev[k];
      }
    } else {
      const float4 *src = s_commit ? a4 : e4;
      for (int i = t; i < n4; i += kThreads) o4[i] = src[i];
    }
  }
}

// ------------------------------------------------------------- dispatch ---

// Launch whose status is that of this launch alone (hipLaunchKernel
// returns it), not whatever error an earlier call in the thread left for
// hipGetLastError.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block,
                  hipStream_t s, Args... a) {
  std::tuple<KArgs...> t(a...);
  return std::apply(
      [&](auto &...x) {
        void *argv[] = {(void *)&x...};
        return hipLaunchKernel((const void *)kern, grid, block, argv, 0, s);
      },
      t);
}

template <class KV, int D, int G>
hipError_t partials_kg(const PlanArgs &pa, PartialsSet set, const float *q,
                       const void *k, const void *v, float sm_log2,
                       const WsPtrs &w, hipStream_t s) {
  const int nA = pa.itemA_pre[pa.B], nM = pa.itemM_pre[pa.B];
  const int items = set == kPartialsApprox   ? nA
                    : set == kPartialsMiddle ? nM
                                             : nA + nM;
  if (items == 0) return hipSuccess;
  using E = typename KV::elem;
  const dim3 grid(items), block(kThreads);
  if (set == kPartialsAll)
    return launch(partials_all_kernel<KV, D, G>, grid, block, s, pa, q,
                  (const E *)k, (const E *)v, sm_log2, w);
  auto kern = set == kPartialsApprox ? partials_kernel<KV, D, G, true>
                                     : partials_kernel<KV, D, G, false>;
  return launch(kern, grid, block, s, pa, q, (const E *)k, (const E *)v,
                sm_log2, w);
}

template <class KV, int D>
hipError_t partials_g(const PlanArgs &pa, PartialsSet set, const float *q,
                      const void *k, const void *v, float sm_log2,
                      const WsPtrs &w, hipStream_t s) {
  switch (pa.G) {
    case 1:
      return partials_kg<KV, D, 1>(pa, set, q, k, v, sm_log2, w, s);
    case 2:
      return partials_kg<KV, D, 2>(pa, set, q, k, v, sm_log2, w, s);
    case 4:
      return partials_kg<KV, D, 4>(pa, set, q, k, v, sm_log2, w, s);
    case 8:
      return partials_kg<KV, D, 8>(pa, set, q, k, v, sm_log2, w, s);
  }
  return hipErrorInvalidValue;
}

template <class KV, int D, int G>
hipError_t approx_fused_kg(const PlanArgs &pa, const float *q, const void *k,
                           const void *v, float sm_log2, const WsPtrs &w,
                           const Outs &o, hipStream_t s) {
  const int items = pa.itemA_pre[pa.B];
  if (items == 0) return hipSuccess;
  using E = typename KV::elem;
  if (pa.B == 1)
    return launch(approx_fused_one_kernel<KV, D, G>, dim3(items),
                  dim3(kThreads), s, pa.nsink[0] + pa.nwin[0], pa.s_end[0],
                  pa.w_begin[0], pa.Tw, pa.L[0], pa.L_cap, pa.Hq, q,
                  (const E *)k, (const E *)v, pa, sm_log2, w, o);
  return launch(approx_fused_kernel<KV, D, G>, dim3(items), dim3(kThreads), s,
                pa, q, (const E *)k, (const E *)v, sm_log2, w, o);
}

template <class KV, int D>
hipError_t approx_fused_g(const PlanArgs &pa, const float *q, const void *k,
                          const void *v, float sm_log2, const WsPtrs &w,
                          const Outs &o, hipStream_t s) {
  switch (pa.G) {
    case 1:
      return approx_fused_kg<KV, D, 1>(pa, q, k, v, sm_log2, w, o, s);
    case 2:
      return approx_fused_kg<KV, D, 2>(pa, q, k, v, sm_log2, w, o, s);
    case 4:
      return approx_fused_kg<KV, D, 4>(pa, q, k, v, sm_log2, w, o, s);
    case 8:
      return approx_fused_kg<KV, D, 8>(pa, q, k, v, sm_log2, w, o, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t approx_combine_d(const PlanArgs &pa, const WsPtrs &w,
                            const Outs &o, hipStream_t s) {
  dim3 grid(pa.B * pa.Hkv), block(kThreads);
  switch (pa.G) {
    case 1:
      return launch(approx_combine_kernel<D, 1>, grid, block, s, pa, w, o);
    case 2:
      return launch(approx_combine_kernel<D, 2>, grid, block, s, pa, w, o);
    case 4:
      return launch(approx_combine_kernel<D, 4>, grid, block, s, pa, w, o);
    case 8:
      return launch(approx_combine_kernel<D, 8>, grid, block, s, pa, w, o);
  }
  return hipErrorInvalidValue;
}

template <class KV, int D, int G>
hipError_t chain_kg(const PlanArgs &pa, const ChainLayer *mid,
                    const ChainLayer *app, const ChainLayer *ver,
                    bool merge_mid, float sm_log2, hipStream_t s) {
  const ChainLayer none{};
  const int nV = ver ? pa.B * pa.Hq / pa.NHv : 0;
  const int nA = app ? pa.itemA_pre[pa.B] : 0;
  const int nM = mid ? pa.itemM_pre[pa.B] : 0;
  const int nG = mid && merge_mid ? pa.B * pa.Hkv : 0;
  if (nG + nV + nA + nM == 0) return hipSuccess;
  return launch(chain_kernel<KV, D, G>, dim3(nG + nV + nA + nM),
                dim3(kThreads), s, pa, mid ? *mid : none, app ? *app : none,
                ver ? *ver : none, nG, nM, nA, sm_log2);
}

template <class KV, int D>
hipError_t chain_g(const PlanArgs &pa, const ChainLayer *mid,
                   const ChainLayer *app, const ChainLayer *ver, bool mm,
                   float sm_log2, hipStream_t s) {
  switch (pa.G) {
    case 1:
      return chain_kg<KV, D, 1>(pa, mid, app, ver, mm, sm_log2, s);
    case 2:
      return chain_kg<KV, D, 2>(pa, mid, app, ver, mm, sm_log2, s);
    case 4:
      return chain_kg<KV, D, 4>(pa, mid, app, ver, mm, sm_log2, s);
    case 8:
      return chain_kg<KV, D, 8>(pa, mid, app, ver, mm, sm_log2, s);
  }
  return hipErrorInvalidValue;
}

template <class KV, int D, int G>
hipError_t one_chain_kg(const PlanArgs &pa, const OneChainArgs &ca,
                        float sm_log2, hipStream_t s) {
  return launch(one_chain_kernel<KV, D, G>,
                dim3(one_chain_items(pa, ca.n)), dim3(kThreads), s, pa, ca,
                sm_log2);
}

template <class KV, int D>
hipError_t one_chain_g(const PlanArgs &pa, const OneChainArgs &ca,
                       float sm_log2, hipStream_t s) {
  switch (pa.G) {
    case 1:
      return one_chain_kg<KV, D, 1>(pa, ca, sm_log2, s);
    case 2:
      return one_chain_kg<KV, D, 2>(pa, ca, sm_log2, s);
    case 4:
      return one_chain_kg<KV, D, 4>(pa, ca, sm_log2, s);
    case 8:
      return one_chain_kg<KV, D, 8>(pa, ca, sm_log2, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_one_chain(const PlanArgs &pa, int kv_dtype,
                            const OneChainArgs &ca, float sm_log2,
                            hipStream_t s) {
  if (kv_dtype == ALSPEC_KV_BF16) {
    if (pa.D == 128) return one_chain_g<KvBf16, 128>(pa, ca, sm_log2, s);
    return one_chain_g<KvBf16, 64>(pa, ca, sm_log2, s);
  }
  if (pa.D == 128) return one_chain_g<KvF32, 128>(pa, ca, sm_log2, s);
  return one_chain_g<KvF32, 64>(pa, ca, sm_log2, s);
}

hipError_t launch_chain_table(const ChainEntry *src, int n, ChainEntry *dst,
                              hipStream_t s) {
  for (int i = 0; i < n; i += kChainTableChunk) {
    ChainTableChunk c;
    c.dst = dst + i;
    c.n = n - i < kChainTableChunk ? n - i : kChainTableChunk;
    for (int j = 0; j < c.n; ++j) c.e[j] = src[i + j];
    const hipError_t e =
        launch(chain_table_kernel, dim3(1), dim3(64), s, c);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_chain(const PlanArgs &pa, int kv_dtype,
                        const ChainLayer *mid, const ChainLayer *app,
                        const ChainLayer *ver, bool merge_mid, float sm_log2,
                        hipStream_t s) {
  const bool mm = merge_mid;
  if (kv_dtype == ALSPEC_KV_BF16) {
    if (pa.D == 128)
      return chain_g<KvBf16, 128>(pa, mid, app, ver, mm, sm_log2, s);
    return chain_g<KvBf16, 64>(pa, mid, app, ver, mm, sm_log2, s);
  }
  if (pa.D == 128) return chain_g<KvF32, 128>(pa, mid, app, ver, mm, sm_log2, s);
  return chain_g<KvF32, 64>(pa, mid, app, ver, mm, sm_log2, s);
}

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

hipError_t launch_partials(const PlanArgs &pa, int kv_dtype, PartialsSet set,
                           const float *q, const void *k, const void *v,
                           float sm_log2, const WsPtrs &w, hipStream_t s) {
  if (kv_dtype == ALSPEC_KV_BF16) {
    if (pa.D == 128)
      return partials_g<KvBf16, 128>(pa, set, q, k, v, sm_log2, w, s);
    return partials_g<KvBf16, 64>(pa, set, q, k, v, sm_log2, w, s);
  }
  if (pa.D == 128)
    return partials_g<KvF32, 128>(pa, set, q, k, v, sm_log2, w, s);
  return partials_g<KvF32, 64>(pa, set, q, k, v, sm_log2, w, s);
}

hipError_t launch_approx_fused(const PlanArgs &pa, int kv_dtype,
                               const float *q, const void *k, const void *v,
                               float sm_log2, const WsPtrs &w, const Outs &o,
                               hipStream_t s) {
  if (kv_dtype == ALSPEC_KV_BF16) {
    if (pa.D == 128)
      return approx_fused_g<KvBf16, 128>(pa, q, k, v, sm_log2, w, o, s);
    return approx_fused_g<KvBf16, 64>(pa, q, k, v, sm_log2, w, o, s);
  }
  if (pa.D == 128)
    return approx_fused_g<KvF32, 128>(pa, q, k, v, sm_log2, w, o, s);
  return approx_fused_g<KvF32, 64>(pa, q, k, v, sm_log2, w, o, s);
}

hipError_t launch_approx_combine(const PlanArgs &pa, const WsPtrs &w,
                                 const Outs &o, hipStream_t s) {
  if (pa.D == 128) return approx_combine_d<128>(pa, w, o, s);
  return approx_combine_d<64>(pa, w, o, s);
}

hipError_t launch_merge_verify(const PlanArgs &pa, const WsPtrs &w,
                               const Outs &o, hipStream_t s) {
  dim3 grid(pa.B * pa.Hq / pa.NHv), block(kThreads);
  if (pa.NHv == 4) {
    if (pa.D == 128)
      return launch(merge_verify_kernel<128, 4>, grid, block, s, pa, w, o);
    return launch(merge_verify_kernel<64, 4>, grid, block, s, pa, w, o);
  }
  if (pa.NHv == 2) {
    if (pa.D == 128)
      return launch(merge_verify_kernel<128, 2>, grid, block, s, pa, w, o);
    return launch(merge_verify_kernel<64, 2>, grid, block, s, pa, w, o);
  }
  if (pa.D == 128)
    return launch(merge_verify_kernel<128, 1>, grid, block, s, pa, w, o);
  return launch(merge_verify_kernel<64, 1>, grid, block, s, pa, w, o);
}

hipError_t launch_lse_combine(const PlanArgs &pa, const WsPtrs &w,
                              float *o_exact, float *lse_exact,
                              hipStream_t s) {
  // the sink+window state (as the approximation merges it), then the middle
  // states on top of it
  const Outs none{};
  const hipError_t e = launch_approx_combine(pa, w, none, s);
  if (e != hipSuccess) return e;
  dim3 grid(pa.B * pa.Hq / pa.NHv), block(kThreads);
  if (pa.NHv == 4) {
    if (pa.D == 128)
      return launch(lse_middle_kernel<128, 4>, grid, block, s, pa, w, o_exact,
                    lse_exact);
    return launch(lse_middle_kernel<64, 4>, grid, block, s, pa, w, o_exact,
                  lse_exact);
  }
  if (pa.NHv == 2) {
    if (pa.D == 128)
      return launch(lse_middle_kernel<128, 2>, grid, block, s, pa, w, o_exact,
                    lse_exact);
    return launch(lse_middle_kernel<64, 2>, grid, block, s, pa, w, o_exact,
                  lse_exact);
  }
  if (pa.D == 128)
    return launch(lse_middle_kernel<128, 1>, grid, block, s, pa, w, o_exact,
                  lse_exact);
  return launch(lse_middle_kernel<64, 1>, grid, block, s, pa, w, o_exact,
                lse_exact);
}

hipError_t launch_verify(const PlanArgs &pa, const float *o_approx,
                         const float *o_exact, float *ratio, uint8_t *commit,
                         float *o_committed, float lambda, hipStream_t s) {
  return launch(verify_kernel, dim3(pa.B), dim3(kThreads), s, pa.Hq * pa.D,
                o_approx, o_exact, ratio, commit, o_committed, lambda);
}

}  // namespace alspec
