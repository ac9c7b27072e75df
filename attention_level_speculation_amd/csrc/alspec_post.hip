// Post-attention operators of one decoder layer for a decode token per
// batch entry, the work that attention-level speculation runs early on the
// approximate attention output ("Attention-Level Speculation", research-map
// page, summary and Approach: the post-attention ops run speculatively
// while exact attention is computed).  The operators follow the Llama
// decoder layer that the pages' 8B and 70B shapes name, with random bf16
// weights:
//   h1  = h_in + W_o o                             (output projection)
//   m   = silu(W_gate x) * (W_up x),  x = rmsnorm(h1) * g_mlp
//   h2  = h1 + W_down m
//   qkv = W_qkv y,  y = rmsnorm(h2) * g_attn        (next layer's input)
// with rmsnorm(v) = v / sqrt(mean(v^2) + eps).
//
// Every product is a skinny matrix-vector product (B <= 8 rows of
// activations against a bf16 weight matrix read once), so each kernel is
// bound by HBM bandwidth: 2 bytes per weight for B fused multiply-adds.
// One wave owns kRows (4, 2 or 1, chosen per matrix so that the blocks
// fill whole rounds of the CUs) consecutive weight rows and walks the
// shared dimension K in 16-byte chunks (8 bf16), lane l taking chunks l,
// l + 64, ...; U chunks per row are loaded before any is used.  For one or
// two entries the gated MLP and the down projection, the products with the
// most K per row, split K across the four waves of a block instead (one
// block per 2 or 4 rows, the waves' sums added in wave order): four times
// the waves in flight, which the few multiply-adds per loaded weight of a
// small batch leave room for.  The
// activations are read from L2 (they are a few KiB and shared by every
// wave), for small batches in the same round as the weights.  The row sums are reduced across the wave by
// butterflies in a fixed order, so results do not depend on timing.
//
// The RMSNorm is folded into the products: sum_k W[n][k] (v[k] r g[k]) =
// r * sum_k W[n][k] (v[k] g[k]), and each wave accumulates sum_k v[k]^2
// from the same chunks it multiplies, so no separate pass or kernel
// computes the norm.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>


#include "alspec_kernels.h"

#pragma clang fp contract(on)

namespace alspec {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCUs = 256;  // compute units of an MI355X

__device__ __forceinline__ void unpack_bf16(const uint4 r, float *f) {
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

// Weight chunks are read once per product, so they are loaded nontemporal:
// at the 8B layer that took the four products from 81.0 to 76.7 us, the
// same bits.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_weights(const uint16_t *p) {
  const u32x4v t = __builtin_nontemporal_load((const u32x4v *)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// True when entry b's outputs are to be written (no skip flags, or its
// flag is zero).
__device__ __forceinline__ bool active(const uint8_t *skip, int b) {
  return skip == nullptr || skip[b] == 0;
}

template <int B>
__device__ __forceinline__ bool any_active(const uint8_t *skip) {
  if (skip == nullptr) return true;
  bool any = false;
#pragma unroll
  for (int b = 0; b < B; ++b) any = any || skip[b] == 0;
  return any;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Row sums acc[m][r][b] = sum_k W_m[n0 + r][k] * x[b][k] * (g[k] if G)
// over k in [0, K), for NW weight matrices sharing rows n0 .. n0+kRows-1
// (rows past `nrows` repeat the last valid row and are not written by the
// callers).  With G, ss[b] = sum_k x[b][k]^2.  Sums are complete in every
// lane on return.
template <int B, int NW, bool G, int kRows>
__device__ __forceinline__ void wave_rows(const uint16_t *const *W, int n0,
                                          int nrows, int K,
                                          const float *__restrict__ x,
                                          const uint16_t *__restrict__ g,
                                          float (&acc)[NW][kRows][B],
                                          float (&ss)[B], int cb, int ce) {
  constexpr int U = 4 / NW;  // chunks per row in flight
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < NW; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[m][r][b] = 0.f;
#pragma unroll
  for (int b = 0; b < B; ++b) ss[b] = 0.f;
  const uint16_t *rowp[NW][kRows];
#pragma unroll
  for (int m = 0; m < NW; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      rowp[m][r] = W[m] + (size_t)(n0 + min(r, nrows - 1)) * K;

  // The activation chunks (and norm weights) of small batches are loaded
  // with the weight chunks, so one wait covers both round trips.
  constexpr bool XPRE = B <= 2;
  for (int c0 = cb; c0 < ce; c0 += 64 * U) {
    uint4 wv[NW][kRows][U];
    float4 xp[XPRE ? B : 1][U][2];
    uint4 gp[G && XPRE ? U : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u * 64 + lane, ce - 1);
#pragma unroll
      for (int m = 0; m < NW; ++m)
#pragma unroll
        for (int r = 0; r < kRows; ++r)
          wv[m][r][u] = load_weights(rowp[m][r] + (size_t)c * 8);
      if constexpr (XPRE) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          xp[b][u][0] = *(const float4 *)(x + (size_t)b * K + c * 8);
          xp[b][u][1] = *(const float4 *)(x + (size_t)b * K + c * 8 + 4);
        }
        if constexpr (G) gp[u] = *(const uint4 *)(g + (size_t)c * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < ce) {
        float gs[8];
        if constexpr (G) {
          if constexpr (XPRE)
            unpack_bf16(gp[u], gs);
          else
            unpack_bf16(*(const uint4 *)(g + (size_t)c * 8), gs);
        }
        float wf[NW][kRows][8];
#pragma unroll
        for (int m = 0; m < NW; ++m)
#pragma unroll
          for (int r = 0; r < kRows; ++r) unpack_bf16(wv[m][r][u], wf[m][r]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float4 xa, xb;
          if constexpr (XPRE) {
            xa = xp[b][u][0];
            xb = xp[b][u][1];
          } else {
            xa = *(const float4 *)(x + (size_t)b * K + c * 8);
            xb = *(const float4 *)(x + (size_t)b * K + c * 8 + 4);
          }
          float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
          if constexpr (G) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              ss[b] += xv[i] * xv[i];
              xv[i] *= gs[i];
            }
          }
#pragma unroll
          for (int m = 0; m < NW; ++m)
#pragma unroll
            for (int r = 0; r < kRows; ++r)
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[m][r][b] += wf[m][r][i] * xv[i];
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NW; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[m][r][b] = wave_sum(acc[m][r][b]);
  if constexpr (G) {
#pragma unroll
    for (int b = 0; b < B; ++b) ss[b] = wave_sum(ss[b]);
  }
}

// Split K across the block: the four waves share rows n0 .. n0+kRows-1,
// wave w taking chunks [w n / 4, (w+1) n / 4) of the n = K / 8; the waves'
// sums are then added in wave order (fixed, so results do not depend on
// timing).  On return thread t < kRows * B holds row t / B, entry t % B in
// *v (and v2 for the second matrix) and the full sum of squares in *s2.
template <int B, int NW, bool G, int kRows>
__device__ __forceinline__ void block_rows_sk(const uint16_t *const *W,
                                              int n0, int nrows, int K,
                                              const float *__restrict__ x,
                                              const uint16_t *__restrict__ g,
                                              float *v, float *v2,
                                              float *s2) {
  constexpr int NV = NW * kRows * B;
  __shared__ float red[kWaves][NV + B];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nchunk = K >> 3;
  float acc[NW][kRows][B], ss[B];
  wave_rows<B, NW, G, kRows>(W, n0, nrows, K, x, g, acc, ss,
                             wave * nchunk / kWaves,
                             (wave + 1) * nchunk / kWaves);
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < NW; ++m)
#pragma unroll
      for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b)
          red[wave][(m * kRows + r) * B + b] = acc[m][r][b];
#pragma unroll
    for (int b = 0; b < B; ++b) red[wave][NV + b] = G ? ss[b] : 0.f;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < kRows * B) {
    const int b = t % B;
    float a = red[0][t], a2 = NW > 1 ? red[0][kRows * B + t] : 0.f;
    float q = red[0][NV + b];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      a += red[w][t];
      if (NW > 1) a2 += red[w][kRows * B + t];
      q += red[w][NV + b];
    }
    *v = a;
    *v2 = a2;
    *s2 = q;
  }
}

struct PostArgsK {
  int N, K;
  float eps;
  const uint16_t *w0, *w1;  // weight matrices [N][K]
  const uint16_t *g;        // norm weight [K] (norm kernels)
  const float *x;           // activations [B][K]
  const float *base;        // residual [B][N] (residual kernels)
  float *y;                 // output [B][N]
  const uint8_t *skip;      // [B] or null
};

// y[b][n] = base[b][n] + sum_k W[n][k] x[b][k]   (output and down
// projections; y may alias base).
template <int B, int kRows>
__global__ __launch_bounds__(kThreads) void gemv_residual_kernel(PostArgsK a) {
  if (!any_active<B>(a.skip)) return;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int n0 = wave * kRows;
  if (n0 >= a.N) return;
  const int nrows = min(kRows, a.N - n0);
  const uint16_t *W[1] = {a.w0};
  float acc[1][kRows][B], ss[B];
  wave_rows<B, 1, false, kRows>(W, n0, nrows, a.K, a.x, nullptr, acc, ss, 0,
                                a.K >> 3);
  const int lane = threadIdx.x & 63;
  if (lane < kRows * B) {
    const int r = lane / B, b = lane % B;
    float v = 0.f;
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
      for (int bb = 0; bb < B; ++bb)
        if (rr == r && bb == b) v = acc[0][rr][bb];
    if (r < nrows && active(a.skip, b)) {
      const size_t i = (size_t)b * a.N + n0 + r;
      a.y[i] = a.base[i] + v;
    }
  }
}

// m[b][n] = silu(r_b gate) * (r_b up), gate/up = sum_k W_{gate,up}[n][k]
// x[b][k] g[k], r_b = 1 / sqrt(mean_k x[b][k]^2 + eps).
template <int B, int kRows>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(PostArgsK a) {
  if (!any_active<B>(a.skip)) return;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int n0 = wave * kRows;
  if (n0 >= a.N) return;
  const int nrows = min(kRows, a.N - n0);
  const uint16_t *W[2] = {a.w0, a.w1};
  float acc[2][kRows][B], ss[B];
  wave_rows<B, 2, true, kRows>(W, n0, nrows, a.K, a.x, a.g, acc, ss, 0,
                               a.K >> 3);
  const int lane = threadIdx.x & 63;
  if (lane < kRows * B) {
    const int r = lane / B, b = lane % B;
    float gv = 0.f, uv = 0.f, s2 = 0.f;
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
      for (int bb = 0; bb < B; ++bb)
        if (rr == r && bb == b) {
          gv = acc[0][rr][bb];
          uv = acc[1][rr][bb];
        }
#pragma unroll
    for (int bb = 0; bb < B; ++bb)
      if (bb == b) s2 = ss[bb];
    if (r < nrows && active(a.skip, b)) {
      const float rn = 1.f / sqrtf(s2 / (float)a.K + a.eps);
      gv *= rn;
      uv *= rn;
      a.y[(size_t)b * a.N + n0 + r] = gv / (1.f + expf(-gv)) * uv;
    }
  }
}

// y[b][n] = r_b sum_k W[n][k] x[b][k] g[k]   (next layer's QKV).
template <int B, int kRows>
__global__ __launch_bounds__(kThreads) void gemv_norm_kernel(PostArgsK a) {
  if (!any_active<B>(a.skip)) return;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int n0 = wave * kRows;
  if (n0 >= a.N) return;
  const int nrows = min(kRows, a.N - n0);
  const uint16_t *W[1] = {a.w0};
  float acc[1][kRows][B], ss[B];
  wave_rows<B, 1, true, kRows>(W, n0, nrows, a.K, a.x, a.g, acc, ss, 0,
                               a.K >> 3);
  const int lane = threadIdx.x & 63;
  if (lane < kRows * B) {
    const int r = lane / B, b = lane % B;
    float v = 0.f, s2 = 0.f;
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
      for (int bb = 0; bb < B; ++bb)
        if (rr == r && bb == b) v = acc[0][rr][bb];
#pragma unroll
    for (int bb = 0; bb < B; ++bb)
      if (bb == b) s2 = ss[bb];
    if (r < nrows && active(a.skip, b))
      a.y[(size_t)b * a.N + n0 + r] = v / sqrtf(s2 / (float)a.K + a.eps);
  }
}

// Row form for one entry and K up to kStageK: the block copies x (and the
// norm weight) into LDS once, where each wave of the plain form loads all
// of it, and every wave requests all its weights in one round (the plain
// form takes two at K = 4096).  Each wave then reads x and g from LDS
// while its weights are in flight and does the plain form's arithmetic in
// its order (the same bits).  y = base + W x (RES) or
// y = r W (x g) with r = 1 / sqrt(mean x^2 + eps) (G).
constexpr int kStageK = 4096;

template <int kRows, bool G, bool RES>
__global__ __launch_bounds__(kThreads) void gemv_staged_kernel(PostArgsK a) {
  if (!any_active<1>(a.skip)) return;
  constexpr int U = kStageK / 8 / 64;          // chunks per lane and row
  constexpr int SC = kStageK / 8 / kThreads;   // staged chunks per thread
  __shared__ uint4 xs[kStageK / 4];            // x as fp32, 4 per uint4
  __shared__ uint4 gs_[G ? kStageK / 8 : 1];   // g as bf16, 8 per uint4
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int K = a.K, nck = K >> 3;
  const int n0 = (blockIdx.x * kWaves + wave) * kRows;
  // waves past the last row still take part in the barrier
  const int nrows = max(0, min(kRows, a.N - n0));

  // staging loads first: memory counters drain in issue order, so the
  // wait for them before the LDS stores leaves the weights in flight
  uint4 xr[SC][2], gr[G ? SC : 1];
#pragma unroll
  for (int s = 0; s < SC; ++s) {
    const int c = min(threadIdx.x + s * kThreads, nck - 1);
    xr[s][0] = *(const uint4 *)(a.x + (size_t)c * 8);
    xr[s][1] = *(const uint4 *)(a.x + (size_t)c * 8 + 4);
    if constexpr (G) gr[s] = *(const uint4 *)(a.g + (size_t)c * 8);
  }
  uint4 wv[kRows][U];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const uint16_t *rowp =
        a.w0 + (size_t)min(n0 + r, a.N - 1) * K;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(u * 64 + lane, nck - 1);
      wv[r][u] = load_weights(rowp + (size_t)c * 8);
    }
  }
  // threads past the last chunk store the last chunk again (same values)
#pragma unroll
  for (int s = 0; s < SC; ++s) {
    const int c = min(threadIdx.x + s * kThreads, nck - 1);
    xs[2 * c] = xr[s][0];
    xs[2 * c + 1] = xr[s][1];
    if constexpr (G) gs_[c] = gr[s];
  }
  __syncthreads();

  float acc[kRows], ss = 0.f;
  float xv[U][8];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = u * 64 + lane;
    if (c < nck) {
      const uint4 x0 = xs[2 * c], x1 = xs[2 * c + 1];
      const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[u][i] = __uint_as_float(xw[i]);
      if constexpr (G) {
        float gf[8];
        unpack_bf16(gs_[c], gf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ss += xv[u][i] * xv[u][i];
          xv[u][i] *= gf[i];
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = u * 64 + lane;
    if (c < nck) {
      float wf[kRows][8];
#pragma unroll
      for (int r = 0; r < kRows; ++r) unpack_bf16(wv[r][u], wf[r]);
#pragma unroll
      for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[r] += wf[r][i] * xv[u][i];
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = wave_sum(acc[r]);
  if constexpr (G) ss = wave_sum(ss);
  if (lane < kRows) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      if (r == lane) v = acc[r];
    if (lane < nrows && active(a.skip, 0)) {
      const size_t i = (size_t)n0 + lane;
      if constexpr (RES)
        a.y[i] = a.base[i] + v;
      else
        a.y[i] = v / sqrtf(ss / (float)K + a.eps);
    }
  }
}

// Split-K forms: one block per kRows rows (see block_rows_sk).
template <int B, int kRows>
__global__ __launch_bounds__(kThreads) void gemv_residual_sk_kernel(
    PostArgsK a) {
  if (!any_active<B>(a.skip)) return;
  const int n0 = blockIdx.x * kRows;
  const int nrows = min(kRows, a.N - n0);
  const uint16_t *W[1] = {a.w0};
  float v = 0.f, v2 = 0.f, s2 = 0.f;
  block_rows_sk<B, 1, false, kRows>(W, n0, nrows, a.K, a.x, nullptr, &v, &v2,
                                    &s2);
  const int t = threadIdx.x;
  if (t < kRows * B) {
    const int r = t / B, b = t % B;
    if (r < nrows && active(a.skip, b)) {
      const size_t i = (size_t)b * a.N + n0 + r;
      a.y[i] = a.base[i] + v;
    }
  }
}

template <int B, int kRows>
__global__ __launch_bounds__(kThreads) void gate_up_sk_kernel(PostArgsK a) {
  if (!any_active<B>(a.skip)) return;
  const int n0 = blockIdx.x * kRows;
  const int nrows = min(kRows, a.N - n0);
  const uint16_t *W[2] = {a.w0, a.w1};
  float gv = 0.f, uv = 0.f, s2 = 0.f;
  block_rows_sk<B, 2, true, kRows>(W, n0, nrows, a.K, a.x, a.g, &gv, &uv,
                                   &s2);
  const int t = threadIdx.x;
  if (t < kRows * B) {
    const int r = t / B, b = t % B;
    if (r < nrows && active(a.skip, b)) {
      const float rn = 1.f / sqrtf(s2 / (float)a.K + a.eps);
      gv *= rn;
      uv *= rn;
      a.y[(size_t)b * a.N + n0 + r] = gv / (1.f + expf(-gv)) * uv;
    }
  }
}

template <int B, int R>
struct ResidualSK {
  static const void *ptr() {
    return (const void *)gemv_residual_sk_kernel<B, R>;
  }
};
template <int B, int R>
struct GateUpSK {
  static const void *ptr() { return (const void *)gate_up_sk_kernel<B, R>; }
};

// Split-K launch with R rows per block.
template <template <int, int> class K, int B, int R>
hipError_t launch_sk(int n_rows, hipStream_t s, PostArgsK a) {
  const dim3 grid((n_rows + R - 1) / R), block(kThreads);
  void *argv[1] = {&a};
  return hipLaunchKernel(K<B, R>::ptr(), grid, block, argv, 0, s);
}

// Rows per wave for N rows: of 2, 4 and 1 (two rows first for one or two
// entries, four first for more, as measured fastest where all fill the CUs
// evenly), the one whose blocks (4 waves each) fill whole rounds of the
// 256 CUs best, so no CU runs an extra block while others idle.
int rows_per_wave(int N, int B) {
  const int order_small[3] = {2, 4, 1}, order_large[3] = {4, 2, 1};
  const int *order = B <= 2 ? order_small : order_large;
  int best = order[0];
  double best_eff = -1.0;
  for (int i = 0; i < 3; ++i) {
    const int r = order[i];
    const long blocks = ((N + r - 1) / r + kWaves - 1) / kWaves;
    const long rounds = (blocks + kCUs - 1) / kCUs;
    const double eff = (double)blocks / (double)(rounds * kCUs);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = r;
    }
  }
  return best;
}

template <template <int, int> class K, int B>
hipError_t launch_k(int n_rows, hipStream_t s, PostArgsK a) {
  const int r = rows_per_wave(n_rows, B);
  const int waves = (n_rows + r - 1) / r;
  const dim3 grid((waves + kWaves - 1) / kWaves), block(kThreads);
  void *argv[1] = {&a};
  const void *kern = r == 4   ? K<B, 4>::ptr()
                     : r == 2 ? K<B, 2>::ptr()
                              : K<B, 1>::ptr();
  return hipLaunchKernel(kern, grid, block, argv, 0, s);
}

// Staged row form (one entry, K <= kStageK) with the rows per wave that
// the plain form would take.
template <bool G, bool RES>
hipError_t launch_staged(int n_rows, hipStream_t s, PostArgsK a) {
  const int r = rows_per_wave(n_rows, 1);
  const int waves = (n_rows + r - 1) / r;
  const dim3 grid((waves + kWaves - 1) / kWaves), block(kThreads);
  void *argv[1] = {&a};
  const void *kern = r == 4   ? (const void *)gemv_staged_kernel<4, G, RES>
                     : r == 2 ? (const void *)gemv_staged_kernel<2, G, RES>
                              : (const void *)gemv_staged_kernel<1, G, RES>;
  return hipLaunchKernel(kern, grid, block, argv, 0, s);
}

template <int B, int R>
struct ResidualK {
  static const void *ptr() { return (const void *)gemv_residual_kernel<B, R>; }
};
template <int B, int R>
struct GateUpK {
  static const void *ptr() { return (const void *)gate_up_kernel<B, R>; }
};
template <int B, int R>
struct NormK {
  static const void *ptr() { return (const void *)gemv_norm_kernel<B, R>; }
};

template <int B>
hipError_t post_b(const PostShape &sh, const PostPtrs &p, hipStream_t s) {
  PostArgsK a{};
  a.eps = sh.eps;
  a.skip = p.skip;
  // h1 = h_in + W_o o, into h_out
  a.N = sh.hidden;
  a.K = sh.attn_dim;
  a.w0 = p.w_o;
  a.x = p.o;
  a.base = p.h_in;
  a.y = p.h_out;
  hipError_t e = B == 1 && a.K <= kStageK
                     ? launch_staged<false, true>(a.N, s, a)
                     : launch_k<ResidualK, B>(a.N, s, a);
  if (e != hipSuccess) return e;
  // m = silu(gate) * up over rmsnorm(h1) * g_mlp
  a = PostArgsK{};
  a.eps = sh.eps;
  a.skip = p.skip;
  a.N = sh.ffn;
  a.K = sh.hidden;
  a.w0 = p.w_gate;
  a.w1 = p.w_up;
  a.g = p.norm_mlp;
  a.x = p.h_out;
  a.y = p.m;
  if constexpr (B <= 2)
    e = launch_sk<GateUpSK, B, 2>(a.N, s, a);
  else
    e = launch_k<GateUpK, B>(a.N, s, a);
  if (e != hipSuccess) return e;
  // h2 = h1 + W_down m, in place
  a = PostArgsK{};
  a.eps = sh.eps;
  a.skip = p.skip;
  a.N = sh.hidden;
  a.K = sh.ffn;
  a.w0 = p.w_down;
  a.x = p.m;
  a.base = p.h_out;
  a.y = p.h_out;
  if constexpr (B <= 2)
    e = launch_sk<ResidualSK, B, 4>(a.N, s, a);
  else
    e = launch_k<ResidualK, B>(a.N, s, a);
  if (e != hipSuccess) return e;
  // qkv = W_qkv (rmsnorm(h2) * g_attn)
  a = PostArgsK{};
  a.eps = sh.eps;
  a.skip = p.skip;
  a.N = sh.qkv_dim;
  a.K = sh.hidden;
  a.w0 = p.w_qkv;
  a.g = p.norm_attn;
  a.x = p.h_out;
  a.y = p.qkv;
  if (B == 1 && a.K <= kStageK) return launch_staged<true, false>(a.N, s, a);
  return launch_k<NormK, B>(a.N, s, a);
}

}  // namespace

hipError_t launch_post_attention(const PostShape &sh, const PostPtrs &p,
                                 hipStream_t s) {
  switch (sh.batch) {
    case 1: return post_b<1>(sh, p, s);
    case 2: return post_b<2>(sh, p, s);
    case 3: return post_b<3>(sh, p, s);
    case 4: return post_b<4>(sh, p, s);
    case 5: return post_b<5>(sh, p, s);
    case 6: return post_b<6>(sh, p, s);
    case 7: return post_b<7>(sh, p, s);
    case 8: return post_b<8>(sh, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace alspec
