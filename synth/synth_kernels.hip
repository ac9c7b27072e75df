// Device twin of synth/gen.py's kv_slice: the same Philox4x32-10 counters,
// the same double-precision Box-Muller transform and planted-bias formula,
// and the same rounding (double -> float32 -> bf16, nearest even).  Built
// with -ffp-contract=off so every double operation is rounded on its own,
// as numpy does.  This library only draws inputs; it holds none of the
// attention method's arithmetic and is not part of the attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxBiasRows = 64;
constexpr int kMaxDim = 256;

struct BiasArgs {
  int n;
  int row[kMaxBiasRows];
  double coef[kMaxBiasRows];
  double u[kMaxDim];
};

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0,
                                              uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)M0 * c[0];
    uint64_t p1 = (uint64_t)M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

__device__ __forceinline__ void box_muller(uint32_t r0, uint32_t r1,
                                           double* z0, double* z1) {
  const double two_m32 = 2.3283064365386963e-10;
  const double two_pi = 6.283185307179586;
  double u1 = ((double)r0 + 0.5) * two_m32;
  double u2 = ((double)r1 + 0.5) * two_m32;
  double rad = sqrt(-2.0 * log(u1));
  double th = two_pi * u2;
  *z0 = rad * cos(th);
  *z1 = rad * sin(th);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__global__ void synth_kv_kernel(void* out, int bf16, int64_t n_groups, int D,
                                uint32_t k0, uint32_t k1, uint32_t x1,
                                uint32_t x2, uint32_t x3, double sqrt_d,
                                BiasArgs bias) {
  int64_t ge = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ge >= n_groups) return;
  uint32_t c[4] = {(uint32_t)ge, x1, x2, x3};
  philox4x32_10(c, k0, k1);
  double z[4];
  box_muller(c[0], c[1], &z[0], &z[1]);
  box_muller(c[2], c[3], &z[2], &z[3]);
  int64_t e0 = ge * 4;
  int64_t row = e0 / D;
  int d0 = (int)(e0 - row * D);
  int hit = -1;
  for (int i = 0; i < bias.n; ++i)
    if (bias.row[i] == row) hit = i;
  float f[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double x = z[i] / sqrt_d;
    if (hit >= 0) x = x + bias.coef[hit] * bias.u[d0 + i];
    f[i] = (float)x;
  }
  if (bf16) {
    uint16_t* o = (uint16_t*)out + e0;
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16_bits(f[0]) |
           ((uint32_t)f32_to_bf16_bits(f[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16_bits(f[2]) |
           ((uint32_t)f32_to_bf16_bits(f[3]) << 16);
    *(uint2*)o = pk;
  } else {
    *(float4*)((float*)out + e0) = make_float4(f[0], f[1], f[2], f[3]);
  }
}

}  // namespace

// Fill rows [0, rows) of one [rows][D] slice (D % 4 == 0, D <= 256) with the
// generator's values for counter words (x1, x2, x3) under key (k0, k1).
// bias_rows/bias_coef/u are host arrays (n_bias <= 64 rows, u of length D).
// `out` is a device pointer aligned to 16 (f32) or 8 (bf16) bytes.
// Returns 0 or a HIP error code (nothing is launched on an argument error).
extern "C" int synth_kv_fill(void* out, int kv_bf16, int rows, int D,
                             uint32_t k0, uint32_t k1, uint32_t x1,
                             uint32_t x2, uint32_t x3, double sqrt_d,
                             int n_bias, const int* bias_rows,
                             const double* bias_coef, const double* u,
                             void* stream) {
  if (!out || rows < 0 || D <= 0 || D % 4 || D > kMaxDim || n_bias < 0 ||
      n_bias > kMaxBiasRows || (n_bias && (!bias_rows || !bias_coef || !u)))
    return (int)hipErrorInvalidValue;
  BiasArgs b;
  b.n = n_bias;
  for (int i = 0; i < n_bias; ++i) {
    b.row[i] = bias_rows[i];
    b.coef[i] = bias_coef[i];
  }
  for (int d = 0; d < kMaxDim; ++d) b.u[d] = (u && d < D) ? u[d] : 0.0;
  int64_t n_groups = (int64_t)rows * D / 4;
  if (n_groups == 0) return 0;
  int64_t blocks = (n_groups + 255) / 256;
  hipLaunchKernelGGL(synth_kv_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, out, kv_bf16, n_groups, D, k0, k1,
                     x1, x2, x3, sqrt_d, b);
  return (int)hipGetLastError();
}
