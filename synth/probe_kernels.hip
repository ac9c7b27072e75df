// Bandwidth probes for the benchmark: a streaming read of n bytes (with 1
// to 8 loads in flight per thread) and a plain copy of n bytes, both with
// 16-byte accesses and a grid-stride loop.
// They give the achievable HBM rate on the box and the reading of the
// hardware byte counters for a kernel whose traffic is known exactly.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// U loads of 16 bytes in flight per thread (U consecutive strides of the
// grid), nontemporal or plain; the remainder in a single-load loop.
template <int U, bool NT>
__global__ __launch_bounds__(256) void read_probe_kernel(
    const u32x4 *__restrict__ src, size_t n16, uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = NT ? __builtin_nontemporal_load(src + i + u * stride)
                : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 x = src[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  // one word per block keeps the loads alive
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

__global__ __launch_bounds__(256) void copy_probe_kernel(
    const uint4 *__restrict__ src, uint4 *__restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += stride)
    dst[i] = src[i];
}

}  // namespace

// src (and dst) 16-byte aligned device buffers of `bytes` (multiple of 16);
// `sink` has room for `blocks` words.  probe_read takes 1, 2, 4 or 8 loads
// in flight per thread (`unroll`), nontemporal if `nt`.  Returns 0 or a HIP
// error code.
extern "C" int probe_read(const void *src, size_t bytes, void *sink,
                          int blocks, int unroll, int nt, void *stream) {
  if (!src || !sink || bytes % 16 || blocks < 1)
    return (int)hipErrorInvalidValue;
  const u32x4 *p = (const u32x4 *)src;
  uint32_t *k = (uint32_t *)sink;
  const size_t n16 = bytes / 16;
  hipStream_t s = (hipStream_t)stream;
#define PROBE_READ(U)                                                      \
  if (unroll == U) {                                                       \
    if (nt)                                                                \
      hipLaunchKernelGGL((read_probe_kernel<U, true>), dim3(blocks),       \
                         dim3(256), 0, s, p, n16, k);                      \
    else                                                                   \
      hipLaunchKernelGGL((read_probe_kernel<U, false>), dim3(blocks),      \
                         dim3(256), 0, s, p, n16, k);                      \
    return (int)hipGetLastError();                                         \
  }
  PROBE_READ(1)
  PROBE_READ(2)
  PROBE_READ(4)
  PROBE_READ(8)
#undef PROBE_READ
  return (int)hipErrorInvalidValue;
}

extern "C" int probe_copy(const void *src, void *dst, size_t bytes,
                          int blocks, void *stream) {
  if (!src || !dst || bytes % 16 || blocks < 1)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0,
                     (hipStream_t)stream, (const uint4 *)src, (uint4 *)dst,
                     bytes / 16);
  return (int)hipGetLastError();
}
