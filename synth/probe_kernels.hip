// Bandwidth probes for the benchmark: a streaming read of n bytes and a
// plain copy of n bytes, both with 16-byte accesses and a grid-stride loop.
// They give the achievable HBM rate on the box and the reading of the
// hardware byte counters for a kernel whose traffic is known exactly.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(
    const u32x4 *__restrict__ src, size_t n16, uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += stride) {
    const u32x4 x = __builtin_nontemporal_load(src + i);
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
// `sink` has room for `blocks` words.  Returns 0 or a HIP error code.
extern "C" int probe_read(const void *src, size_t bytes, void *sink,
                          int blocks, void *stream) {
  if (!src || !sink || bytes % 16 || blocks < 1)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0,
                     (hipStream_t)stream, (const u32x4 *)src, bytes / 16,
                     (uint32_t *)sink);
  return (int)hipGetLastError();
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
