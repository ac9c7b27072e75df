// Static device scratch of the allocation-free fused call
// (alspec_spec_decode_noalloc): a file-scope device array that serves as
// that call's workspace, one copy per GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "alspec_plan.h"
#include "alspec_scratch.h"

namespace alspec {

// Zero-initialised when the code object is loaded on a device; its
// counters are cleared once more at set-up, and every call leaves them at
// zero again.  Host code never passes this name to a kernel: in host code
// it is only a stand-in for the symbol, and its device address (one per
// GPU) comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void *g_addr[kScratchMaxDevices];  // device address of `scratch`, per GPU

__global__ void zero_words_kernel(unsigned *__restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

hipError_t scratch_setup(int device, hipStream_t s, void **out) {
  *out = nullptr;
  if (device < 0 || device >= kScratchMaxDevices) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[device]) {
    *out = g_addr[device];
    return hipSuccess;
  }
  // `device` is current (the caller's set-up made it so).
  void *ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  // The workspace contract: counters start at zero.  A fill kernel (no
  // memset node) on the set-up stream, waited for here, once per device.
  const size_t words = kCounterBytes / 4;
  void *argv[] = {&ptr, (void *)&words};
  e = hipLaunchKernel((const void *)zero_words_kernel, dim3(64), dim3(256),
                      argv, 0, s);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  g_addr[device] = ptr;
  *out = ptr;
  return hipSuccess;
}

}  // namespace alspec
