// Static device scratch of the allocation-free fused call (defined in
// alspec_scratch.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>

namespace alspec {

// Bytes of the static scratch: the workspace of every automatic plan up to
// 64 users at the Llama-3-70B shape (14.8 MiB) fits.
constexpr size_t kScratchBytes = (size_t)16 << 20;
// GPUs whose scratch address the library keeps.
constexpr int kScratchMaxDevices = 64;

// Once per device (with `device` current): looks up the device address of
// the scratch array, clears its counters with a kernel on `s` and waits for
// it.  Later calls return the stored address.  *out is NULL for a device
// index past kScratchMaxDevices.
hipError_t scratch_setup(int device, hipStream_t s, void **out);

}  // namespace alspec
