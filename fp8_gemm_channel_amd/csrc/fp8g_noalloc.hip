// fp8g_noalloc.hip -- the allocation-free entry point of libfp8g.so,
// fp8_gemm_scaled_noalloc: fp8_gemm_scaled_ex for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The plans that need a workspace -- split-K with several K slices (fp32
// partials and the per-column-tile tickets) and stream-K (partial tiles and
// tickets) -- take it from `scratch`, a file-scope device array of
// FP8G_NOALLOC_SCRATCH_BYTES, instead of the library's memory pool.  Each GPU
// the library runs on holds its own copy of the array, at its own address, until
// the process ends.
//
// In host code `scratch` names a host-side stand-in, not a device address: the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept; kernels and everything else on the host side
// get that address, never the array's name.
//
// Contents between calls: nothing has to start at zero.  A ticket carries the
// id of the call that took it, so a ticket left by an earlier call (or the
// array's initial zeros) restarts at one arrival, and every partial sum is
// written before it is read.  All calls on one GPU share its array, so calls
// whose kernels overlap on one GPU (different streams, no ordering between
// them) race on it; calls must be ordered, e.g. issued on one stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fp8g.h"
#include "fp8g_internal.h"

namespace {

constexpr uint64_t kScratchBytes = (uint64_t)FP8G_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The scratch array's device address on the device `stream` runs on, looked up
// on the first call for that device.
hipError_t scratch_for(hipStream_t stream, void **out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int current = -1;
    e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t r = current != dev ? hipSetDevice(current) : hipSuccess;
    if (e != hipSuccess) return e;
    if (r != hipSuccess) return r;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

const fp8g::FixedWorkspace kScratch{kScratchBytes, scratch_for};

}  // namespace

extern "C" int fp8_gemm_scaled_noalloc(const void *x, const void *w, const float *scale, void *y, int64_t M, int64_t N,
                                       int64_t K, int32_t path, int32_t variant, int32_t split_k, void *stream) {
  return fp8g::run_fixed_workspace(x, w, scale, y, M, N, K, path, variant, split_k, stream, kScratch);
}
