// exl3_linear_noalloc: the quantized linear for callers that cannot allocate
// (code under graph capture, serving loops that forbid hipMalloc).  Its
// split-k partials and arrival counters live in `scratch`, a device array
// of EXL3_NOALLOC_SCRATCH_BYTES that the library owns: each GPU the library
// runs on holds its own copy, at its own address, until the process ends.
//
// Host code never passes the array's name to a kernel or a copy (on the
// host that name is a stand-in, not a device address): the first call on a
// device asks the runtime for that device's address of the array
// (hipGetSymbolAddress, with the device current) and keeps it; every launch
// uses the kept address.  The array starts zeroed (the code object's
// zero-initialised data), and the first call on a device also clears the
// counters in stream order with a fill kernel (no memset node, so the call
// may be captured).  Every call leaves the counters zero again.  All calls
// on one GPU share the array: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/exl3.h"
#include "exl3_launch.hpp"

namespace exl3 {
exl3_status linear_in_scratch(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y, int32_t y_dtype,
                              void *scratch, size_t scratch_bytes, void *stream, bool launch);
exl3_status scratch_setup_error(hipError_t e, const char *what);
}  // namespace exl3

static __device__ __align__(256) uint8_t scratch[EXL3_NOALLOC_SCRATCH_BYTES];

namespace {

__global__ void clear_counters_kernel(uint32_t *__restrict__ counters, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counters[i] = 0u;
}

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];  // device address of `scratch`, per device (null: not set up)

// The device address of this device's `scratch`, set up on first use.
exl3_status scratch_for_device(void **out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return exl3::scratch_setup_error(e, "device query");
  if (dev < 0 || dev >= MAX_DEVICES) return exl3::scratch_setup_error(hipErrorInvalidDevice, "device index");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return exl3::scratch_setup_error(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch symbol address");
    constexpr int n = EXL3_WORKSPACE_COUNTER_BYTES / 4;
    hipLaunchKernelGGL(clear_counters_kernel, dim3((n + 255) / 256), dim3(256), 0, s, static_cast<uint32_t *>(p), n);
    if ((e = hipGetLastError()) != hipSuccess) return exl3::scratch_setup_error(e, "scratch clear launch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EXL3_OK;
}

// A 256-byte aligned address that stands in for the scratch while the
// arguments are checked (never dereferenced).
void *const CHECK_ONLY = reinterpret_cast<void *>(uintptr_t{1} << 20);

}  // namespace

extern "C" exl3_status exl3_linear_noalloc(const exl3_weight *w, const uint16_t *x_rot, int32_t M, void *y,
                                           int32_t y_dtype, void *stream) {
  // every argument and the schedule are checked before any device work
  exl3_status st = exl3::linear_in_scratch(w, x_rot, M, y, y_dtype, CHECK_ONLY, EXL3_NOALLOC_SCRATCH_BYTES, stream,
                                           false);
  if (st != EXL3_OK || M == 0) return st;
  void *p = nullptr;
  if ((st = scratch_for_device(&p, (hipStream_t)stream)) != EXL3_OK) return st;
  return exl3::linear_in_scratch(w, x_rot, M, y, y_dtype, p, EXL3_NOALLOC_SCRATCH_BYTES, stream, true);
}
