// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// the C ABI's host code makes, so that the host code (argument checks, the
// shape-only part rule, the planner, the tuner's table, workspace and row
// chunk arithmetic) can be built and run on a CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Launchers record the grid they were given and
// check it against the limits of a real launch; nothing touches memory.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "../../linear_exl3_input_amd/csrc/exl3_launch.hpp"

long g_launches = 0;

namespace {
void check_grid(const char *what, dim3 g) {
  ++g_launches;
  if (g.x == 0 || g.y == 0 || g.z == 0 || g.x > 0x7fffffffu || g.y > 65535u || g.z > 65535u) {
    std::fprintf(stderr, "%s: grid (%u, %u, %u) outside the launch limits\n", what, g.x, g.y, g.z);
    std::abort();
  }
}
}  // namespace

namespace exl3 {
hipError_t launch_gemm(int, int, int bm, int, bool, bool, const GemmParams &p, dim3 grid, hipStream_t) {
  if (p.row_end <= p.row_base || p.row_end > p.M || bm <= 0) std::abort();
  check_grid("gemm", grid);
  return hipSuccess;
}
hipError_t launch_debug_decode(int, int, const DecodeParams &, hipStream_t) { return hipSuccess; }
hipError_t launch_dequant(int, int, const DecodeParams &p, hipStream_t) {
  check_grid("dequant", dim3(p.N / 128, p.K / 128));
  return hipSuccess;
}
hipError_t launch_gemm_dense(bool multi, const GemmParams &p, dim3 grid, int bulk_tiles, int which, hipStream_t) {
  if (p.row_end <= p.row_base || p.row_end > p.M) std::abort();
  if (which < 1 || which > 3 || (!multi && bulk_tiles < 0)) std::abort();
  check_grid("dense", grid);
  return hipSuccess;
}
hipError_t launch_gemm_table(int, int, const GemmParams &, int grid, hipStream_t) {
  check_grid("table", dim3(grid));
  return hipSuccess;
}
hipError_t launch_input_transform(const void *, bool, bool, int32_t M, int32_t K, const uint16_t *, int32_t, uint16_t *,
                                  hipStream_t, const int32_t *, const int32_t *, int32_t, int32_t, int32_t) {
  if (M <= 0 || K <= 0) std::abort();
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_moe_align(const int32_t *, int32_t, int32_t, int32_t, int32_t, int32_t *, int32_t *, int32_t *,
                            hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_moe_combine(const void *, bool, const int32_t *, const float *, int32_t, int32_t, int32_t, void *,
                              hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_epilogue(const float *, int32_t n_slabs, int32_t fold_q, int32_t row_base, int32_t row_end, int32_t,
                           const uint16_t *, const uint16_t *, void *, bool, hipStream_t) {
  if (n_slabs <= 0 || fold_q <= 0 || n_slabs % fold_q || row_end <= row_base) std::abort();
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_debug_codebook(int, uint16_t *, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_rate(int, int, const DecodeParams &, hipStream_t) { return hipSuccess; }
hipError_t launch_stream_read(const void *, size_t, uint32_t *, hipStream_t) { return hipSuccess; }
hipError_t launch_mfma_loop(int32_t, uint16_t, float *, hipStream_t) { return hipSuccess; }
}  // namespace exl3

// The runtime calls the host code makes: one device of 256 compute units,
// never capturing; events are not available (the tuner refuses cleanly).
extern "C" {
hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *s) {
  *s = hipStreamCaptureStatusNone;
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t *) { return hipErrorNotSupported; }
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipErrorNotSupported; }
hipError_t hipEventElapsedTime(float *, hipEvent_t, hipEvent_t) { return hipErrorNotSupported; }
const char *hipGetErrorString(hipError_t) { return "stubbed runtime"; }
}
