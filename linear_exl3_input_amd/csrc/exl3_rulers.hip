// Measurement rulers: what this GPU's HBM and matrix cores deliver to
// simple kernels in the same run as the layer timings, so the layer kernels
// can be judged against attainable rates as well as the data-sheet peaks.
#include "exl3_device.hpp"
#include "exl3_launch.hpp"

namespace exl3 {

constexpr int RULER_WG = 256;
constexpr int RULER_GRID = RULER_THREADS / RULER_WG;

// Grid-stride streaming read: every thread keeps four 16-byte loads in
// flight per trip and XORs what it reads into one word.
__global__ __launch_bounds__(RULER_WG) void stream_read_kernel(const u32x4_t *__restrict__ buf, size_t n16,
                                                               uint32_t *__restrict__ out) {
  const size_t tid = (size_t)blockIdx.x * RULER_WG + threadIdx.x;
  const size_t stride = (size_t)RULER_THREADS;
  uint32_t x = 0;
  size_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = buf[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[tid] = x;
}

// 16 independent accumulation chains per wave (64 VGPRs), A = B = `one`
// everywhere: every MFMA adds 32 * one * one to each accumulator element.
__global__ __launch_bounds__(RULER_WG) void mfma_loop_kernel(int32_t iters, uint16_t one, float *__restrict__ out) {
  const _Float16 h = __builtin_bit_cast(_Float16, one);
  const half8_t a = {h, h, h, h, h, h, h, h};
  float4_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, acc[c], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) t += acc[c][0];
  out[(size_t)blockIdx.x * RULER_WG + threadIdx.x] = t;
}

// The same loop on operands that change from one product to the next: two
// sets of pseudo-random fp16 values (magnitudes in [0.5, 1), random signs,
// from a hash of the thread index) used alternately, so the multipliers
// toggle as they do on real data.  On this GPU the matrix cores draw more
// power then and the clock drops: this is the rate real operands can reach.
__global__ __launch_bounds__(RULER_WG) void mfma_toggle_kernel(int32_t iters, float *__restrict__ out) {
  const uint32_t tid = blockIdx.x * RULER_WG + threadIdx.x;
  half8_t a[2], b[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t x = tid * 0x9E3779B1u + (uint32_t)(s * 8 + e) * 0x85EBCA6Bu;
      x ^= x >> 15;
      x *= 0x2C1B3C6Du;
      x ^= x >> 12;
      a[s][e] = __builtin_bit_cast(_Float16, (uint16_t)((x & 0x83FFu) | 0x3800u));
      b[s][e] = __builtin_bit_cast(_Float16, (uint16_t)(((x >> 16) & 0x83FFu) | 0x3800u));
    }
  float4_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[c & 1], b[c & 1], acc[c], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) t += acc[c][0];
  out[(size_t)blockIdx.x * RULER_WG + threadIdx.x] = t;
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(RULER_GRID), dim3(RULER_WG), 0, s,
                     static_cast<const u32x4_t *>(buf), bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(int32_t iters, uint16_t one, float *out, hipStream_t s) {
  if (one == 0) hipLaunchKernelGGL(mfma_toggle_kernel, dim3(RULER_GRID), dim3(RULER_WG), 0, s, iters, out);
  else hipLaunchKernelGGL(mfma_loop_kernel, dim3(RULER_GRID), dim3(RULER_WG), 0, s, iters, one, out);
  return hipGetLastError();
}

}  // namespace exl3
