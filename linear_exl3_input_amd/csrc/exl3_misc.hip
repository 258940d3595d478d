// Input rotation, ordered split-k output stage and the codebook hook.
#include "exl3_device.hpp"
#include "exl3_launch.hpp"

namespace exl3 {

// ------------------------------------------------------- input rotation
//
// x~[s][m][:] = fp16_rne(2^-4 * H128(x[m][:] * suh[s][:])) per 128 block
// (TensorFold PR "cuda: EXL3 projections behind qlinear", "Arithmetic" step
// 1).  One wave per (row, 128-block); x is read once and reused for every
// shard's suh row (cuda-exl3 README, "One op per layer": all shards in one
// launch, reading x once, with bf16 -> fp32 folded into the load).  x*suh is
// exact in fp32, so the product may be contracted into an add freely.  The
// output is stored in k-step tiles, x~[s][k/32][m][32], with the 32 values of
// a row in fragment order (frag_order_k), so that one MFMA lane's eight A
// values are 16 contiguous bytes and one k-step of a run of rows is one
// contiguous block.
template <bool X_BF16>
__global__ __launch_bounds__(256) void input_transform_kernel(const uint16_t *__restrict__ x,
                                                              const uint16_t *__restrict__ suh,
                                                              uint16_t *__restrict__ x_rot, int32_t M,
                                                              int32_t K, int32_t n_shards) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int kblocks = K >> 7;
  if (item >= (int64_t)M * kblocks) return;  // whole wave exits together
  const int64_t m = item / kblocks;
  const int k0 = (int)(item - m * kblocks) * 128 + 2 * lane;
  const uint32_t xv = *(const uint32_t *)(x + m * K + k0);
  float x0, x1;
  if constexpr (X_BF16) {
    x0 = bf16_bits_to_f32(xv & 0xFFFFu);
    x1 = bf16_bits_to_f32(xv >> 16);
  } else {
    x0 = f16_bits_to_f32(xv & 0xFFFFu);
    x1 = f16_bits_to_f32(xv >> 16);
  }
  for (int s = 0; s < n_shards; ++s) {
    const uint32_t sv = *(const uint32_t *)(suh + (int64_t)s * K + k0);
    float t0 = x0 * f16_bits_to_f32(sv & 0xFFFFu);
    float t1 = x1 * f16_bits_to_f32(sv >> 16);
    hadamard128_wave(t0, t1, lane);
    const uint32_t packed = f32_to_f16_bits(t0 * 0.0625f) | (f32_to_f16_bits(t1 * 0.0625f) << 16);
    const int64_t tile = (int64_t)s * (K >> 5) + (k0 >> 5);
    *(uint32_t *)(x_rot + (tile * M + m) * 32 + (frag_order_k(k0) & 31)) = packed;
  }
}

hipError_t launch_input_transform(const void *x, bool x_bf16, int32_t M, int32_t K, const uint16_t *suh,
                                  int32_t n_shards, uint16_t *x_rot, hipStream_t s) {
  const int64_t items = (int64_t)M * (K / 128);
  const dim3 grid((unsigned)((items + 3) / 4));
  if (x_bf16)
    hipLaunchKernelGGL((input_transform_kernel<true>), grid, dim3(256), 0, s, (const uint16_t *)x, suh, x_rot,
                       M, K, n_shards);
  else
    hipLaunchKernelGGL((input_transform_kernel<false>), grid, dim3(256), 0, s, (const uint16_t *)x, suh, x_rot,
                       M, K, n_shards);
  return hipGetLastError();
}

// ------------------------------------------------- ordered part sum + output
//
// z = the ordered sum of the partial slabs (reduce_rows4: groups of fold_q
// slabs, then the groups, each in order) in fp32, then y = rne(svh * 2^-3 *
// H128(z)) (TensorFold PR, "Arithmetic" step 3 and its ordered part sum).
// The partials are stored [slab][M4][N][4] (rows padded to a multiple of 4):
// the four rows of one column are 16 contiguous bytes, which is what a GEMM
// lane holds for one output column, so both the GEMM's stores and these
// loads move whole cache lines.  One wave per (4-row group, 128-column
// block) of rows [row_base, row_end).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void epilogue_kernel(const float *__restrict__ slabs, int32_t n_slabs,
                                                       int32_t fold_q, int32_t row_base, int32_t row_end,
                                                       int32_t N, const uint16_t *__restrict__ svh,
                                                       uint16_t *__restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nblocks = N >> 7;
  const int rows = row_end - row_base;
  const int M4 = (rows + 3) >> 2;
  if (item >= (int64_t)M4 * nblocks) return;
  const int64_t m4 = item / nblocks;
  const int n0 = (int)(item - m4 * nblocks) * 128;
  const int64_t r0 = 4 * m4;
  reduce_rows4<OUT_BF16>(slabs, n_slabs, fold_q, (int64_t)M4 * N * 4, N, m4, n0, svh, y, row_base + r0,
                         (int)min((int64_t)4, rows - r0), lane);
}

hipError_t launch_epilogue(const float *slabs, int32_t n_slabs, int32_t fold_q, int32_t row_base, int32_t row_end,
                           int32_t N, const uint16_t *svh, void *y, bool out_bf16, hipStream_t s) {
  const int64_t items = (int64_t)((row_end - row_base + 3) / 4) * (N / 128);
  const dim3 grid((unsigned)((items + 3) / 4));
  if (out_bf16)
    hipLaunchKernelGGL((epilogue_kernel<true>), grid, dim3(256), 0, s, slabs, n_slabs, fold_q, row_base, row_end, N,
                       svh, (uint16_t *)y);
  else
    hipLaunchKernelGGL((epilogue_kernel<false>), grid, dim3(256), 0, s, slabs, n_slabs, fold_q, row_base, row_end,
                       N, svh, (uint16_t *)y);
  return hipGetLastError();
}

// ------------------------------------------------------ codebook hook
//
// Every state through decode_pair, the function the GEMM's decoder uses.
template <uint32_t CB>
__global__ __launch_bounds__(256) void codebook_kernel(uint32_t *__restrict__ out) {
  const uint32_t i = blockIdx.x * 256 + threadIdx.x;  // pair index, 0..32767
  out[i] = decode_pair<CB>(2 * i, 2 * i + 1);
}

hipError_t launch_debug_codebook(int cb, uint16_t *out, hipStream_t s) {
  const dim3 grid(32768 / 256);
  switch (cb) {
    case 0: hipLaunchKernelGGL((codebook_kernel<CB_3INST>), grid, dim3(256), 0, s, (uint32_t *)out); break;
    case 1: hipLaunchKernelGGL((codebook_kernel<CB_MCG>), grid, dim3(256), 0, s, (uint32_t *)out); break;
    case 2: hipLaunchKernelGGL((codebook_kernel<CB_MUL1>), grid, dim3(256), 0, s, (uint32_t *)out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------ bit-width dispatch

hipError_t launch_gemm(int bits, int cb, int bm, int quads, bool multi, const GemmParams &p, dim3 grid,
                       hipStream_t s) {
  switch (bits) {
    case 1: return launch_gemm_b1(cb, bm, quads, multi, p, grid, s);
    case 2: return launch_gemm_b2(cb, bm, quads, multi, p, grid, s);
    case 3: return launch_gemm_b3(cb, bm, quads, multi, p, grid, s);
    case 4: return launch_gemm_b4(cb, bm, quads, multi, p, grid, s);
    case 5: return launch_gemm_b5(cb, bm, quads, multi, p, grid, s);
    case 6: return launch_gemm_b6(cb, bm, quads, multi, p, grid, s);
    case 7: return launch_gemm_b7(cb, bm, quads, multi, p, grid, s);
    case 8: return launch_gemm_b8(cb, bm, quads, multi, p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_table(int bits, int cb, const GemmParams &p, int grid, hipStream_t s) {
  switch (bits) {
    case 1: return launch_table_b1(cb, p, grid, s);
    case 2: return launch_table_b2(cb, p, grid, s);
    case 3: return launch_table_b3(cb, p, grid, s);
    case 4: return launch_table_b4(cb, p, grid, s);
    case 5: return launch_table_b5(cb, p, grid, s);
    case 6: return launch_table_b6(cb, p, grid, s);
    case 7: return launch_table_b7(cb, p, grid, s);
    case 8: return launch_table_b8(cb, p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_debug_decode(int bits, int cb, const DecodeParams &p, hipStream_t s) {
  switch (bits) {
    case 1: return launch_debug_decode_b1(cb, p, s);
    case 2: return launch_debug_decode_b2(cb, p, s);
    case 3: return launch_debug_decode_b3(cb, p, s);
    case 4: return launch_debug_decode_b4(cb, p, s);
    case 5: return launch_debug_decode_b5(cb, p, s);
    case 6: return launch_debug_decode_b6(cb, p, s);
    case 7: return launch_debug_decode_b7(cb, p, s);
    case 8: return launch_debug_decode_b8(cb, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace exl3
