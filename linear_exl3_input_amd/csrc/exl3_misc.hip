// Input rotation, ordered split-k output stage and the codebook hook.
#include "exl3_device.hpp"
#include "exl3_launch.hpp"
#include <type_traits>

namespace exl3 {

// ------------------------------------------------------- input rotation
//
// x~[s][m][:] = fp16_rne(2^-4 * H128(x[m][:] * suh[s][:])) per 128 block
// (TensorFold PR "cuda: EXL3 projections behind qlinear", "Arithmetic" step
// 1).  x is read once and reused for every shard's suh row (cuda-exl3 README,
// "One op per layer": all shards in one launch, reading x once, with bf16 ->
// fp32 folded into the load).  x*suh is exact in fp32.
//
// Sixteen lanes per (row, 128-block), four rows of one block per wave (or,
// below four rows, four blocks of one row); each lane rotates and stores its
// 16-byte piece of the k-step tile layout (rotate_piece in exl3_device.hpp);
// four lanes fill a row's 64-byte k-group.

// SwiGLU folded into the rotation (cuda-exl3 README, "MoE throughput"): x is
// then the gate_up layer's output [M][2K] (gate = columns 0..K-1, up =
// K..2K-1) and the rotated value is act = rne_dtype(silu(g) * u), computed
// in fp32 exactly as the unfused pair would store it.  e^x by Cody-Waite
// range reduction (ln 2 split into a 12-bit head, so n * head is exact, and
// a tail) and the degree-7 Taylor polynomial of e^r on |r| <= ln2/2, every
// step one IEEE fp32 operation in a fixed order (no contraction: keep_f32),
// so the result is reproducible bit for bit.
__device__ __forceinline__ float exp_taylor_f32(float x) {
  constexpr float LOG2E = 1.4426950408889634f;
  constexpr float LN2_HI = (float)(2839.0 / 4096.0);
  constexpr float LN2_LO = (float)(0.6931471805599453 - 2839.0 / 4096.0);
  x = x < -104.f ? -104.f : (x > 104.f ? 104.f : x);  // NaN passes through
  const float n = __builtin_rintf(keep_f32(x * LOG2E));
  const float r = keep_f32(keep_f32(x - keep_f32(n * LN2_HI)) - keep_f32(n * LN2_LO));
  float p = (float)(1.0 / 5040.0);
  p = keep_f32(keep_f32(p * r) + (float)(1.0 / 720.0));
  p = keep_f32(keep_f32(p * r) + (float)(1.0 / 120.0));
  p = keep_f32(keep_f32(p * r) + (float)(1.0 / 24.0));
  p = keep_f32(keep_f32(p * r) + (float)(1.0 / 6.0));
  p = keep_f32(keep_f32(p * r) + 0.5f);
  p = keep_f32(keep_f32(p * r) + 1.0f);
  p = keep_f32(keep_f32(p * r) + 1.0f);
  return __builtin_ldexpf(p, n != n ? 0 : (int)n);
}

template <bool X_BF16>
__device__ __forceinline__ float swiglu_act(uint32_t gbits, uint32_t ubits) {
  const float g = X_BF16 ? bf16_bits_to_f32(gbits) : f16_bits_to_f32(gbits);
  const float u = X_BF16 ? bf16_bits_to_f32(ubits) : f16_bits_to_f32(ubits);
  const float silu = g / keep_f32(1.0f + exp_taylor_f32(-g));
  const float a = keep_f32(keep_f32(silu) * u);
  return X_BF16 ? bf16_bits_to_f32(f32_to_bf16_bits(a)) : f16_bits_to_f32(f32_to_f16_bits(a));
}

// Routed rows (MoE): row m of x~ is the row of pair p = route.row_pair[m]
// (token p / topk of x; -1: a padding row, rotated as zeros), with the suh
// rows of its block's expert (suh + expert * n_shards * K); a block whose
// expert is outside 0 .. n_experts-1 rotates zeros like a padding row.
struct Route {
  const int32_t *row_pair;      // null: row m is x's row m
  const int32_t *block_expert;
  int32_t topk, block, n_experts;
};

template <bool X_BF16, bool SWIGLU, bool ROUTED>
__global__ __launch_bounds__(256) void input_transform_kernel(const uint16_t *__restrict__ x,
                                                              const uint16_t *__restrict__ suh,
                                                              uint16_t *__restrict__ x_rot, int32_t M,
                                                              int32_t K, int32_t n_shards, Route route) {
  const int lane = threadIdx.x & 63;
  const int L = lane & 15;
  const int kblocks = K >> 7;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int64_t m;
  int kb;
  bool live;
  if (M >= 4) {
    // item = (group of 4 rows, block): row 4*rg + lane/16
    const int64_t rgroups = ((int64_t)M + 3) >> 2;
    if (item >= rgroups * kblocks) return;  // whole wave exits together
    const int64_t rg = item / kblocks;
    kb = (int)(item - rg * kblocks);
    m = 4 * rg + (lane >> 4);
    live = m < M;
  } else {
    // few rows: item = (row, group of 4 blocks): block 4*bg + lane/16
    const int bgroups = (kblocks + 3) >> 2;
    if (item >= (int64_t)M * bgroups) return;
    m = item / bgroups;
    kb = 4 * (int)(item - m * bgroups) + (lane >> 4);
    live = kb < kblocks;
    kb = live ? kb : 0;
  }
  const int j = L >> 2, q = L & 3;
  const int k0 = kb * 128 + rotate_piece_k0(L);  // the lane's first k; the second run at k0 + 8
  int64_t src = m;  // x's row
  const uint16_t *suh_e = suh;
  bool zero = false;
  if (ROUTED && live) {
    const int32_t pr = route.row_pair[m];
    const int32_t e = route.block_expert[m / route.block];
    zero = pr < 0 || e < 0 || e >= route.n_experts;
    src = zero ? 0 : pr / route.topk;
    suh_e = suh + (int64_t)(zero ? 0 : e) * n_shards * K;
  }
  float xv[8];
  if constexpr (SWIGLU) {
    u32x2_t glo = {0u, 0u}, ghi = {0u, 0u}, ulo = {0u, 0u}, uhi = {0u, 0u};
    if (live && !zero) {
      const uint16_t *row = x + src * 2 * K;
      glo = *(const u32x2_t *)(row + k0);
      ghi = *(const u32x2_t *)(row + k0 + 8);
      ulo = *(const u32x2_t *)(row + K + k0);
      uhi = *(const u32x2_t *)(row + K + k0 + 8);
    }
    const uint32_t gw[4] = {glo.x, glo.y, ghi.x, ghi.y};
    const uint32_t uw[4] = {ulo.x, ulo.y, uhi.x, uhi.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[2 * i] = swiglu_act<X_BF16>(gw[i] & 0xFFFFu, uw[i] & 0xFFFFu);
      xv[2 * i + 1] = swiglu_act<X_BF16>(gw[i] >> 16, uw[i] >> 16);
    }
  } else {
    u32x2_t lo = {0u, 0u}, hi = {0u, 0u};
    if (live && !zero) {
      lo = *(const u32x2_t *)(x + src * K + k0);
      hi = *(const u32x2_t *)(x + src * K + k0 + 8);
    }
    const uint32_t w[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[2 * i] = X_BF16 ? bf16_bits_to_f32(w[i] & 0xFFFFu) : f16_bits_to_f32(w[i] & 0xFFFFu);
      xv[2 * i + 1] = X_BF16 ? bf16_bits_to_f32(w[i] >> 16) : f16_bits_to_f32(w[i] >> 16);
    }
  }
  for (int s = 0; s < n_shards; ++s) {
    const u32x2_t slo = *(const u32x2_t *)(suh_e + (int64_t)s * K + k0);
    const u32x2_t shi = *(const u32x2_t *)(suh_e + (int64_t)s * K + k0 + 8);
    const uint32_t sw[4] = {slo.x, slo.y, shi.x, shi.y};
    const u32x4_t o = rotate_piece(xv, sw, L);
    if (live) {
      const int64_t tile = (int64_t)s * (K >> 5) + kb * 4 + j;
      *(u32x4_t *)(x_rot + (tile * M + m) * 32 + 8 * q) = o;
    }
  }
}

hipError_t launch_input_transform(const void *x, bool x_bf16, bool swiglu, int32_t M, int32_t K,
                                  const uint16_t *suh, int32_t n_shards, uint16_t *x_rot, hipStream_t s,
                                  const int32_t *row_pair, const int32_t *block_expert, int32_t topk,
                                  int32_t block, int32_t n_experts) {
  const int64_t items = M >= 4 ? (((int64_t)M + 3) / 4) * (K / 128) : (int64_t)M * ((K / 128 + 3) / 4);
  const dim3 grid((unsigned)((items + 3) / 4));
  const uint16_t *xp = static_cast<const uint16_t *>(x);
  const Route r{row_pair, block_expert, topk, block, n_experts};
  const dim3 b(256);
  const int sel = (x_bf16 ? 4 : 0) | (swiglu ? 2 : 0) | (row_pair != nullptr ? 1 : 0);
  switch (sel) {
    case 0: hipLaunchKernelGGL((input_transform_kernel<false, false, false>), grid, b, 0, s, xp, suh, x_rot, M, K, n_shards, r); break;
    case 1: hipLaunchKernelGGL((input_transform_kernel<false, false, true>), grid, b, 0, s, xp, suh, x_rot, M, K, n_shards, r); break;
    case 2: hipLaunchKernelGGL((input_transform_kernel<false, true, false>), grid, b, 0, s, xp, suh, x_rot, M, K, n_shards, r); break;
    case 3: hipLaunchKernelGGL((input_transform_kernel<false, true, true>), grid, b, 0, s, xp, suh, x_rot, M, K, n_shards, r); break;
    case 4: hipLaunchKernelGGL((input_transform_kernel<true, false, false>), grid, b, 0, s, xp, suh, x_rot, M, K, n_shards, r); break;
    case 5: hipLaunchKernelGGL((input_transform_kernel<true, false, true>), grid, b, 0, s, xp, suh, x_rot, M, K, n_shards, r); break;
    case 6: hipLaunchKernelGGL((input_transform_kernel<true, true, false>), grid, b, 0, s, xp, suh, x_rot, M, K, n_shards, r); break;
    default: hipLaunchKernelGGL((input_transform_kernel<true, true, true>), grid, b, 0, s, xp, suh, x_rot, M, K, n_shards, r); break;
  }
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
// block) of rows [row_base, row_end).  U slabs' loads are in flight per round
// trip.  A launch of at most 64 rows has a few waves per column block, each
// waiting out its trips one after another: the launcher picks the smallest
// of 8, 16, 24 that covers every slab (one trip up to 24 slabs).  Larger
// launches are bandwidth-bound and take U = 2: fewer registers, so more
// waves per SIMD keep loads in flight (measured at 128-512 rows on 5, 8 and
// 17 slabs: U = 2 or 3 fastest, 5-12% ahead of U = 8).
template <bool OUT_BF16, int U>
__global__ __launch_bounds__(256) void epilogue_kernel(const float *__restrict__ slabs, int32_t n_slabs,
                                                       int32_t fold_q, int32_t row_base, int32_t row_end,
                                                       int32_t N, const uint16_t *__restrict__ svh,
                                                       uint16_t *__restrict__ y, const uint16_t *__restrict__ bias) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nblocks = N >> 7;
  const int rows = row_end - row_base;
  const int M4 = (rows + 3) >> 2;
  if (item >= (int64_t)M4 * nblocks) return;
  const int64_t m4 = item / nblocks;
  const int n0 = (int)(item - m4 * nblocks) * 128;
  const int64_t r0 = 4 * m4;
  reduce_rows4<OUT_BF16, U>(slabs, n_slabs, fold_q, (int64_t)M4 * N * 4, N, m4, n0, svh, bias, y, row_base + r0,
                         (int)min((int64_t)4, rows - r0), lane);
}

hipError_t launch_epilogue(const float *slabs, int32_t n_slabs, int32_t fold_q, int32_t row_base, int32_t row_end,
                           int32_t N, const uint16_t *svh, const uint16_t *bias, void *y, bool out_bf16,
                           hipStream_t s) {
  const int64_t items = (int64_t)((row_end - row_base + 3) / 4) * (N / 128);
  const dim3 grid((unsigned)((items + 3) / 4));
  auto go = [&](auto bf16_c, auto u_c) {
    hipLaunchKernelGGL((epilogue_kernel<decltype(bf16_c)::value, decltype(u_c)::value>), grid, dim3(256), 0, s, slabs,
                       n_slabs, fold_q, row_base, row_end, N, svh, (uint16_t *)y, bias);
  };
  using T = std::true_type;
  using F = std::false_type;
  using U2 = std::integral_constant<int, 2>;
  using U8 = std::integral_constant<int, 8>;
  using U16 = std::integral_constant<int, 16>;
  using U24 = std::integral_constant<int, 24>;
  if (row_end - row_base > 64) out_bf16 ? go(T{}, U2{}) : go(F{}, U2{});
  else if (n_slabs <= 8) out_bf16 ? go(T{}, U8{}) : go(F{}, U8{});
  else if (n_slabs <= 16) out_bf16 ? go(T{}, U16{}) : go(F{}, U16{});
  else out_bf16 ? go(T{}, U24{}) : go(F{}, U24{});
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

hipError_t launch_gemm(int bits, int cb, int bm, int quads, bool half, bool multi, const GemmParams &p, dim3 grid,
                       hipStream_t s) {
  switch (bits) {
    case 1: return launch_gemm_b1(cb, bm, quads, half, multi, p, grid, s);
    case 2: return launch_gemm_b2(cb, bm, quads, half, multi, p, grid, s);
    case 3: return launch_gemm_b3(cb, bm, quads, half, multi, p, grid, s);
    case 4: return launch_gemm_b4(cb, bm, quads, half, multi, p, grid, s);
    case 5: return launch_gemm_b5(cb, bm, quads, half, multi, p, grid, s);
    case 6: return launch_gemm_b6(cb, bm, quads, half, multi, p, grid, s);
    case 7: return launch_gemm_b7(cb, bm, quads, half, multi, p, grid, s);
    case 8: return launch_gemm_b8(cb, bm, quads, half, multi, p, grid, s);
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

hipError_t launch_dequant(int bits, int cb, const DecodeParams &p, hipStream_t s) {
  switch (bits) {
    case 1: return launch_dequant_b1(cb, p, s);
    case 2: return launch_dequant_b2(cb, p, s);
    case 3: return launch_dequant_b3(cb, p, s);
    case 4: return launch_dequant_b4(cb, p, s);
    case 5: return launch_dequant_b5(cb, p, s);
    case 6: return launch_dequant_b6(cb, p, s);
    case 7: return launch_dequant_b7(cb, p, s);
    case 8: return launch_dequant_b8(cb, p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_rate(int bits, int cb, const DecodeParams &p, hipStream_t s) {
  switch (bits) {
    case 1: return launch_decode_rate_b1(cb, p, s);
    case 2: return launch_decode_rate_b2(cb, p, s);
    case 3: return launch_decode_rate_b3(cb, p, s);
    case 4: return launch_decode_rate_b4(cb, p, s);
    case 5: return launch_decode_rate_b5(cb, p, s);
    case 6: return launch_decode_rate_b6(cb, p, s);
    case 7: return launch_decode_rate_b7(cb, p, s);
    case 8: return launch_decode_rate_b8(cb, p, s);
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
