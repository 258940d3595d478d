// Mixture-of-experts routing around the grouped EXL3 GEMM (cuda-exl3 README,
// "What is supported": routed experts run as a grouped GEMM after the
// (token, expert) pairs are sorted by expert and each expert's run is padded
// to whole row blocks, so every block belongs to one expert; "Determinism":
// the routed rows are written and each token's top-k rows are summed in a
// fixed order in fp32, rounded once).
#include "exl3_device.hpp"
#include "exl3_launch.hpp"

namespace exl3 {

constexpr int AL_THREADS = 1024;
constexpr int AL_MAX_E = 4096;

// One workgroup.  Pairs p = t * topk + j with expert topk_ids[p] (outside
// 0..E-1: dropped, pair_row[p] = -1).  Expert e's pairs fill rows
// start[e] .. start[e] + count[e] - 1, start[e] the sum of the whole-block
// padded counts of the experts before it; padding rows and the blocks after
// the last expert's run are -1.  Within an expert's run the pairs take rows
// in arrival order (an LDS atomic), which may differ between runs: a routed
// row's values depend only on its own token and expert, and the combine
// reads through pair_row, so the results do not.
__global__ __launch_bounds__(AL_THREADS) void moe_align_kernel(const int32_t *__restrict__ topk_ids, int32_t pairs,
                                                               int32_t E, int32_t block, int32_t rows_max,
                                                               int32_t *__restrict__ row_pair,
                                                               int32_t *__restrict__ block_expert,
                                                               int32_t *__restrict__ pair_row) {
  __shared__ int32_t cnt[AL_MAX_E];    // counts, then the running row of each expert
  __shared__ int32_t start[AL_MAX_E];  // first row of each expert's run
  __shared__ int32_t wave_sum[AL_THREADS / 64];
  __shared__ int32_t total_rows;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += AL_THREADS) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < pairs; p += AL_THREADS) {
    const int e = topk_ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // padded run lengths, scanned: each thread owns a contiguous run of experts
  const int per = (E + AL_THREADS - 1) / AL_THREADS;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int sum = 0;
  for (int e = e0; e < e1; ++e) sum += (cnt[e] + block - 1) / block * block;
  // exclusive prefix of the threads' sums (integer adds, so any order gives
  // the same result): within each wave by lane shifts, then over the waves
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    constexpr int W = AL_THREADS / 64;
    int w = lane < W ? wave_sum[lane] : 0;
#pragma unroll
    for (int d = 1; d < W; d <<= 1) {
      const int t = __shfl_up(w, d, 64);
      if (lane >= d) w += t;
    }
    if (lane < W) wave_sum[lane] = w;  // inclusive over the waves
    if (lane == W - 1) total_rows = w;
  }
  __syncthreads();
  int acc = (wave > 0 ? wave_sum[wave - 1] : 0) + incl - sum;
  for (int e = e0; e < e1; ++e) {
    start[e] = acc;
    acc += (cnt[e] + block - 1) / block * block;
  }
  __syncthreads();
  const int total = total_rows;  // <= rows_max by the host's sizing
  for (int r = tid; r < rows_max; r += AL_THREADS) row_pair[r] = -1;
  const int blocks = rows_max / block;
  for (int b = total / block + tid; b < blocks; b += AL_THREADS) block_expert[b] = -1;
  for (int e = e0; e < e1; ++e) {
    const int b0 = start[e] / block, b1 = (start[e] + (cnt[e] + block - 1) / block * block) / block;
    for (int b = b0; b < b1; ++b) block_expert[b] = e;
  }
  __syncthreads();
  for (int e = tid; e < E; e += AL_THREADS) cnt[e] = start[e];
  __syncthreads();
  for (int p = tid; p < pairs; p += AL_THREADS) {
    const int e = topk_ids[p];
    int r = -1;
    if (e >= 0 && e < E) {
      r = atomicAdd(&cnt[e], 1);
      row_pair[r] = p;
    }
    pair_row[p] = r;
  }
}

// out[t][n] = rne( sum_j w[t][j] * y[pair_row[t*topk + j]][n] ), the sum in
// fp32 from 0 in j order, each term rounded to fp32 before it is added
// (dropped pairs add nothing).  Two columns per thread.
template <bool BF16>
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t *__restrict__ y, const int32_t *__restrict__ pair_row,
                                                          const float *__restrict__ w, int32_t T, int32_t topk,
                                                          int32_t N, uint16_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t half = N >> 1;
  if (idx >= (int64_t)T * half) return;
  const int64_t t = idx / half;
  const int c = (int)(idx - t * half) * 2;
  float a0 = 0.f, a1 = 0.f;
  for (int j = 0; j < topk; ++j) {
    const int32_t r = pair_row[t * topk + j];
    if (r < 0) continue;
    const float wt = w[t * topk + j];
    const uint32_t v = *(const uint32_t *)(y + (int64_t)r * N + c);
    const float v0 = BF16 ? bf16_bits_to_f32(v & 0xFFFFu) : f16_bits_to_f32(v & 0xFFFFu);
    const float v1 = BF16 ? bf16_bits_to_f32(v >> 16) : f16_bits_to_f32(v >> 16);
    a0 = keep_f32(a0 + keep_f32(wt * v0));
    a1 = keep_f32(a1 + keep_f32(wt * v1));
  }
  const uint32_t o = BF16 ? (f32_to_bf16_bits(a0) | (f32_to_bf16_bits(a1) << 16))
                          : (f32_to_f16_bits(a0) | (f32_to_f16_bits(a1) << 16));
  *(uint32_t *)(out + t * N + c) = o;
}

hipError_t launch_moe_align(const int32_t *topk_ids, int32_t pairs, int32_t E, int32_t block, int32_t rows_max,
                            int32_t *row_pair, int32_t *block_expert, int32_t *pair_row, hipStream_t s) {
  hipLaunchKernelGGL(moe_align_kernel, dim3(1), dim3(AL_THREADS), 0, s, topk_ids, pairs, E, block, rows_max,
                     row_pair, block_expert, pair_row);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void *y_routed, bool bf16, const int32_t *pair_row, const float *weights,
                              int32_t T, int32_t topk, int32_t N, void *out, hipStream_t s) {
  const int64_t threads = (int64_t)T * (N / 2);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const uint16_t *y = static_cast<const uint16_t *>(y_routed);
  uint16_t *o = static_cast<uint16_t *>(out);
  if (bf16) hipLaunchKernelGGL((moe_combine_kernel<true>), grid, dim3(256), 0, s, y, pair_row, weights, T, topk, N, o);
  else hipLaunchKernelGGL((moe_combine_kernel<false>), grid, dim3(256), 0, s, y, pair_row, weights, T, topk, N, o);
  return hipGetLastError();
}

}  // namespace exl3
