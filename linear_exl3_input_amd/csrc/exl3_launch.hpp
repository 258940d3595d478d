// Host-side launch interface between the C-ABI (exl3_host.cpp) and the
// kernels (the .hip files).  Plain structs of device pointers and sizes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exl3 {

constexpr int MAX_SHARDS = 16;

struct GemmParams {
  const uint16_t *trellis;  // [K/16][N/16][16*bits]
  const uint16_t *x_rot;    // [n_shards][K/32][M][32] fp16 bits (k-step tiles)
  const uint16_t *svh;      // [N] fp16 bits
  const uint16_t *dense;    // dense path: W_q as B fragments (dequant_kernel order)
  void *y;                  // [M][N] bf16/fp16
  float *slabs;             // [units][ceil(rows/4)][N][4] fp32 (slab mode)
  uint32_t *counters;       // slab mode: per-tile arrival counters (zero on
                            // entry, left zero); null: partials only
  int32_t M;                // rows of x_rot (the row stride of its k-step tiles)
  int32_t row_base;         // this launch computes rows [row_base, row_end);
  int32_t row_end;          // slab row r is row row_base + r
  int32_t K, N;
  int32_t parts;            // P K parts
  int32_t unit;             // parts per workgroup unit: a workgroup folds the
                            // parts [unit*blockIdx.y, unit*(blockIdx.y+1)) in
                            // order (fused mode: unit = P, blockIdx.y = 0)
  int32_t fold_q;           // finisher: consecutive slabs that form one group
  int32_t slab_mode;        // 1: write the unit's sum to slab blockIdx.y
  int32_t out_bf16;
  int32_t n_shards;
  int32_t shard_end_blk[MAX_SHARDS];  // exclusive end of shard s, in 128-col blocks
  // (appended last: the fields above keep their argument offsets)
  const uint16_t *bias;         // [N] fp16 added before the output rounding, or null
  const int32_t *block_expert;  // grouped (MoE) calls: expert of each row block (-1: none), else null
  int64_t expert_trellis;       // grouped calls: trellis words per expert
  int32_t n_experts;            // grouped calls: experts in the stack; a block's
                                // expert outside 0..n_experts-1 is skipped like -1
  // Rotation in the GEMM (small tiles only, exl3_forward): when x_in is set,
  // x_rot is unused and each workgroup rotates its own rows and K range of
  // x [M][K] (bf16 if x_in_bf16, else fp16) with suh_in [n_shards][K] into
  // its stage slots; the host sets it only when every stage of a quad's K
  // range fits the slots (small_tile_slots).
  const uint16_t *x_in;
  const uint16_t *suh_in;
  int32_t x_in_bf16;
};

// Stage slots per quad of the small-tile kernel (gemm_kernel): two when QD
// quads of two fit in 152 KB of LDS, else one.  Host and device use this one
// definition (the host to decide whether a quad's stages all fit the slots).
constexpr int small_tile_slots(int bits, int mt, int qw, int qd) {
  const int bm = 16 * mt, qt = 64 * qw, nts = 2 * qw;
  const int t_chunks = 8 * nts * (2 * bits + 2);
  const int t_ops = (t_chunks + qt - 1) / qt;
  const int junk = t_ops * qt - t_chunks;
  const int slot_dw = t_chunks * 4 + bm * 64;
  return qd * (2 * slot_dw + junk * 4) * 4 <= 152 * 1024 ? 2 : 1;
}

struct DecodeParams {
  const uint16_t *trellis;
  uint16_t *wq;  // [K][N] fp16 bits
  int32_t K, N;
};

// Launchers (one per bit width; codebook and rows-per-tile bm are runtime
// choices that select a template instance: bm 16/32/64 -> gemm_kernel,
// 128 -> gemm_big_kernel, 256/512 -> gemm_wide_kernel).  Return hipSuccess or the
// launch error.
hipError_t launch_gemm(int bits, int cb, int bm, int quads, bool half, bool multi_part, const GemmParams &p,
                       dim3 grid, hipStream_t s);
hipError_t launch_debug_decode(int bits, int cb, const DecodeParams &p, hipStream_t s);
// W_q as matrix-core B fragments (p.wq: K*N fp16 in the fragment order of
// dequant_kernel), and the dense GEMM over them (same arithmetic as the tile
// kernels: p.trellis unused, p.dense the fragments), 256-row tiles.
hipError_t launch_dequant(int bits, int cb, const DecodeParams &p, hipStream_t s);
// bulk_tiles: 256 x 256 column tiles of the first launch (-1: all); which:
// 1 that launch, 2 the 256 x 128 launch over the remaining blocks, 3 both.
hipError_t launch_gemm_dense(bool multi, const GemmParams &p, dim3 grid, int bulk_tiles, int which, hipStream_t s);
// Table-decode GEMM (M <= 16): `grid` persistent workgroups of 1024 threads,
// one per CU; fused (parts folded in order) or slab mode as in p.
hipError_t launch_gemm_table(int bits, int cb, const GemmParams &p, int grid, hipStream_t s);

// swiglu: x is the gate_up output [M][2K]; the rotated value is
// rne_dtype(silu(gate) * up) (see input_transform_kernel).
// row_pair / block_expert (may be null): routed rows, see Route in exl3_misc.hip.
hipError_t launch_input_transform(const void *x, bool x_bf16, bool swiglu, int32_t M, int32_t K,
                                  const uint16_t *suh, int32_t n_shards, uint16_t *x_rot, hipStream_t s,
                                  const int32_t *row_pair = nullptr, const int32_t *block_expert = nullptr,
                                  int32_t topk = 1, int32_t block = 16, int32_t n_experts = 0);
// MoE routing: alignment of (token, expert) pairs into row blocks, and the
// ordered combine of each token's routed rows (exl3_moe.hip).
hipError_t launch_moe_align(const int32_t *topk_ids, int32_t pairs, int32_t E, int32_t block, int32_t rows_max,
                            int32_t *row_pair, int32_t *block_expert, int32_t *pair_row, hipStream_t s);
hipError_t launch_moe_combine(const void *y_routed, bool bf16, const int32_t *pair_row, const float *weights,
                              int32_t T, int32_t topk, int32_t N, void *out, hipStream_t s);
// Ordered sum of n_slabs partial slabs (groups of fold_q consecutive slabs
// folded first, then the groups in order) + output transform, for rows
// [row_base, row_end) (slab row r = row row_base + r).
hipError_t launch_epilogue(const float *slabs, int32_t n_slabs, int32_t fold_q, int32_t row_base, int32_t row_end,
                           int32_t N, const uint16_t *svh, const uint16_t *bias, void *y, bool out_bf16,
                           hipStream_t s);
hipError_t launch_debug_codebook(int cb, uint16_t *out, hipStream_t s);

// Measurement rulers.  decode_rate: the tile kernels' trellis staging and
// decode alone, one XOR word per 128 x 128 block into p.wq (as uint32_t).
// stream_read: XOR of every 16-byte word of `bytes` (a multiple of 16) into
// RULER_THREADS words.  mfma_loop: `iters` rounds of 16 independent
// v_mfma_f32_16x16x32_f16 chains per wave on RULER_THREADS / 64 waves, with
// every A and B element equal to `one`; lane word = the sum of its 16
// chains' first elements.
constexpr int RULER_THREADS = 1 << 18;
hipError_t launch_decode_rate(int bits, int cb, const DecodeParams &p, hipStream_t s);
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *out, hipStream_t s);
hipError_t launch_mfma_loop(int32_t iters, uint16_t one, float *out, hipStream_t s);

// Per-bit-width entry points, defined in gemm_b<bits>.hip.
#define EXL3_DECLARE_BITS(B)                                                                  \
  hipError_t launch_gemm_b##B(int cb, int bm, int quads, bool half, bool multi_part,              \
                              const GemmParams &p, dim3 grid, hipStream_t s);                   \
  hipError_t launch_debug_decode_b##B(int cb, const DecodeParams &p, hipStream_t s);            \
  hipError_t launch_dequant_b##B(int cb, const DecodeParams &p, hipStream_t s);                 \
  hipError_t launch_decode_rate_b##B(int cb, const DecodeParams &p, hipStream_t s);             \
  hipError_t launch_table_b##B(int cb, const GemmParams &p, int grid, hipStream_t s);
EXL3_DECLARE_BITS(1)
EXL3_DECLARE_BITS(2)
EXL3_DECLARE_BITS(3)
EXL3_DECLARE_BITS(4)
EXL3_DECLARE_BITS(5)
EXL3_DECLARE_BITS(6)
EXL3_DECLARE_BITS(7)
EXL3_DECLARE_BITS(8)
#undef EXL3_DECLARE_BITS

}  // namespace exl3
