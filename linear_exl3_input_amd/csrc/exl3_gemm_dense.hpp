// Dense GEMM over dequantized B fragments, for large batches on gfx950.
//
// At a few hundred rows and more the trellis decode inside the tile kernels
// (about five VALU instructions per weight, interleaved with the matrix-core
// work and the LDS traffic of the rotated activations) keeps the matrix core
// busy well under half the time.  Decoding the layer once into fp16 B
// fragments (dequant_kernel: K*N*2 bytes of workspace) and then running a
// plain MFMA GEMM over them takes the decode out of the loop.  Every MFMA
// multiplies the same A and B fragments (same lanes, same k slots) in the
// same k-step order, and the K parts are folded the same way, so the result
// has the same bits as the decoding kernels.
//
// Tile: 256 rows x 128 columns on 8 waves, two per SIMD, so each wave has at
// most 256 registers and the compiler keeps the accumulators in ordinary
// VGPRs (with 4 waves and 512 registers a wave it moved them through the
// accumulation registers with copies around every MFMA, a third of the
// matrix-core rate).  Wave w = 2*rw + cw owns rows 64*rw .. +63 (A fragments
// 4rw .. 4rw+3) and the 64 columns of B fragments 4cw .. 4cw+3 (fragment
// f = 2w' + h is column half h of n-tiles 2w', 2w'+1): per 32-k step it
// reads 4 A and 4 B fragments from LDS and issues 16 MFMAs into 64
// accumulators (64 more hold the part fold).  Both operands arrive by
// direct-to-LDS loads into a ring of DN_PF k-step slots (16 KB of x~ rows
// m0 .. m0+255, contiguous in the k-step tile layout, and the block's 8 KB of
// fragments, contiguous in the dequantized layout), in lane order, so every
// LDS read is one conflict-free ds_read_b128.  Per k-step: wait for the next
// k-step's loads, one barrier, issue the loads of the k-step DN_PF ahead into
// the slot just consumed, read the next k-step's fragments into the second
// register set, then the 16 MFMAs on the first.
#pragma once

#include "exl3_gemm.hpp"

namespace exl3 {

constexpr int DN_THREADS = 512;
constexpr int DN_BM = 256;
constexpr int DN_PF = 6;                          // ring slots, k-steps in flight
constexpr int DN_A_DW = 16 * 256;                 // 16 fragments of 16 rows: 16 KB
constexpr int DN_B_DW = 8 * 256;                  // 8 fragments: 8 KB
constexpr int DN_SLOT_DW = DN_A_DW + DN_B_DW;
constexpr int DN_LOADS = DN_SLOT_DW / DN_THREADS / 4;  // 16-byte loads per lane per k-step (3)

// Tile order.  Workgroups go to the 8 XCDs (each with its own L2) in turn:
// workgroup L runs on XCD L % 8.  Each XCD takes a contiguous range of the
// tile order, and the order runs through up to 8 row tiles of one column
// block before the next block, so the row tiles that read the same B block
// run together on one XCD and share its L2 (and the workgroups an XCD holds
// at a time read the same few x~ row tiles).  A bijection for any count;
// only the speed depends on the dispatch order.
__device__ __forceinline__ void dense_tile(int L, int total, int mtiles, int &nb, int &mt) {
  const int q = total >> 3, r = total & 7, x = L & 7;
  const int T = x * q + (x < r ? x : r) + (L >> 3);
  const int nblk = total / mtiles;
  const int g = T / (nblk * 8);             // group of 8 row tiles
  const int gs = mtiles - 8 * g < 8 ? mtiles - 8 * g : 8;
  const int rem = T - g * nblk * 8;
  nb = rem / gs;
  mt = 8 * g + rem % gs;
}

// nb0: the first column block of the launch (a launch that covers the
// blocks after a 256 x 256 launch's, see launch_gemm_dense).
template <bool MULTI>
__global__ __launch_bounds__(DN_THREADS, 1) void gemm_dense_kernel(const GemmParams p, int nb0) {
  constexpr int PF = DN_PF;
  constexpr int MAIN_DW = PF * DN_SLOT_DW;
  constexpr int Z_DW = 64 * Z_ROW;
  constexpr int LDS_DW = MAIN_DW > Z_DW ? MAIN_DW : Z_DW;
  static_assert(LDS_DW * 4 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint32_t lds[LDS_DW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = wave >> 1;
  const int cw = wave & 1;
  const int j = lane & 15;
  const int g = lane >> 4;
  int nb, mt;
  dense_tile(blockIdx.x, gridDim.x, (p.row_end - p.row_base + DN_BM - 1) / DN_BM, nb, mt);
  nb += nb0;
  const int m0 = p.row_base + mt * DN_BM;
  const int rend = p.row_end;
  const int M = p.M, K = p.K, N = p.N;
  const int KB = K >> 7;
  const int nblk = N >> 7;

  const int p_begin = blockIdx.y * p.unit;
  const int p_end = p_begin + p.unit;
  const int kb_begin = (int)((int64_t)p_begin * KB / p.parts);
  const int kb_end = (int)((int64_t)p_end * KB / p.parts);
  const int ks_begin = 4 * kb_begin;
  const int nks = 4 * (kb_end - kb_begin);

  int shard = 0;
  while (shard + 1 < p.n_shards && nb >= p.shard_end_blk[shard]) ++shard;
  const uint16_t *__restrict__ xs = p.x_rot + (int64_t)shard * M * K;

  // Load sources (16-bit words).  A: the lane's chunk of fragment 8r + wave
  // of a k-step: row 16(8r + wave) + (lane & 15), 16-byte piece lane >> 4
  // (rows past the launch's last load that row: finite, never stored).  B:
  // chunk 64 wave + lane of the block's 8 KB.
  uint32_t a_src[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    int row = m0 + 16 * (8 * r + wave) + (lane & 15);
    row = row < rend ? row : rend - 1;
    a_src[r] = (uint32_t)(row * 32 + 8 * (lane >> 4));
  }
  auto issue = [&](int ks, int slot) __attribute__((always_inline)) {
    const int kk = ks_begin + (ks < nks ? ks : nks - 1);
    uint32_t *const sl = lds + slot * DN_SLOT_DW;
    const uint16_t *const abase = xs + (int64_t)kk * M * 32;
#pragma unroll
    for (int r = 0; r < 2; ++r)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(abase + a_src[r]),
                                       (__attribute__((address_space(3))) void *)(sl + (8 * r + wave) * 256), 16, 0,
                                       0);
    const uint16_t *const bbase = p.dense + ((int64_t)kk * nblk + nb) * (8 * 64 * 8);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(bbase + (wave * 64 + lane) * 8),
                                     (__attribute__((address_space(3))) void *)(sl + DN_A_DW + wave * 256), 16, 0, 0);
  };

  half8_t A[2][4], B[2][4];
  auto read_frags = [&](int ks, int set) __attribute__((always_inline)) {
    const uint32_t *const sl = lds + (ks % PF) * DN_SLOT_DW + 4 * lane;
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) B[set][fi] = *(const half8_t *)(sl + DN_A_DW + (4 * cw + fi) * 256);
#pragma unroll
    for (int m = 0; m < 4; ++m) A[set][m] = *(const half8_t *)(sl + (4 * rw + m) * 256);
  };

  float4_t acc[4][4];
  float4_t tot[MULTI ? 4 : 1][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) acc[m][fi] = float4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < PF; ++i) issue(i, i);
  wait_vmcnt<DN_LOADS * (PF - 1)>();  // k-step 0 landed
  barrier_lds();
  read_frags(0, 0);

  // part boundaries (in k-steps from ks_begin): part q ends at block
  // floor((q+1)*KB/P); the first part's sum is copied, later ones added
  int part = p_begin;
  int part_end = 4 * ((int)((int64_t)(part + 1) * KB / p.parts) - kb_begin);

  auto step = [&](int i, auto set_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(set_c)::value;
    wait_vmcnt<DN_LOADS * (PF - 2)>();  // k-step i+1 landed
    barrier_lds();                        // ... for every wave; slot i % PF is free
    issue(i + PF, i % PF);
    if (i + 1 < nks) read_frags(i + 1, cur ^ 1);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
        acc[m][fi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[cur][m], B[cur][fi], acc[m][fi], 0, 0, 0);
    if constexpr (MULTI) {
      if (i + 1 == part_end) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int fi = 0; fi < 4; ++fi) {
            tot[m][fi] = part == p_begin ? acc[m][fi] : tot[m][fi] + acc[m][fi];
            acc[m][fi] = float4_t{0.f, 0.f, 0.f, 0.f};
          }
        ++part;
        part_end = 4 * ((int)((int64_t)(part + 1) * KB / p.parts) - kb_begin);
      }
    }
  };
  // nks is a multiple of 4: two k-steps per trip keep the register sets static
  for (int i = 0; i < nks; i += 2) {
    step(i, std::integral_constant<int, 0>{});
    step(i + 1, std::integral_constant<int, 1>{});
  }
  if constexpr (MULTI) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int fi = 0; fi < 4; ++fi) acc[m][fi] = tot[m][fi];
  }
  wait_vmcnt<0>();  // the clamped tail loads land before LDS is reused
  barrier_lds();

  // lane's column (within the block) of acc[.][fi]: fragment f = 4cw + fi is
  // column half f & 1 of n-tiles 2(f >> 1), 2(f >> 1) + 1
  int col[4];
#pragma unroll
  for (int fi = 0; fi < 4; ++fi) col[fi] = lane_col((4 * cw + fi) >> 1, j, (4 * cw + fi) & 1);

  if (p.slab_mode) {
    const int rows = rend - p.row_base;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
        store_partial(p.slabs, blockIdx.y, rows, N, m0 - p.row_base + 64 * rw + 16 * m + 4 * g, nb * 128 + col[fi],
                      acc[m][fi]);
    return;
  }

  // output transform, 64 rows (one row of waves) per pass through LDS
  const OutWords16 ow = out_words16(p.svh, p.bias, nb * 128, lane);
  float *z = reinterpret_cast<float *>(lds);
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (pass > 0) barrier_lds();
    if (rw == pass) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
#pragma unroll
          for (int e = 0; e < 4; ++e) z[(m * 16 + 4 * g + e) * Z_ROW + col[fi]] = acc[m][fi][e];
    }
    barrier_lds();
    if (p.out_bf16) output_rows8<true>(z, Z_ROW, 8 * wave, ow, p.bias != nullptr, y, m0 + pass * 64 + 8 * wave, rend, N,
                                       nb * 128, lane);
    else output_rows8<false>(z, Z_ROW, 8 * wave, ow, p.bias != nullptr, y, m0 + pass * 64 + 8 * wave, rend, N,
                             nb * 128, lane);
  }
}

// Wide tiles for one part per workgroup (one K part, or slab mode with one
// part per slab): 256 rows x 256 columns (two column blocks of one shard) on
// 8 waves, two per SIMD; wave w = 4 rw + cw owns rows 128 rw .. +127 (A
// fragments 8 rw .. 8 rw + 7) and the 64 columns of fragments 4 (cw & 1) ..
// +3 of column block cw >> 1: per 32-k step 8 A and 4 B fragment reads and 32
// MFMAs into 128 accumulators.  Against 64 x 64 wave tiles on a 256 x 128
// tile, each product needs a quarter less LDS reading, each k-step's
// operand loads serve twice the products, and a barrier comes every 32
// products instead of 16; the 128 accumulators leave no room for a second
// set, so units of several parts keep gemm_dense_kernel.  The accumulators
// live in accumulation registers (mfma_acc).  A shard with an odd number of
// column blocks ends in a one-block tile whose second half is computed on a
// copy of the first block's fragments and never stored.  Same fragments,
// same k order and same chains as every other kernel, so the same bits.
__device__ __forceinline__ void mfma_acc(float4_t &acc, const half8_t &a, const half8_t &b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Reads of asm-product accumulators by vector instructions wait here: the
// compiler cannot see an asm product's latency (eight passes, plus the
// accumulator-read hazard); 24 wait states cover both.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

constexpr int DW_THREADS = 512;
constexpr int DW_PF = 4;                               // ring slots
constexpr int DW_A_DW = 16 * 256;                      // 16 A fragments: 16 KB
constexpr int DW_B_DW = 16 * 256;                      // 2 blocks x 8 B fragments: 16 KB
constexpr int DW_SLOT_DW = DW_A_DW + DW_B_DW;
constexpr int DW_LOADS = DW_SLOT_DW / DW_THREADS / 4;  // 16-byte loads per lane per k-step (4)

// Column tiles of the wide kernel: each shard's blocks in pairs, an odd
// shard ending in a one-block tile.  Tile t -> first block, blocks (1 or 2),
// shard.
__device__ __forceinline__ void wide_col_tile(const GemmParams &p, int t, int &nb, int &nbk, int &shard) {
  int start = 0;
  shard = 0;
  for (int s = 0; s < p.n_shards; ++s) {
    const int end = p.shard_end_blk[s];
    const int tiles = (end - start + 1) >> 1;
    if (t < tiles || s == p.n_shards - 1) {
      nb = start + 2 * t;
      nbk = end - nb >= 2 ? 2 : 1;
      shard = s;
      return;
    }
    t -= tiles;
    start = end;
  }
}

__global__ __launch_bounds__(DW_THREADS, 1) void gemm_dense_wide_kernel(const GemmParams p, int col_tiles) {
  constexpr int PF = DW_PF;
  constexpr int MAIN_DW = PF * DW_SLOT_DW;
  constexpr int Z_DW = DN_BM * Z_ROW;  // one column block of the tile, all rows
  constexpr int LDS_DW = MAIN_DW > Z_DW ? MAIN_DW : Z_DW;
  static_assert(LDS_DW * 4 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint32_t lds[LDS_DW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = wave >> 2;
  const int cw = wave & 3;
  const int j = lane & 15;
  const int g = lane >> 4;
  int ct, mt;
  dense_tile(blockIdx.x, gridDim.x, (p.row_end - p.row_base + DN_BM - 1) / DN_BM, ct, mt);
  (void)col_tiles;
  int nb, nbk, shard;
  wide_col_tile(p, ct, nb, nbk, shard);
  const int m0 = p.row_base + mt * DN_BM;
  const int rend = p.row_end;
  const int M = p.M, K = p.K, N = p.N;
  const int KB = K >> 7;
  const int nblk = N >> 7;

  // one part: blockIdx.y (slab mode, one part per slab) or all of K
  const int part = blockIdx.y;
  const int kb_begin = (int)((int64_t)part * KB / p.parts);
  const int kb_end = (int)((int64_t)(part + 1) * KB / p.parts);
  const int ks_begin = 4 * kb_begin;
  const int nks = 4 * (kb_end - kb_begin);

  const uint16_t *__restrict__ xs = p.x_rot + (int64_t)shard * M * K;
  // the second block of a one-block tile reads the first block's fragments
  const int b_second = nbk == 2 ? 8 * 64 * 8 : 0;

  uint32_t a_src[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    int row = m0 + 16 * (8 * r + wave) + (lane & 15);
    row = row < rend ? row : rend - 1;
    a_src[r] = (uint32_t)(row * 32 + 8 * (lane >> 4));
  }
  // load q (0..3) of a k-step: A fragments wave and wave + 8, then the B
  // fragments wave of each column block
  auto issue_one = [&](int ks, int slot, int q) __attribute__((always_inline)) {
    const int kk = ks_begin + (ks < nks ? ks : nks - 1);
    uint32_t *const sl = lds + slot * DW_SLOT_DW;
    if (q < 2) {
      const uint16_t *const abase = xs + (int64_t)kk * M * 32;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(abase + a_src[q]),
                                       (__attribute__((address_space(3))) void *)(sl + (8 * q + wave) * 256), 16, 0,
                                       0);
    } else {
      const uint16_t *const bbase = p.dense + ((int64_t)kk * nblk + nb) * (8 * 64 * 8);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void *)(bbase + (q - 2) * b_second + (wave * 64 + lane) * 8),
          (__attribute__((address_space(3))) void *)(sl + DW_A_DW + (8 * (q - 2) + wave) * 256), 16, 0, 0);
    }
  };
  auto issue = [&](int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_one(ks, slot, q);
  };

  half8_t A[2][8], B[2][4];
  // fragment reads in three parts: B, then A 0..3, then A 4..7
  auto read_part = [&](int ks, int set, int part) __attribute__((always_inline)) {
    const uint32_t *const sl = lds + (ks % PF) * DW_SLOT_DW + 4 * lane;
    if (part == 0) {
#pragma unroll
      for (int fi = 0; fi < 4; ++fi) B[set][fi] = *(const half8_t *)(sl + DW_A_DW + (4 * cw + fi) * 256);
    } else {
#pragma unroll
      for (int m = 4 * (part - 1); m < 4 * part; ++m) A[set][m] = *(const half8_t *)(sl + (8 * rw + m) * 256);
    }
  };
  auto read_frags = [&](int ks, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int part = 0; part < 3; ++part) read_part(ks, set, part);
  };

  float4_t acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) acc[m][fi] = float4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < PF; ++i) issue(i, i);
  wait_vmcnt<DW_LOADS * (PF - 1)>();  // k-step 0 landed
  barrier_lds();
  read_frags(0, 0);

  // Each k-step's 32 products run in four groups of eight; one of the k-step's
  // four direct loads and a part of the next k-step's fragment reads go out
  // between groups, so no wave stalls on a burst of load issue before its
  // products (a direct load of 64 x 16 bytes is slow to issue).
  auto step = [&](int i, auto set_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(set_c)::value;
    wait_vmcnt<DW_LOADS * (PF - 2)>();  // k-step i+1 landed
    barrier_lds();                        // ... for every wave; slot i % PF is free
    const bool more = i + 1 < nks;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      issue_one(i + PF, i % PF, q);
      if (q < 3 && more) read_part(i + 1, cur ^ 1, q);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 2 * q; m < 2 * q + 2; ++m)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) mfma_acc(acc[m][fi], A[cur][m], B[cur][fi]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // nks is a multiple of 4: two k-steps per trip keep the register sets static
  for (int i = 0; i < nks; i += 2) {
    step(i, std::integral_constant<int, 0>{});
    step(i + 1, std::integral_constant<int, 1>{});
  }
  mfma_drain();
  wait_vmcnt<0>();  // the clamped tail loads land before LDS is reused
  barrier_lds();

  const int cb_w = cw >> 1;  // the wave's column block within the tile
  int col[4];
#pragma unroll
  for (int fi = 0; fi < 4; ++fi) col[fi] = lane_col((4 * (cw & 1) + fi) >> 1, j, (4 * (cw & 1) + fi) & 1);

  if (p.slab_mode) {
    if (cb_w < nbk) {
      const int rows = rend - p.row_base;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
          store_partial(p.slabs, part, rows, N, m0 - p.row_base + 128 * rw + 16 * m + 4 * g,
                        (nb + cb_w) * 128 + col[fi], acc[m][fi]);
    }
    return;
  }

  // output transform through LDS, one column block (all 256 rows) per pass:
  // the four waves of the block write their accumulators, then every wave
  // runs the output stage on 32 rows, eight at a time (output_rows8)
  float *z = reinterpret_cast<float *>(lds);
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
  const bool has_bias = p.bias != nullptr;
  for (int cb = 0; cb < nbk; ++cb) {
    const int n0 = (nb + cb) * 128;
    const OutWords16 w = out_words16(p.svh, p.bias, n0, lane);
    if (cb > 0) barrier_lds();
    if (cb_w == cb) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
#pragma unroll
          for (int e = 0; e < 4; ++e) z[(128 * rw + 16 * m + 4 * g + e) * Z_ROW + col[fi]] = acc[m][fi][e];
    }
    barrier_lds();
#pragma unroll
    for (int r0 = 8 * wave; r0 < DN_BM; r0 += 8 * 8) {
      if (p.out_bf16) output_rows8<true>(z, Z_ROW, r0, w, has_bias, y, m0 + r0, rend, N, n0, lane);
      else output_rows8<false>(z, Z_ROW, r0, w, has_bias, y, m0 + r0, rend, N, n0, lane);
    }
  }
}

int wide_col_tiles(const GemmParams &p) {
  int start = 0, tiles = 0;
  for (int s = 0; s < p.n_shards; ++s) {
    tiles += (p.shard_end_blk[s] - start + 1) >> 1;
    start = p.shard_end_blk[s];
  }
  return tiles;
}

// The first column block of 256 x 256 column tile t (wide_col_tile's order).
static int wide_tile_first_block(const GemmParams &p, int t) {
  int start = 0;
  for (int s = 0; s < p.n_shards; ++s) {
    const int end = p.shard_end_blk[s];
    const int tiles = (end - start + 1) >> 1;
    if (t < tiles) return start + 2 * t;
    t -= tiles;
    start = end;
  }
  return start;
}

hipError_t launch_gemm_dense(bool multi, const GemmParams &p, dim3 grid, int bulk_tiles, int which, hipStream_t s) {
  // grid: (column blocks x row tiles, units).  Several parts a unit: the
  // 256 x 128 kernel.  Else the 256 x 256 kernel on column tiles
  // 0 .. bulk_tiles-1 (which & 1), and the 256 x 128 kernel on the column
  // blocks after them (which & 2): the host sizes the first launch to whole
  // rounds of workgroups over the CUs and gives the rest of the columns to
  // the narrower tiles, twice as many workgroups of half the work each.
  // Columns only split: every output element keeps the same products in
  // the same order, so the bits do not depend on the split.
  if (multi) {
    if (which & 1) hipLaunchKernelGGL((gemm_dense_kernel<true>), grid, dim3(DN_THREADS), 0, s, p, 0);
    return hipGetLastError();
  }
  const int ct = wide_col_tiles(p);
  const int nblk = p.N / 128;
  const int mtiles = (int)grid.x / nblk;
  const int bt = bulk_tiles < 0 || bulk_tiles > ct ? ct : bulk_tiles;
  if ((which & 1) && bt > 0) {
    const dim3 g2((unsigned)(bt * mtiles), grid.y, 1);
    hipLaunchKernelGGL(gemm_dense_wide_kernel, g2, dim3(DW_THREADS), 0, s, p, bt);
  }
  if ((which & 2) && bt < ct) {
    const int nb0 = wide_tile_first_block(p, bt);
    const dim3 g3((unsigned)((nblk - nb0) * mtiles), grid.y, 1);
    hipLaunchKernelGGL((gemm_dense_kernel<false>), g3, dim3(DN_THREADS), 0, s, p, nb0);
  }
  return hipGetLastError();
}

}  // namespace exl3
