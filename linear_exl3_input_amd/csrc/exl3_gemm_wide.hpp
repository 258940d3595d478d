// 256-row x 128-column GEMM tile for large M on gfx950.
//
// Eight waves: wave w = 4*rh + wq owns rows 128*rh .. 128*rh+127 of the tile
// and the 32 columns of n-tiles 2*wq and 2*wq+1 (as in gemm_kernel, one MFMA
// B operand holds column half h = 0 or 1 of both n-tiles).  The two waves that
// share a column quarter split the decode: wave (wq, rh) decodes half h = rh
// of each k-step's B and the pair swaps the halves through LDS, so every
// trellis value is still decoded once per 256 rows while each wave does half
// the decode work.  On this GPU a wave's own VALU work hides only about two
// VALU instructions per MFMA; the second wave on the SIMD fills the rest.
//
// Data movement is by direct loads to LDS (global_load_lds_dwordx4), which
// need no registers and stay in flight across barriers:
//   - the trellis, in stages of 128 k x 128 columns, into a ring of three
//     stage slots, issued two stages ahead.  Tiles are stored raw (16-bit
//     words as they are in memory) with one 16-byte pad chunk on each side
//     (the tile's last chunk before it, its first chunk after it), so a
//     lane's window never wraps.  The word order is repaired in the decoder:
//     for even widths a lane's first stream bit is byte aligned and one
//     v_perm_b32 per window dword both reorders the words and aligns the
//     window; odd widths rotate each dword by 16 first.
//   - the rotated activations x~, one k-step (32 k x 256 rows, 16 KB) per
//     ring slot, PF k-steps ahead.
// Barriers wait only for LDS operations (barrier_lds); the direct loads are
// waited for with exact vmcnt counts.
//
// Arithmetic is the same as gemm_kernel's: the same MFMA shape, k slots,
// k-step order, K parts and part fold, so every schedule gives the same bits.
#pragma once

#include "exl3_gemm.hpp"

namespace exl3 {

template <int BITS>
struct Wide {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BM = 256;
  static constexpr int TSTRIDE = 8 * BITS + 8;           // dwords per padded tile
  static constexpr int T_CHUNKS = 64 * (2 * BITS + 2);   // 16-byte chunks per padded stage
  static constexpr int T_OPS = (T_CHUNKS + THREADS - 1) / THREADS;  // direct loads per wave per stage
  static constexpr int JUNK_CHUNKS = T_OPS * THREADS - T_CHUNKS;    // landing area for the surplus
  static constexpr int TSLOT_DW = T_CHUNKS * 4;
  static constexpr int TSLOTS = 3;
  static constexpr int A_OPS = BM / 16 / WAVES;          // direct loads per wave per k-step
  static constexpr int ASLOT_DW = BM * 16;               // 256 rows x 32 fp16
  static constexpr int XB_DW = WAVES * 256;              // one decoded B half per wave
  static constexpr int FIXED_DW = TSLOTS * TSLOT_DW + JUNK_CHUNKS * 4 + 2 * XB_DW;
  static constexpr int LDS_LIMIT_DW = 160 * 1024 / 4;
  // x~ prefetch distance in k-steps.  x~ of k-step i+1 is complete at the
  // barrier that ends k-step i-1, so a wave reads its first fragments of
  // k-step i+1 before the barrier that starts it.
  static constexpr int PF = FIXED_DW + 6 * ASLOT_DW <= LDS_LIMIT_DW ? 5 : 4;
  static constexpr int ASLOTS = PF + 1;
  static constexpr int MAIN_DW = FIXED_DW + ASLOTS * ASLOT_DW;
  static constexpr int Z_DW = 64 * Z_ROW;
  static constexpr int LDS_DW = MAIN_DW > Z_DW ? MAIN_DW : Z_DW;
  static constexpr int NY = Geom<BITS>::NY;
  static constexpr int NX = Geom<BITS>::NX;
  static constexpr bool PERM = BITS % 2 == 0;
  static_assert(T_CHUNKS % 64 == 0, "each direct load lands whole in a stage or in the surplus area");
  static_assert(LDS_DW <= LDS_LIMIT_DW, "LDS budget");

  // Direct loads this wave issues after the x~ loads of k-step i+2, up to the
  // wait at the end of k-step i (ks = i % 4): the x~ loads of k-steps
  // i+3 .. i+PF and the trellis loads issued at k-steps i+2-PF .. i whose
  // ks is 3 (one trellis stage is issued at ks == 3, after that k-step's
  // x~ loads).  Vector-memory operations complete in issue order, so the
  // wait also covers every earlier trellis stage.
  static constexpr int loads_after(int ks) {
    int t = 0;
    for (int k = ks + 2 - PF; k <= ks; ++k) t += ((k % 4) + 4) % 4 == 3 ? 1 : 0;
    return A_OPS * (PF - 2) + T_OPS * t;
  }
};

// Window of the lane's 8 states for even widths: start dword (after the
// front pad) and the v_perm_b32 selector that turns raw dwords d, d+1 into
// the 32 stream bits starting at the lane's (byte-aligned) first bit.
// Stream byte t of a raw dword is its little-endian byte (1, 0, 3, 2)[t].
template <int BITS>
__device__ __forceinline__ void lane_window_perm(int j, int g, int h, int &doff, uint32_t &sel) {
  const int v0 = 32 * (j & 7) + 4 * h + 16 * (g & 1);
  const int o = v0 * BITS;
  doff = 4 + (o >> 5);
  const int r = (o >> 3) & 3;
  sel = r == 0 ? 0x01000302u : r == 1 ? 0x00030205u : r == 2 ? 0x03020504u : 0x02050407u;
}

template <int BITS>
__device__ __forceinline__ void wide_normalize(const uint32_t (&X)[Wide<BITS>::NX], uint32_t sel, int sh,
                                               uint32_t (&Y)[Wide<BITS>::NY]) {
  using W = Wide<BITS>;
  if constexpr (W::PERM) {
#pragma unroll
    for (int i = 0; i < W::NY; ++i) Y[i] = __builtin_amdgcn_perm(X[i + 1], X[i], sel);
  } else {
    uint32_t Z[W::NX];
#pragma unroll
    for (int i = 0; i < W::NX; ++i) Z[i] = rot16(X[i]);
#pragma unroll
    for (int i = 0; i < W::NY; ++i) Y[i] = __builtin_amdgcn_alignbit(Z[i], Z[i + 1], sh);
  }
}

template <int BITS, uint32_t CB, bool MULTI>
__global__ __launch_bounds__(512, 1) void gemm_wide_kernel(const GemmParams p) {
  using W = Wide<BITS>;
  constexpr int PF = W::PF;
  constexpr int ASLOTS = W::ASLOTS;
  // x~ fragments read ahead across the barrier (fewer when the part fold's
  // second accumulator set needs the registers)
  constexpr int NPRE = MULTI ? 4 : 8;
  __shared__ __attribute__((aligned(16))) uint32_t lds[W::LDS_DW];
  uint32_t *const tring = lds;
  uint32_t *const junk = lds + W::TSLOTS * W::TSLOT_DW;
  uint32_t *const xbuf = junk + W::JUNK_CHUNKS * 4;
  uint32_t *const aring = xbuf + 2 * W::XB_DW;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wq = wave & 3;
  const int rh = wave >> 2;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nb = blockIdx.x;
  const int m0 = blockIdx.z * W::BM;
  const int M = p.M, K = p.K, N = p.N;
  const int NT = N >> 4;
  const int KB = K >> 7;

  int p_begin = 0, p_end = p.parts;
  if (p.slab_mode) {
    p_begin = blockIdx.y;
    p_end = p_begin + 1;
  }
  const int kb_begin = (int)((int64_t)p_begin * KB / p.parts);
  const int kb_end = (int)((int64_t)p_end * KB / p.parts);
  const int nst = kb_end - kb_begin;
  const int nks = 4 * nst;
  const int k_begin = kb_begin * 128;

  int shard = 0;
  while (shard + 1 < p.n_shards && nb >= p.shard_end_blk[shard]) ++shard;
  const uint16_t *__restrict__ xs = p.x_rot + (int64_t)shard * M * K;

  // ---- trellis direct loads: per-lane source offsets (16-bit words) of the
  // chunk that lands at this lane's LDS position in each issue round
  const uint16_t *const tr0 = p.trellis + ((int64_t)kb_begin * 8 * NT + nb * 8) * (16 * BITS);
  const int64_t tr_stage = (int64_t)8 * NT * (16 * BITS);
  uint32_t t_src[W::T_OPS];
#pragma unroll
  for (int r = 0; r < W::T_OPS; ++r) {
    const int q = r * W::THREADS + wave * 64 + lane;
    if (q < W::T_CHUNKS) {
      const int t = q / (2 * BITS + 2);
      const int c = q - t * (2 * BITS + 2);
      const int sc = c == 0 ? 2 * BITS - 1 : (c == 2 * BITS + 1 ? 0 : c - 1);
      t_src[r] = (uint32_t)(((t >> 3) * NT + (t & 7)) * (16 * BITS) + sc * 8);
    } else {
      t_src[r] = (uint32_t)((lane % (2 * BITS)) * 8);
    }
  }
  auto issue_trellis = [&](int stage, int slot) {
    const uint16_t *base = tr0 + (int64_t)min(stage, nst - 1) * tr_stage;
    uint32_t *const dst0 = tring + slot * W::TSLOT_DW;
#pragma unroll
    for (int r = 0; r < W::T_OPS; ++r) {
      const int q0 = r * W::THREADS + wave * 64;
      uint32_t *dst = q0 < W::T_CHUNKS ? dst0 + q0 * 4 : junk + (q0 - W::T_CHUNKS) * 4;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + t_src[r]),
                                       (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
  };
  // ---- x~ direct loads: fragment mf = wave + 8t holds rows 16mf .. 16mf+15;
  // lane L of it loads row L%16, k-chunk L/16 (x~ is in k-step tiles, so a
  // fragment is 1 KB contiguous).  Rows past M load row M-1.
  const uint16_t *a_src[W::A_OPS];
#pragma unroll
  for (int t = 0; t < W::A_OPS; ++t) {
    int row = m0 + 16 * (wave + W::WAVES * t) + (lane & 15);
    row = row < M ? row : M - 1;
    a_src[t] = xs + ((int64_t)(k_begin >> 5) * M + row) * 32 + 8 * (lane >> 4);
  }
  const int64_t a_kstep = (int64_t)M * 32;  // 16-bit words per k-step tile
  auto issue_a = [&](int kstep, int slot) {
    const int64_t k = a_kstep * min(kstep, nks - 1);
    uint32_t *const dst0 = aring + slot * W::ASLOT_DW;
#pragma unroll
    for (int t = 0; t < W::A_OPS; ++t)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(a_src[t] + k),
                                       (__attribute__((address_space(3))) void *)(dst0 + (wave + W::WAVES * t) * 256),
                                       16, 0, 0);
  };

  // ---- per-lane decode constants (half h = rh of n-tiles 2wq, 2wq+1)
  int doff, sh = 0;
  uint32_t sel = 0;
  if constexpr (W::PERM) {
    lane_window_perm<BITS>(j, g, rh, doff, sel);
  } else {
    lane_window<BITS>(j, g, rh, doff, sh);
  }
  const int t_lane = ((g >> 1) * WG_NT + 2 * wq + (j >> 3)) * W::TSTRIDE + doff;
  auto decode_own = [&](const uint32_t *slot, int kp) -> u32x4_t {
    const uint32_t *tp = slot + kp * 2 * WG_NT * W::TSTRIDE + t_lane;
    uint32_t X[W::NX], Y[W::NY];
#pragma unroll
    for (int i = 0; i < W::NX; ++i) X[i] = tp[i];
    wide_normalize<BITS>(X, sel, sh, Y);
    return u32x4_t{frag_pair<BITS, CB, 0>(Y), frag_pair<BITS, CB, 1>(Y), frag_pair<BITS, CB, 2>(Y),
                   frag_pair<BITS, CB, 3>(Y)};
  };
  uint32_t *const xb_own0 = xbuf + wave * 256 + 4 * lane;
  const uint32_t *const xb_par0 = xbuf + (wave ^ 4) * 256 + 4 * lane;
  const uint32_t *const a_lane = aring + rh * 8 * 256 + 4 * lane;

  // acc[mt][0]: own half (h = rh), acc[mt][1]: the partner's half
  float4_t acc[8][2];
  float4_t tot[MULTI ? 8 : 1][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: trellis stages 0..2, x~ k-steps 0..PF-1, own B of k-step 0
  issue_trellis(0, 0);
  issue_trellis(1, 1);
#pragma unroll
  for (int i = 0; i < PF; ++i) issue_a(i, i);
  issue_trellis(2, 2);
  wait_vmcnt<0>();
  barrier_lds();
  u32x4_t b_own = decode_own(tring, 0);
  *(u32x4_t *)xb_own0 = b_own;
  half8_t a_cur[8], a_nxt[NPRE];
#pragma unroll
  for (int q = 0; q < NPRE; ++q) a_cur[q] = *(const half8_t *)(a_lane + q * 256);
  barrier_lds();

  int st = 0;
  int ts0 = 0;     // trellis slot of stage st
  int as_cur = 0;  // x~ slot of k-step 4*st
  auto run_stages = [&](int st_end) {
    for (; st < st_end; ++st) {
      const int ts1 = ts0 == W::TSLOTS - 1 ? 0 : ts0 + 1;
      auto kstep = [&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        const int i = 4 * st + ks;
        int as = as_cur + ks;
        as = as >= ASLOTS ? as - ASLOTS : as;
        const int as_pf = as == 0 ? ASLOTS - 1 : as - 1;  // (i + PF) % ASLOTS, PF = ASLOTS - 1
        const int as_nx = as == ASLOTS - 1 ? 0 : as + 1;   // (i + 1) % ASLOTS
        issue_a(i + PF, as_pf);
        asm volatile("" ::: "memory");  // keep the issue order loads_after() counts
        if constexpr (ks == 3) issue_trellis(st + 3, ts0);
        asm volatile("" ::: "memory");
        const u32x4_t b_par = *(const u32x4_t *)(xb_par0 + (i & 1) * W::XB_DW);
        const half8_t B0 = __builtin_bit_cast(half8_t, b_own);
        const half8_t B1 = __builtin_bit_cast(half8_t, b_par);
        // decode inputs for the own half of k-step i+1
        const uint32_t *tslot = tring + (ks < 3 ? ts0 : ts1) * W::TSLOT_DW;
        const uint32_t *tp = tslot + ((ks + 1) & 3) * 2 * WG_NT * W::TSTRIDE + t_lane;
        uint32_t X[W::NX], Y[W::NY];
#pragma unroll
        for (int q = 0; q < W::NX; ++q) X[q] = tp[q];
        const uint32_t *as_n = a_lane + as_nx * W::ASLOT_DW;
        // a_cur[0 .. NPRE-1] hold this k-step's first x~ fragments (read
        // during the previous k-step), so the own-half products start right
        // after the barrier; the partner-half products follow, while the next
        // k-step's fragments are read (x~ of k-step i+1 is complete by now).
        u32x4_t nb4;
        if constexpr (NPRE < 8) {
          const uint32_t *as_p = a_lane + as * W::ASLOT_DW;
#pragma unroll
          for (int q = NPRE; q < 8; ++q) a_cur[q] = *(const half8_t *)(as_p + q * 256);
        }
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, 16>([&](auto it_c) {
          constexpr int it = decltype(it_c)::value;
          if constexpr (it < 8) {
            acc[it][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur[it], B0, acc[it][0], 0, 0, 0);
          } else {
            acc[it - 8][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur[it - 8], B1, acc[it - 8][1], 0, 0, 0);
            if constexpr (it - 8 < NPRE) a_nxt[it - 8] = *(const half8_t *)(as_n + (it - 8) * 256);
          }
          if constexpr (it == 2) wide_normalize<BITS>(X, sel, sh, Y);
          if constexpr (it >= 3 && it < 7) nb4[it - 3] = frag_pair<BITS, CB, it - 3>(Y);
          if constexpr (it == 7) *(u32x4_t *)(xb_own0 + ((i + 1) & 1) * W::XB_DW) = nb4;
          __builtin_amdgcn_sched_barrier(0);
        });
        wait_vmcnt<W::loads_after(ks)>();
        barrier_lds();
        b_own = nb4;
#pragma unroll
        for (int q = 0; q < NPRE; ++q) a_cur[q] = a_nxt[q];
      };
      kstep(std::integral_constant<int, 0>{});
      kstep(std::integral_constant<int, 1>{});
      kstep(std::integral_constant<int, 2>{});
      kstep(std::integral_constant<int, 3>{});
      ts0 = ts1;
      as_cur = as_cur + 4 >= ASLOTS ? as_cur + 4 - ASLOTS : as_cur + 4;
    }
  };

  if constexpr (MULTI) {
    // first part copied, later parts added in part order
    run_stages((int)((int64_t)(p_begin + 1) * KB / p.parts) - kb_begin);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        tot[mt][h] = acc[mt][h];
        acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
    for (int part = p_begin + 1; part < p_end; ++part) {
      run_stages((int)((int64_t)(part + 1) * KB / p.parts) - kb_begin);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          tot[mt][h] = tot[mt][h] + acc[mt][h];
          acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[mt][h] = tot[mt][h];
  } else {
    run_stages(nst);
  }
  wait_vmcnt<0>();  // the clamped tail loads land before LDS is reused
  barrier_lds();

  // column (within the 128) of acc[.][x] for this lane
  const int col_own = lane_col(wq, j, rh);
  const int col_par = lane_col(wq, j, rh ^ 1);
  if (p.slab_mode) {
    float *__restrict__ sl = p.slabs + (int64_t)p_begin * M * N + nb * 128;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + rh * 128 + mt * 16 + 4 * g + i;
        if (row < M) {
          sl[(int64_t)row * N + col_own] = acc[mt][0][i];
          sl[(int64_t)row * N + col_par] = acc[mt][1][i];
        }
      }
    return;
  }

  // output transform, 64 rows per pass through LDS
  float *z = reinterpret_cast<float *>(lds);
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (pass > 0) barrier_lds();
    if (rh == (pass >> 1)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int mt = 4 * (pass & 1) + q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[(q * 16 + 4 * g + i) * Z_ROW + col_own] = acc[mt][0][i];
          z[(q * 16 + 4 * g + i) * Z_ROW + col_par] = acc[mt][1][i];
        }
      }
    }
    barrier_lds();
    for (int r = wave; r < 64; r += W::WAVES) {
      const int row = m0 + pass * 64 + r;
      if (row >= M) break;
      const float z0 = z[r * Z_ROW + 2 * lane];
      const float z1 = z[r * Z_ROW + 2 * lane + 1];
      if (p.out_bf16) output_row<true>(z0, z1, p.svh, y + (int64_t)row * N, nb * 128, lane);
      else output_row<false>(z0, z1, p.svh, y + (int64_t)row * N, nb * 128, lane);
    }
  }
}

template <int BITS, uint32_t CB>
hipError_t launch_wide_t(bool multi, const GemmParams &p, dim3 grid, hipStream_t s) {
  if (multi) hipLaunchKernelGGL((gemm_wide_kernel<BITS, CB, true>), grid, dim3(512), 0, s, p);
  else hipLaunchKernelGGL((gemm_wide_kernel<BITS, CB, false>), grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace exl3
