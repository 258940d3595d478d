// 2*RW-row x 128-column GEMM tile for large M on gfx950 (RW = 128; RW = 64
// for 128-row tiles of one part per workgroup; 512-row tiles are
// gemm_wide4_kernel below).
//
// RW = 64 is sized for two workgroups per CU (four waves per SIMD): two
// trellis stage slots and at most 80 KB of LDS, at most 128 VGPRs.  At 128
// rows the decode costs about six VALU instructions per MFMA, and with only
// one workgroup's two waves per SIMD the SIMD sat idle half the time waiting
// on its own dependences; the second workgroup fills those gaps (gate_up
// 5120 x 34816 at 128 rows 155 -> 121 us, whose 272 tiles also no longer
// leave a second round of 16; q_proj / down_proj at 128 rows in slabs
// 50 / 70 -> 44 / 63 us against the 4-wave 128-row tile).  The same budget
// at RW = 128 forces a one-k-step x~ prefetch and spills, and was slower
// (q_proj / down_proj at 256 rows 68 / 96 -> 73 / 110 us).
//
// Eight waves: wave w = 4*rh + wq owns rows RW*rh .. RW*rh+RW-1 of the tile
// and the 32 columns of n-tiles 2*wq and 2*wq+1 (as in gemm_kernel, one MFMA
// B operand holds column half h = 0 or 1 of both n-tiles).  The two waves that
// share a column quarter split the decode: wave (wq, rh) decodes half h = rh
// of each k-step's B and the pair swaps the halves through LDS, so every
// trellis value is still decoded once per 256 rows while each wave does half
// the decode work.
//
// The two partners run on the same SIMD (wave w and w+4) and are scheduled
// in opposite phases: the rh = 0 wave issues its sixteen MFMAs first and then
// decodes, the rh = 1 wave decodes first and then issues its MFMAs, so one
// wave's VALU work runs while the other wave's MFMAs occupy the matrix core
// (a wave's own VALU instructions hide behind only about two MFMAs each).
//
// Data movement is by direct loads to LDS (global_load_lds_dwordx4), which
// need no registers and stay in flight across barriers.  The rh = 0 waves
// load x~, the rh = 1 waves load the trellis, so that x~ loads (L2 hits)
// never wait behind trellis loads (HBM) in a wave's in-order load queue:
//   - the trellis, in stages of 128 k x 128 columns, into a ring of TSLOTS
//     stage slots, issued TSLOTS-1 stages ahead.  Tiles are stored raw
//     (16-bit words as they are in memory) with one 16-byte pad chunk on each
//     side (the tile's last chunk before it, its first chunk after it), so a
//     lane's window never wraps.  The word order is repaired in the decoder:
//     for even widths a lane's first stream bit is byte aligned and one
//     v_perm_b32 per window dword both reorders the words and aligns the
//     window; odd widths rotate each dword by 16 first.
//   - the rotated activations x~, one k-step (32 k x 256 rows, 16 KB, one
//     contiguous block in the k-step tile layout) per ring slot, PF k-steps
//     ahead.
// Barriers wait only for LDS operations (barrier_lds); the direct loads are
// waited for with exact vmcnt counts.
//
// Arithmetic is the same as gemm_kernel's: the same MFMA shape, k slots,
// k-step order, K parts and part fold, so every schedule gives the same bits.
#pragma once

#include "exl3_gemm.hpp"

namespace exl3 {

template <int BITS, int RW>
struct Wide {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int MF = RW / 16;                     // 16-row fragments per wave
  static constexpr int BM = 2 * RW;
  static constexpr int LOADERS = 4;                      // waves per load role
  static constexpr int TSTRIDE = 8 * BITS + 8;           // dwords per padded tile
  static constexpr int T_CHUNKS = 64 * (2 * BITS + 2);   // 16-byte chunks per padded stage
  static constexpr int T_OPS = (T_CHUNKS + 64 * LOADERS - 1) / (64 * LOADERS);  // per trellis wave per stage
  static constexpr int JUNK_CHUNKS = T_OPS * 64 * LOADERS - T_CHUNKS;           // landing area for the surplus
  static constexpr int TSLOT_DW = T_CHUNKS * 4;
  static constexpr int OCC = RW == 64 ? 2 : 1;             // workgroups per CU
  static constexpr int TSLOTS = OCC == 2 ? 2 : 4;
  static constexpr int A_OPS = BM / 16 / LOADERS;        // direct loads per x~ wave per k-step
  static constexpr int ASLOT_DW = BM * 16;               // BM rows x 32 fp16
  static constexpr int XB_DW = WAVES * 256;              // one decoded B half per wave
  static constexpr int FIXED_DW = TSLOTS * TSLOT_DW + JUNK_CHUNKS * 4 + 2 * XB_DW;
  static constexpr int LDS_LIMIT_DW = 160 * 1024 / 4 / OCC;
  // x~ prefetch distance in k-steps (as deep as LDS allows).  With PF >= 3
  // (AHEAD) x~ of k-step i+1 is complete at the barrier that ends k-step
  // i-1, and a wave reads its first fragments of k-step i+1 before the
  // barrier that starts it.
  static constexpr int PF = FIXED_DW + 5 * ASLOT_DW <= LDS_LIMIT_DW ? 4
                            : FIXED_DW + 4 * ASLOT_DW <= LDS_LIMIT_DW ? 3 : 2;
  static constexpr bool AHEAD = PF >= 3 && RW == 128;
  static constexpr int ASLOTS = PF + 1;
  static constexpr int MAIN_DW = FIXED_DW + ASLOTS * ASLOT_DW;
  // output stage: ZR rows (of one row half) per pass through LDS, a whole
  // row half when the main loop's LDS holds it
  static constexpr int ZR = MAIN_DW >= RW * Z_ROW ? RW : 64;
  static constexpr int Z_DW = ZR * Z_ROW;
  static constexpr int LDS_DW = MAIN_DW > Z_DW ? MAIN_DW : Z_DW;
  static constexpr int NY = Geom<BITS>::NY;
  static constexpr int NX = Geom<BITS>::NX;
  static constexpr bool PERM = BITS % 2 == 0;
  static_assert(T_CHUNKS % 64 == 0, "each direct load lands whole in a stage or in the surplus area");
  static_assert(LDS_DW <= LDS_LIMIT_DW, "LDS budget");

  // x~ waves: at the end of k-step i, x~ of k-step i+2 (AHEAD) or i+1 must
  // have landed.  Issued after it are the x~ loads of the later k-steps up
  // to i+PF.  Vector-memory operations complete in issue order.
  static constexpr int A_WAIT = A_OPS * (AHEAD ? PF - 2 : PF - 1);
  // trellis waves: at the end of k-step i (ks = i % 4, stage st = i / 4) the
  // stage the next k-step decodes from, (i + 2) / 4, must have landed.  Stage
  // st + TSLOTS is issued at ks == 3 of stage st, so the stages issued after
  // the needed one number TSLOTS - 1 + [ks == 3] - [ks >= 2].
  static constexpr int t_wait(int ks) {
    return T_OPS * (TSLOTS - 1 + (ks == 3 ? 1 : 0) - (ks >= 2 ? 1 : 0));
  }
};

// (launch bounds: 512 threads and, for RW = 64, at least four waves per SIMD,
// which caps a wave at 128 VGPRs)
template <int BITS, uint32_t CB, int RW, bool MULTI, int SCHED = 1>
__global__ __launch_bounds__(512, RW == 64 ? 4 : 1) void gemm_wide_kernel(const GemmParams p) {
  using W = Wide<BITS, RW>;
  constexpr int MF = W::MF;
  constexpr int PF = W::PF;
  constexpr int ASLOTS = W::ASLOTS;
  constexpr int TSLOTS = W::TSLOTS;
  // x~ fragments read ahead across the barrier (fewer when the part fold's
  // second accumulator set needs the registers; none without AHEAD)
  constexpr int NPRE = !W::AHEAD ? 0 : (MULTI ? 4 : 8);
  static_assert(!W::AHEAD || MF == 8, "read-ahead schedule is for 128-row waves");
  static_assert(RW == 64 || RW == 128, "512-row tiles are gemm_wide4_kernel");
  __shared__ __attribute__((aligned(16))) uint32_t lds[W::LDS_DW];
  uint32_t *const tring = lds;
  uint32_t *const junk = lds + TSLOTS * W::TSLOT_DW;
  uint32_t *const xbuf = junk + W::JUNK_CHUNKS * 4;
  uint32_t *const aring = xbuf + 2 * W::XB_DW;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wq = wave & 3;
  const int rh = wave >> 2;  // 0: x~ loads, MFMA first; 1: trellis loads, decode first
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nb = blockIdx.x;
  const int m0 = p.row_base + blockIdx.z * W::BM;
  const int rend = p.row_end;
  const int M = p.M, K = p.K, N = p.N;
  const int NT = N >> 4;
  const int KB = K >> 7;

  const int p_begin = blockIdx.y * p.unit;  // the workgroup's unit: parts p_begin .. p_end-1
  const int p_end = p_begin + p.unit;
  const int kb_begin = (int)((int64_t)p_begin * KB / p.parts);
  const int kb_end = (int)((int64_t)p_end * KB / p.parts);
  const int nst = kb_end - kb_begin;
  const int nks = 4 * nst;
  const int k_begin = kb_begin * 128;

  int shard = 0;
  while (shard + 1 < p.n_shards && nb >= p.shard_end_blk[shard]) ++shard;
  const uint16_t *__restrict__ xs = p.x_rot + (int64_t)shard * M * K;

  // ---- load sources.  The rh = 0 waves use src[t] for x~ fragment
  // wq + 4t (rows 16(wq+4t) .. +15; lane L loads row L%16, k-chunk L/16;
  // rows past M load row M-1).  The rh = 1 waves use src[r] for the trellis
  // chunk that lands at this lane's LDS position in round r.
  // Offsets are in 16-bit words from a_base / t_base (wave-uniform).
  const uint16_t *const a_base = xs + (int64_t)(k_begin >> 5) * M * 32;
  const uint16_t *const t_base = p.trellis + ((int64_t)kb_begin * 8 * NT + nb * 8) * (16 * BITS);
  uint32_t src[W::A_OPS > W::T_OPS ? W::A_OPS : W::T_OPS];
  if (rh == 0) {
#pragma unroll
    for (int t = 0; t < W::A_OPS; ++t) {
      int row = m0 + 16 * (wq + W::LOADERS * t) + (lane & 15);
      row = row < rend ? row : rend - 1;
      src[t] = (uint32_t)(row * 32 + 8 * (lane >> 4));
    }
  } else {
#pragma unroll
    for (int r = 0; r < W::T_OPS; ++r) {
      const int q = r * 64 * W::LOADERS + wq * 64 + lane;
      uint32_t off;
      if (q < W::T_CHUNKS) {
        const int t = q / (2 * BITS + 2);
        const int c = q - t * (2 * BITS + 2);
        const int sc = c == 0 ? 2 * BITS - 1 : (c == 2 * BITS + 1 ? 0 : c - 1);
        off = (uint32_t)(((t >> 3) * NT + (t & 7)) * (16 * BITS) + sc * 8);
      } else {
        off = (uint32_t)((lane % (2 * BITS)) * 8);
      }
      src[r] = off;
    }
  }
  const int64_t a_kstep = (int64_t)M * 32;                 // 16-bit words per x~ k-step tile
  const int64_t tr_stage = (int64_t)8 * NT * (16 * BITS);  // 16-bit words per trellis stage
  auto issue_a = [&](int kstep, int slot) {
    const uint16_t *const base = a_base + a_kstep * min(kstep, nks - 1);
    uint32_t *const dst0 = aring + slot * W::ASLOT_DW;
#pragma unroll
    for (int t = 0; t < W::A_OPS; ++t)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + src[t]),
                                       (__attribute__((address_space(3))) void *)(dst0 + (wq + W::LOADERS * t) * 256),
                                       16, 0, 0);
  };
  auto issue_trellis = [&](int stage, int slot) {
    const uint16_t *const base = t_base + tr_stage * min(stage, nst - 1);
    uint32_t *const dst0 = tring + slot * W::TSLOT_DW;
#pragma unroll
    for (int r = 0; r < W::T_OPS; ++r) {
      const int q0 = r * 64 * W::LOADERS + wq * 64;
      uint32_t *dst = q0 < W::T_CHUNKS ? dst0 + q0 * 4 : junk + (q0 - W::T_CHUNKS) * 4;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + src[r]),
                                       (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
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
    raw_normalize<BITS>(X, sel, sh, Y);
    return u32x4_t{frag_pair<BITS, CB, 0>(Y), frag_pair<BITS, CB, 1>(Y), frag_pair<BITS, CB, 2>(Y),
                   frag_pair<BITS, CB, 3>(Y)};
  };
  uint32_t *const xb_own0 = xbuf + wave * 256 + 4 * lane;
  const uint32_t *const xb_par0 = xbuf + (wave ^ 4) * 256 + 4 * lane;
  const uint32_t *const a_lane = aring + rh * MF * 256 + 4 * lane;

  // acc[mt][0]: own half (h = rh), acc[mt][1]: the partner's half
  float4_t acc[MF][2];
  float4_t tot[MULTI ? MF : 1][2];
#pragma unroll
  for (int mt = 0; mt < MF; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: trellis stages 0 .. TSLOTS-1, x~ k-steps 0 .. PF-1, own B
  // of k-step 0, first x~ fragments of k-step 0
  if (rh == 0) {
#pragma unroll
    for (int i = 0; i < PF; ++i) issue_a(i, i);
  } else {
#pragma unroll
    for (int s = 0; s < TSLOTS; ++s) issue_trellis(s, s);
  }
  wait_vmcnt<0>();
  barrier_lds();
  u32x4_t b_own = decode_own(tring, 0);
  *(u32x4_t *)xb_own0 = b_own;
  half8_t a_cur[8], a_nxt[NPRE > 0 ? NPRE : 1];
#pragma unroll
  for (int q = 0; q < NPRE; ++q) a_cur[q] = *(const half8_t *)(a_lane + q * 256);
  barrier_lds();

  int st = 0;
  int ts0 = 0;     // trellis slot of stage st
  int as_cur = 0;  // x~ slot of k-step 4*st
  auto run_stages = [&](int st_end, auto ph_c) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_c)::value;  // == rh
    for (; st < st_end; ++st) {
      const int ts1 = ts0 == TSLOTS - 1 ? 0 : ts0 + 1;
      auto kstep = [&](auto ks_c) __attribute__((always_inline)) {
        constexpr int ks = decltype(ks_c)::value;
        const int i = 4 * st + ks;
        const int as = (as_cur + ks) % ASLOTS;  // x~ slot of k-step i
        const int as_pf = as == 0 ? ASLOTS - 1 : as - 1;  // (i + PF) % ASLOTS, PF = ASLOTS - 1
        const int as_nx = as == ASLOTS - 1 ? 0 : as + 1;   // (i + 1) % ASLOTS
        if constexpr (PH == 0) issue_a(i + PF, as_pf);
        else if constexpr (ks == 3) issue_trellis(st + TSLOTS, ts0);
        asm volatile("" ::: "memory");  // keep the issue order the waits count
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
        const uint32_t *as_p = a_lane + as * W::ASLOT_DW;
        if constexpr (NPRE > 0 && NPRE < 8) {
#pragma unroll
          for (int q = NPRE; q < 8; ++q) a_cur[q] = *(const half8_t *)(as_p + q * 256);
        }
        u32x4_t nb4;
        auto decode = [&]() __attribute__((always_inline)) {
          raw_normalize<BITS>(X, sel, sh, Y);
          nb4[0] = frag_pair<BITS, CB, 0>(Y);
          nb4[1] = frag_pair<BITS, CB, 1>(Y);
          nb4[2] = frag_pair<BITS, CB, 2>(Y);
          nb4[3] = frag_pair<BITS, CB, 3>(Y);
          *(u32x4_t *)(xb_own0 + ((i + 1) & 1) * W::XB_DW) = nb4;
        };
        // own-half products first (operands in registers), then the
        // partner half, while the next k-step's first fragments are read
        // (x~ of k-step i+1 is complete by now)
        auto products = [&]() __attribute__((always_inline)) {
          if constexpr (NPRE > 0) {
            static_for<0, 16>([&](auto it_c) {
              constexpr int it = decltype(it_c)::value;
              if constexpr (it < 8) {
                acc[it][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur[it], B0, acc[it][0], 0, 0, 0);
              } else {
                acc[it - 8][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_cur[it - 8], B1, acc[it - 8][1], 0, 0, 0);
                if constexpr (it - 8 < NPRE) a_nxt[it - 8] = *(const half8_t *)(as_n + (it - 8) * 256);
              }
            });
          } else {
            // fragment mt read RD fragments ahead of its two products
            constexpr int RD = 3;
            half8_t af[MF];
#pragma unroll
            for (int q = 0; q < RD; ++q) af[q] = *(const half8_t *)(as_p + q * 256);
            static_for<0, MF>([&](auto mt_c) {
              constexpr int mt = decltype(mt_c)::value;
              if constexpr (mt + RD < MF) af[mt + RD] = *(const half8_t *)(as_p + (mt + RD) * 256);
              acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], B0, acc[mt][0], 0, 0, 0);
              acc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], B1, acc[mt][1], 0, 0, 0);
            });
          }
        };
        // Without the read-ahead across the barrier (64-row waves): a ring
        // of four x~ fragments read three ahead of their products, and the
        // decode cut into six pieces between the product pairs, each step
        // fenced so the compiler keeps the reads early (left to itself, at
        // this register pressure it issued every read just before its use).
        auto products_pipelined = [&]() __attribute__((always_inline)) {
          constexpr int RD = 3;
          half8_t af[4];
#pragma unroll
          for (int q = 0; q < RD; ++q) af[q] = *(const half8_t *)(as_p + q * 256);
          static_for<0, MF>([&](auto mt_c) {
            constexpr int mt = decltype(mt_c)::value;
            if constexpr (mt + RD < MF) af[(mt + RD) % 4] = *(const half8_t *)(as_p + (mt + RD) * 256);
            acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt % 4], B0, acc[mt][0], 0, 0, 0);
            acc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt % 4], B1, acc[mt][1], 0, 0, 0);
            static_for<mt * 6 / MF, (mt + 1) * 6 / MF>([&](auto pc) {
              constexpr int piece = decltype(pc)::value;
              if constexpr (piece == 0) raw_normalize<BITS>(X, sel, sh, Y);
              else if constexpr (piece < 5) nb4[piece - 1] = frag_pair<BITS, CB, piece - 1>(Y);
              else *(u32x4_t *)(xb_own0 + ((i + 1) & 1) * W::XB_DW) = nb4;
            });
            __builtin_amdgcn_sched_barrier(0);
          });
        };
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SCHED == 1 && NPRE == 0) {
          products_pipelined();
        } else if constexpr (SCHED == 1) {
          // interleaved: each MFMA followed by about three VALU instructions
          // of the decode (a wave issues VALU at most every ~8 cycles, so
          // the decode is spread over the whole k-step in both waves)
          products();
          decode();
          static_for<0, 2 * MF>([&](auto it_c) {
            constexpr int it = decltype(it_c)::value;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, MF == 8 ? 3 : 2, 0);  // VALU
            if constexpr (NPRE > 0 ? it >= 8 : (it % 2 == 0 && it / 2 + 3 < MF))
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          });
        } else if constexpr (PH == 0) {
          products();
          __builtin_amdgcn_sched_barrier(0);
          decode();
        } else {
          decode();
          __builtin_amdgcn_sched_barrier(0);
          products();
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PH == 0) wait_vmcnt<W::A_WAIT>();
        else wait_vmcnt<W::t_wait(ks)>();
        barrier_lds();
        b_own = nb4;
#pragma unroll
        for (int q = 0; q < NPRE; ++q) a_cur[q] = a_nxt[q];
        (void)as_n;
      };
      kstep(std::integral_constant<int, 0>{});
      kstep(std::integral_constant<int, 1>{});
      kstep(std::integral_constant<int, 2>{});
      kstep(std::integral_constant<int, 3>{});
      ts0 = ts1;
      as_cur = (as_cur + 4) % ASLOTS;  // four k-steps per stage; ASLOTS may be 3
    }
  };

  // the whole K loop, for one phase (the branch on rh is taken once)
  auto main_loop = [&](auto ph_c) __attribute__((always_inline)) {
  if constexpr (MULTI) {
    // first part copied, later parts added in part order
    run_stages((int)((int64_t)(p_begin + 1) * KB / p.parts) - kb_begin, ph_c);
#pragma unroll
    for (int mt = 0; mt < MF; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        tot[mt][h] = acc[mt][h];
        acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
    for (int part = p_begin + 1; part < p_end; ++part) {
      run_stages((int)((int64_t)(part + 1) * KB / p.parts) - kb_begin, ph_c);
#pragma unroll
      for (int mt = 0; mt < MF; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          tot[mt][h] = tot[mt][h] + acc[mt][h];
          acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int mt = 0; mt < MF; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[mt][h] = tot[mt][h];
  } else {
    run_stages(nst, ph_c);
  }
  };
  if (rh == 0) main_loop(std::integral_constant<int, 0>{});
  else main_loop(std::integral_constant<int, 1>{});
  wait_vmcnt<0>();  // the clamped tail loads land before LDS is reused
  barrier_lds();

  // column (within the 128) of acc[.][x] for this lane
  const int col_own = lane_col(wq, j, rh);
  const int col_par = lane_col(wq, j, rh ^ 1);
  if (p.slab_mode) {
    const int rows = rend - p.row_base;
#pragma unroll
    for (int mt = 0; mt < MF; ++mt) {
      const int row0 = m0 - p.row_base + rh * RW + mt * 16 + 4 * g;
      store_partial(p.slabs, blockIdx.y, rows, N, row0, nb * 128 + col_own, acc[mt][0]);
      store_partial(p.slabs, blockIdx.y, rows, N, row0, nb * 128 + col_par, acc[mt][1]);
    }
    return;
  }

  // output transform, W::ZR rows of one row half per pass through LDS:
  // the half's four waves write their accumulators, then every wave runs the
  // output stage on eight rows at a time (output_rows8)
  float *z = reinterpret_cast<float *>(lds);
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
  constexpr int ZR = W::ZR;
  constexpr int PPH = RW / ZR;  // passes per row half
  const OutWords16 ow = out_words16(p.svh, p.bias, nb * 128, lane);
  const bool has_bias = p.bias != nullptr;
#pragma unroll
  for (int pass = 0; pass < 2 * PPH; ++pass) {
    if (pass > 0) barrier_lds();
    if (rh == pass / PPH) {
#pragma unroll
      for (int q = 0; q < ZR / 16; ++q) {
        const int mt = (ZR / 16) * (pass % PPH) + q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[(q * 16 + 4 * g + i) * Z_ROW + col_own] = acc[mt][0][i];
          z[(q * 16 + 4 * g + i) * Z_ROW + col_par] = acc[mt][1][i];
        }
      }
    }
    barrier_lds();
#pragma unroll
    for (int r0 = 8 * wave; r0 < ZR; r0 += 8 * W::WAVES) {
      if (p.out_bf16) output_rows8<true>(z, Z_ROW, r0, ow, has_bias, y, m0 + pass * ZR + r0, rend, N, nb * 128, lane);
      else output_rows8<false>(z, Z_ROW, r0, ow, has_bias, y, m0 + pass * ZR + r0, rend, N, nb * 128, lane);
    }
  }
}

// 512-row x 128-column tile on 8 waves as 4 row quarters x 2 column halves
// (wave w: rows 128 (w >> 1) .. +127, the 64 columns of n-tiles 4 (w & 1) ..
// +3).  Per 32-k step a wave reads 8 x~ fragments and the 4 decoded B
// fragments of its column half from LDS and issues 32 MFMAs into 128
// accumulators; the four waves of a column half each decode one of the four
// B fragments (pair 2ch + (rq >> 1), half rq & 1) and share them through LDS
// (a wave reads its own back too: keeping it in registers pushed the kernel
// past 256 VGPRs into spills).  Against two row halves of 256 rows (16 x~
// fragments and one B fragment read per wave and k-step) that is 96 KB of
// LDS reads per k-step instead of 136 KB, for the same decode work per wave.
// The decode runs two k-steps ahead, so a wave reads the next k-step's B
// fragments between this k-step's products and, after each barrier, waits
// only for its first x~ fragments (the products of a k-step used to wait for
// all four B fragments and three x~ fragments of every wave, 56 KB of LDS
// reads, after the barrier).  Loads and ring slots are gemm_wide_kernel's;
// same fragments, k order and chains, so the same bits.
template <int BITS>
struct Wide4 {
  static constexpr int WAVES = 8;
  static constexpr int MF = 8;   // 16-row fragments per wave
  static constexpr int NF = 4;   // B fragments per wave
  static constexpr int BM = 512;
  static constexpr int LOADERS = 4;
  static constexpr int TSTRIDE = 8 * BITS + 8;
  static constexpr int T_CHUNKS = 64 * (2 * BITS + 2);
  static constexpr int T_OPS = (T_CHUNKS + 64 * LOADERS - 1) / (64 * LOADERS);
  static constexpr int JUNK_CHUNKS = T_OPS * 64 * LOADERS - T_CHUNKS;
  static constexpr int TSLOT_DW = T_CHUNKS * 4;
  static constexpr int A_OPS = BM / 16 / LOADERS;
  static constexpr int ASLOT_DW = BM * 16;
  static constexpr int XB_DW = WAVES * 256;
  // decoded B fragments: during k-step i the waves read k-step i+1's from
  // buffer (i+1) & 1 and decode k-step i+2's into buffer i & 1, whose
  // k-step i fragments they read into registers during k-step i-1
  static constexpr int XBUFS = 2;
  static constexpr int LDS_LIMIT_DW = 160 * 1024 / 4;
  static constexpr int fixed_dw(int tslots) { return tslots * TSLOT_DW + JUNK_CHUNKS * 4 + XBUFS * XB_DW; }
  static constexpr int TSLOTS = fixed_dw(3) + 3 * ASLOT_DW <= LDS_LIMIT_DW ? 3 : 2;
  static constexpr int FIXED_DW = fixed_dw(TSLOTS);
  static constexpr int PF = FIXED_DW + 4 * ASLOT_DW <= LDS_LIMIT_DW ? 3 : 2;
  static constexpr int ASLOTS = PF + 1;
  static constexpr int MAIN_DW = FIXED_DW + ASLOTS * ASLOT_DW;
  static constexpr int ZR = 128;  // output rows per pass: one row quarter
  static constexpr int Z_DW = ZR * Z_ROW;
  static constexpr int LDS_DW = MAIN_DW > Z_DW ? MAIN_DW : Z_DW;
  static constexpr int NY = Geom<BITS>::NY;
  static constexpr int NX = Geom<BITS>::NX;
  static constexpr bool PERM = BITS % 2 == 0;
  static_assert(T_CHUNKS % 64 == 0, "each direct load lands whole in a stage or in the surplus area");
  static_assert(LDS_DW <= LDS_LIMIT_DW, "LDS budget");
  static constexpr int A_WAIT = A_OPS * (PF - 1);
  // Trellis stage st + TSLOTS is issued at ks == 2 of stage st (the last
  // decode from its slot, of k-step 4st+3, ran during ks == 1).  The decode
  // during k-step i+1 reads stage (i + 3) / 4, which must have landed by the
  // end of k-step i: the stages issued after it number
  // TSLOTS - 1 + [ks >= 2] - [ks >= 1].
  static constexpr int t_wait(int ks) {
    return T_OPS * (TSLOTS - 1 + (ks >= 2 ? 1 : 0) - (ks >= 1 ? 1 : 0));
  }
};

template <int BITS, uint32_t CB>
__global__ __launch_bounds__(512, 1) void gemm_wide4_kernel(const GemmParams p) {
  using W = Wide4<BITS>;
  constexpr int MF = W::MF;
  constexpr int NF = W::NF;
  constexpr int PF = W::PF;
  constexpr int ASLOTS = W::ASLOTS;
  constexpr int TSLOTS = W::TSLOTS;
  __shared__ __attribute__((aligned(16))) uint32_t lds[W::LDS_DW];
  uint32_t *const tring = lds;
  uint32_t *const junk = lds + TSLOTS * W::TSLOT_DW;
  uint32_t *const xbuf = junk + W::JUNK_CHUNKS * 4;
  uint32_t *const aring = xbuf + W::XBUFS * W::XB_DW;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lw = wave & 3;     // loader index
  const int role = wave >> 2;  // 0: x~ loads; 1: trellis loads
  const int ch = wave & 1;     // column half
  const int rq = wave >> 1;    // row quarter; decodes fragment f = rq of its half
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nb = blockIdx.x;
  const int m0 = p.row_base + blockIdx.z * W::BM;
  const int rend = p.row_end;
  const int M = p.M, K = p.K, N = p.N;
  const int NT = N >> 4;
  const int KB = K >> 7;

  const int p_begin = blockIdx.y * p.unit;
  const int kb_begin = (int)((int64_t)p_begin * KB / p.parts);
  const int kb_end = (int)((int64_t)(p_begin + 1) * KB / p.parts);
  const int nst = kb_end - kb_begin;
  const int nks = 4 * nst;
  const int k_begin = kb_begin * 128;

  int shard = 0;
  while (shard + 1 < p.n_shards && nb >= p.shard_end_blk[shard]) ++shard;
  const uint16_t *__restrict__ xs = p.x_rot + (int64_t)shard * M * K;

  const uint16_t *const a_base = xs + (int64_t)(k_begin >> 5) * M * 32;
  const uint16_t *const t_base = p.trellis + ((int64_t)kb_begin * 8 * NT + nb * 8) * (16 * BITS);
  uint32_t src[W::A_OPS > W::T_OPS ? W::A_OPS : W::T_OPS];
  if (role == 0) {
#pragma unroll
    for (int t = 0; t < W::A_OPS; ++t) {
      int row = m0 + 16 * (lw + W::LOADERS * t) + (lane & 15);
      row = row < rend ? row : rend - 1;
      src[t] = (uint32_t)(row * 32 + 8 * (lane >> 4));
    }
  } else {
#pragma unroll
    for (int r = 0; r < W::T_OPS; ++r) {
      const int q = r * 64 * W::LOADERS + lw * 64 + lane;
      uint32_t off;
      if (q < W::T_CHUNKS) {
        const int t = q / (2 * BITS + 2);
        const int c = q - t * (2 * BITS + 2);
        const int sc = c == 0 ? 2 * BITS - 1 : (c == 2 * BITS + 1 ? 0 : c - 1);
        off = (uint32_t)(((t >> 3) * NT + (t & 7)) * (16 * BITS) + sc * 8);
      } else {
        off = (uint32_t)((lane % (2 * BITS)) * 8);
      }
      src[r] = off;
    }
  }
  const int64_t a_kstep = (int64_t)M * 32;
  const int64_t tr_stage = (int64_t)8 * NT * (16 * BITS);
  auto issue_a = [&](int kstep, int slot) {
    const uint16_t *const base = a_base + a_kstep * min(kstep, nks - 1);
    uint32_t *const dst0 = aring + slot * W::ASLOT_DW;
#pragma unroll
    for (int t = 0; t < W::A_OPS; ++t)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + src[t]),
                                       (__attribute__((address_space(3))) void *)(dst0 + (lw + W::LOADERS * t) * 256),
                                       16, 0, 0);
  };
  auto issue_trellis = [&](int stage, int slot) {
    const uint16_t *const base = t_base + tr_stage * min(stage, nst - 1);
    uint32_t *const dst0 = tring + slot * W::TSLOT_DW;
#pragma unroll
    for (int r = 0; r < W::T_OPS; ++r) {
      const int q0 = r * 64 * W::LOADERS + lw * 64;
      uint32_t *dst = q0 < W::T_CHUNKS ? dst0 + q0 * 4 : junk + (q0 - W::T_CHUNKS) * 4;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + src[r]),
                                       (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
  };

  // decode constants of the wave's own fragment: pair 2ch + (rq >> 1), half rq & 1
  const int dpair = 2 * ch + (rq >> 1);
  int doff, sh = 0;
  uint32_t sel = 0;
  if constexpr (W::PERM) {
    lane_window_perm<BITS>(j, g, rq & 1, doff, sel);
  } else {
    lane_window<BITS>(j, g, rq & 1, doff, sh);
  }
  const int t_lane = ((g >> 1) * WG_NT + 2 * dpair + (j >> 3)) * W::TSTRIDE + doff;
  auto decode_own = [&](const uint32_t *slot, int kp) -> u32x4_t {
    const uint32_t *tp = slot + kp * 2 * WG_NT * W::TSTRIDE + t_lane;
    uint32_t X[W::NX], Y[W::NY];
#pragma unroll
    for (int i = 0; i < W::NX; ++i) X[i] = tp[i];
    raw_normalize<BITS>(X, sel, sh, Y);
    return u32x4_t{frag_pair<BITS, CB, 0>(Y), frag_pair<BITS, CB, 1>(Y), frag_pair<BITS, CB, 2>(Y),
                   frag_pair<BITS, CB, 3>(Y)};
  };
  // xbuf[buf][wave]: the fragment wave w decoded; fragment f of this wave's
  // column half comes from wave 2f + ch
  uint32_t *const xb_own0 = xbuf + wave * 256 + 4 * lane;
  const uint32_t *const xb_half0 = xbuf + ch * 256 + 4 * lane;
  const uint32_t *const a_lane = aring + rq * MF * 256 + 4 * lane;

  float4_t acc[MF][NF];
#pragma unroll
  for (int mt = 0; mt < MF; ++mt)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[mt][f] = float4_t{0.f, 0.f, 0.f, 0.f};

  if (role == 0) {
#pragma unroll
    for (int i = 0; i < PF; ++i) issue_a(i, i);
  } else {
#pragma unroll
    for (int s = 0; s < TSLOTS; ++s) issue_trellis(s, s);
  }
  wait_vmcnt<0>();
  barrier_lds();
  *(u32x4_t *)xb_own0 = decode_own(tring, 0);
  *(u32x4_t *)(xb_own0 + W::XB_DW) = decode_own(tring, 1);
  barrier_lds();
  // B[i & 1]: the column half's four fragments (this wave's own among them)
  // of k-step i = 4 st + ks, read during k-step i-1 from the buffer the
  // waves decoded them into during k-step i-2, so that a k-step's products
  // wait after its barrier only for its first x~ reads
  half8_t B[2][NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) B[0][f] = *(const half8_t *)(xb_half0 + f * 512);

  int st = 0;
  int ts0 = 0;
  int as_cur = 0;
  auto run_stages = [&](auto ph_c) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_c)::value;
    for (; st < nst; ++st) {
      const int ts1 = ts0 == TSLOTS - 1 ? 0 : ts0 + 1;
      auto kstep = [&](auto ks_c) __attribute__((always_inline)) {
        constexpr int ks = decltype(ks_c)::value;
        constexpr int cur = ks & 1;
        const int i = 4 * st + ks;
        const int as = (as_cur + ks) % ASLOTS;
        const int as_pf = as == 0 ? ASLOTS - 1 : as - 1;
        if constexpr (PH == 0) issue_a(i + PF, as_pf);
        else if constexpr (ks == 2) issue_trellis(st + TSLOTS, ts0);
        asm volatile("" ::: "memory");
        // the decode of k-step i+2: stage st (ks < 2) or st+1
        const uint32_t *tslot = tring + (ks < 2 ? ts0 : ts1) * W::TSLOT_DW;
        const uint32_t *tp = tslot + ((ks + 2) & 3) * 2 * WG_NT * W::TSTRIDE + t_lane;
        uint32_t X[W::NX], Y[W::NY];
#pragma unroll
        for (int q = 0; q < W::NX; ++q) X[q] = tp[q];
        const uint32_t *as_p = a_lane + as * W::ASLOT_DW;
        const uint32_t *xbn = xb_half0 + (cur ^ 1) * W::XB_DW;  // k-step i+1's fragments
        u32x4_t nb4;
        // x~ fragments in a ring read three ahead of their four products,
        // the next k-step's B fragments one per two products, and the decode
        // of k-step i+2 cut into six pieces between them
        constexpr int RD = 3;
        __builtin_amdgcn_sched_barrier(0);
        half8_t af[4];
#pragma unroll
        for (int q = 0; q < RD; ++q) af[q] = *(const half8_t *)(as_p + q * 256);
        static_for<0, MF>([&](auto mt_c) {
          constexpr int mt = decltype(mt_c)::value;
          if constexpr (mt + RD < MF) af[(mt + RD) % 4] = *(const half8_t *)(as_p + (mt + RD) * 256);
          if constexpr (mt % 2 == 1) B[cur ^ 1][mt / 2] = *(const half8_t *)(xbn + (mt / 2) * 512);
#pragma unroll
          for (int f = 0; f < NF; ++f)
            acc[mt][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt % 4], B[cur][f], acc[mt][f], 0, 0, 0);
          static_for<mt * 6 / MF, (mt + 1) * 6 / MF>([&](auto pc) {
            constexpr int piece = decltype(pc)::value;
            if constexpr (piece == 0) raw_normalize<BITS>(X, sel, sh, Y);
            else if constexpr (piece < 5) nb4[piece - 1] = frag_pair<BITS, CB, piece - 1>(Y);
            else *(u32x4_t *)(xb_own0 + cur * W::XB_DW) = nb4;  // k-step i+2's
          });
          __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (PH == 0) wait_vmcnt<W::A_WAIT>();
        else wait_vmcnt<W::t_wait(ks)>();
        barrier_lds();
      };
      kstep(std::integral_constant<int, 0>{});
      kstep(std::integral_constant<int, 1>{});
      kstep(std::integral_constant<int, 2>{});
      kstep(std::integral_constant<int, 3>{});
      ts0 = ts1;
      as_cur = (as_cur + 4) % ASLOTS;
    }
  };
  if (role == 0) run_stages(std::integral_constant<int, 0>{});
  else run_stages(std::integral_constant<int, 1>{});
  wait_vmcnt<0>();
  barrier_lds();

  int col[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) col[f] = lane_col(2 * ch + (f >> 1), j, f & 1);
  if (p.slab_mode) {
    const int rows = rend - p.row_base;
#pragma unroll
    for (int mt = 0; mt < MF; ++mt) {
      const int row0 = m0 - p.row_base + rq * 128 + mt * 16 + 4 * g;
#pragma unroll
      for (int f = 0; f < NF; ++f) store_partial(p.slabs, blockIdx.y, rows, N, row0, nb * 128 + col[f], acc[mt][f]);
    }
    return;
  }

  // output transform, one row quarter (128 rows) per pass through LDS
  float *z = reinterpret_cast<float *>(lds);
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
  const OutWords16 ow = out_words16(p.svh, p.bias, nb * 128, lane);
  const bool has_bias = p.bias != nullptr;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (pass > 0) barrier_lds();
    if (rq == pass) {
#pragma unroll
      for (int mt = 0; mt < MF; ++mt)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) z[(mt * 16 + 4 * g + i) * Z_ROW + col[f]] = acc[mt][f][i];
    }
    barrier_lds();
#pragma unroll
    for (int r0 = 8 * wave; r0 < W::ZR; r0 += 8 * W::WAVES) {
      if (p.out_bf16) output_rows8<true>(z, Z_ROW, r0, ow, has_bias, y, m0 + pass * W::ZR + r0, rend, N, nb * 128, lane);
      else output_rows8<false>(z, Z_ROW, r0, ow, has_bias, y, m0 + pass * W::ZR + r0, rend, N, nb * 128, lane);
    }
  }
}

// bm 128: 64-row waves, one part per workgroup (fused or slabs); bm 256:
// 128-row waves (both fold modes); bm 512: gemm_wide4_kernel, single part per
// workgroup only (the host never asks for the fold there).
template <int BITS, uint32_t CB>
hipError_t launch_wide_t(int bm, bool multi, const GemmParams &p, dim3 grid, hipStream_t s) {
  if (bm == 128 && !multi) {
    hipLaunchKernelGGL((gemm_wide_kernel<BITS, CB, 64, false>), grid, dim3(512), 0, s, p);
  } else if (bm == 256) {
    if (multi) hipLaunchKernelGGL((gemm_wide_kernel<BITS, CB, 128, true>), grid, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((gemm_wide_kernel<BITS, CB, 128, false>), grid, dim3(512), 0, s, p);
  } else if (bm == 512 && !multi) {
    hipLaunchKernelGGL((gemm_wide4_kernel<BITS, CB>), grid, dim3(512), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace exl3
