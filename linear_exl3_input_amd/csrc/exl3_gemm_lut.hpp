// Table-decode GEMM for M <= 32 rows.
//
// At a handful of rows the op streams the trellis once and its cost is the
// decode: the ALU decode of the tile kernels spends about five VALU
// instructions per weight, which on this GPU is fewer weights per clock than
// HBM delivers at 4..6 bits.  This kernel moves part of that work to the LDS
// pipe: every workgroup first fills a 65,536-entry table (state -> fp16
// value, 128 KB of LDS) with the same decode_pair the ALU path uses, so both
// give the same bits, and then decodes TP of the four state pairs of every
// half-fragment by table lookup (two and a half VALU instructions and one
// LDS gather per weight, against four and a half by the ALU) and the other
// 4 - TP by the ALU.
//
// The table fills the LDS, so one 1024-thread workgroup runs per CU and
// loops over work units; nothing is staged in LDS.  Each lane loads the 16
// consecutive states it needs (both column halves of its MFMA B fragment) as
// one window of 2..5 dwords straight from the trellis in HBM, in one or two
// buffer loads (a window of separate dword loads touches every cache line
// several times and runs at half the speed), and its 8 x~ values, four
// k-steps ahead; the window is normalized once and all 16 states are cut out
// at compile-time bit offsets.
//
// Work: a unit is one 128-column block and the parts of one workgroup unit
// (slab mode: p.unit consecutive parts, their sum stored as one slab) or all
// parts (fused mode), folded in part order at every part end.  Grouped
// (MoE) calls, fused only: a unit is one 16-row block of routed rows and one
// column block, multiplied by the block's expert (trellis, svh and bias at
// fixed strides behind expert 0's), blocks of no expert skipped; the parts
// are folded as the shape's two-level tree (p.fold_q parts a group, first
// part of each group copied, then the groups in order, first copied), the
// same adds as the output kernel and the finishing workgroup.  The 16
// waves are 4 teams of 4 waves; wave tw of a team multiplies n-tiles 2tw,
// 2tw+1 against the (up to) 16 rows.  Units are dealt to the workgroups in
// turn (unit u to workgroup u mod G, team (u / G) mod 4).  A team walks its units as one
// continuous stream of k-steps, so the loads of the next unit are in flight
// while the current one finishes.  Same MFMA shape, k-slot order, k-step
// order and parts as the tile kernels, so the same bits.
#pragma once

#include "exl3_gemm.hpp"

namespace exl3 {

constexpr int TBL_THREADS = 1024;
constexpr int TBL_TEAMS = 4;
constexpr int TBL_DEPTH = 4;  // k-steps in flight per lane; divides every unit's k-step count

template <int BITS>
struct TblGeom {
  static constexpr int TILE_DW = 8 * BITS;
  // the lane's 16 states span 15*BITS + 16 bits from a 16-bit aligned start
  static constexpr int NY = (15 * BITS + 16 + 31) / 32;
  // odd widths start mid-dword on half the lanes: one more dword
  static constexpr int NX = NY + (BITS % 2);
};

// Byte offset 2*s in the table of the 16-bit state s that starts D bits into Y.
template <int D, int NY>
__device__ __forceinline__ uint32_t table_offset(const uint32_t (&Y)[NY]) {
  constexpr int a = D / 32;
  constexpr int s = D % 32;
  if constexpr (s <= 15) return (Y[a] >> (15 - s)) & 0x1FFFEu;
  else return __builtin_amdgcn_alignbit(Y[a], Y[a + 1], 47 - s) & 0x1FFFEu;
}

// First state of pair k of column half h, in MFMA slot order (states
// v0+4h + 0,1 | 8,9 | 2,3 | 10,11 for k = 0..3), as a bit offset into Y.
template <int BITS, int H, int K>
constexpr int pair_bit() {
  return (4 * H + (K == 0 ? 0 : K == 1 ? 8 : K == 2 ? 2 : 10)) * BITS;
}

// Pairs 0 .. TP-1 of half H by table: two 16-bit LDS reads per pair,
// packed into one register.  (The pair is packed by the ALU: 16-bit loads
// into the high half of a register do not keep its low half when the LDS
// runs with SRAM ECC, as on this GPU.)  The table is at LDS offset 0.
template <int BITS, int TP, int H>
__device__ __forceinline__ void table_pairs_of(const uint32_t (&Y)[TblGeom<BITS>::NY], const uint8_t *table,
                                               u32x4_t &f) {
  constexpr int NY = TblGeom<BITS>::NY;
  static_for<0, TP>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int D = pair_bit<BITS, H, k>();
    const uint32_t lo = *(const uint16_t *)(table + table_offset<D, NY>(Y));
    const uint32_t hi = *(const uint16_t *)(table + table_offset<D + BITS, NY>(Y));
    f[k] = lo | (hi << 16);
  });
}

template <int BITS, uint32_t CB, int TP, int H>
__device__ __forceinline__ void alu_pairs(const uint32_t (&Y)[TblGeom<BITS>::NY], u32x4_t &f) {
  constexpr int NY = TblGeom<BITS>::NY;
  static_for<TP, 4>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int D = pair_bit<BITS, H, k>();
    f[k] = decode_pair<CB>(window16<D, NY>(Y), window16<D + BITS, NY>(Y));
  });
}

// The wave-uniform description of one work unit.
struct TblUnit {
  uint32_t t;     // trellis byte offset of the unit's first k-step: tile (first k-tile, n-tile 0 of the block)
  const char *a;  // x~ bytes of the unit's first k-step (row 0, k-group 0)
  int nks;        // k-steps (4 per 128-k block; 0: no unit)
  int nb, part;   // column block; first part of the unit
  int slab;       // slab mode: the unit's slab
  int kb_begin;
  int rb, e;      // grouped calls: row block and its expert
};

// TEAMS teams of 4 waves: 4 (1024 threads, 128 VGPRs a wave) up to 32 rows,
// 2 (512 threads, 256 VGPRs) for the four A fragments of up to 64 rows.
template <int BITS, uint32_t CB, int TP, int MT, int TEAMS = 4, bool MOE = false>
__global__ __launch_bounds__(256 * TEAMS, 1) void gemm_table_kernel(const GemmParams p) {
  static_assert(!MOE || MT == 1, "grouped calls take 16-row blocks");
  using G = TblGeom<BITS>;
  constexpr int NX = G::NX, NY = G::NY, TILE_DW = G::TILE_DW;
  constexpr int DEPTH = TBL_DEPTH;
  // [0, 128 KB): the table; [128 KB, 160 KB): per team 16 rows x 128 fp32
  __shared__ __attribute__((aligned(16))) uint32_t lds[40960];
  float *const zbuf_all = reinterpret_cast<float *>(lds + 32768);
  const uint8_t *const table = reinterpret_cast<const uint8_t *>(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave >> 2;
  const int tw = wave & 3;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int M = p.M, K = p.K, N = p.N;
  const int NT = N >> 4;
  const int KB = K >> 7;
  const int P = p.parts;
  const int nblk = N >> 7;
  const bool slab = p.slab_mode != 0;
  const int NU = P / p.unit;  // units per column block (slab mode)
  const int rows = p.row_end - p.row_base;
  const int units = MOE ? (rows >> 4) * nblk : slab ? nblk * NU : nblk;
  const int stride = gridDim.x * TEAMS;
  const int rounds = (units + stride - 1) / stride;

  const int64_t tsb = (int64_t)2 * NT * TILE_DW * 4;  // trellis bytes per k-step (two k-tiles)
  const int64_t asb = (int64_t)M * 64;                // x~ bytes per k-step
  const char *const xrot = reinterpret_cast<const char *>(p.x_rot);
  // The trellis through a buffer resource (at most 2 GiB, checked on the
  // host): 32-bit offsets, and a read past its end returns zeros.
  const uint64_t expert_bytes = (uint64_t)K * (uint64_t)N * BITS / 8;
  const uint32_t t_bytes = (uint32_t)(MOE ? expert_bytes * (uint64_t)p.n_experts : expert_bytes);
  const auto trs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.trellis), (short)0, (int)t_bytes,
                                                     0x00020000);

  auto make_unit = [&](int r) __attribute__((always_inline)) {
    TblUnit u;
    // units go round the workgroups first, so that fewer units than teams
    // still spread over every CU
    const int id = (r * TEAMS + team) * (int)gridDim.x + (int)blockIdx.x;
    u.t = 0;
    u.a = xrot;
    u.nks = 0;
    u.nb = 0;
    u.part = 0;
    u.slab = 0;
    u.kb_begin = 0;
    u.rb = 0;
    u.e = 0;
    if (r >= rounds || id >= units) return u;
    if constexpr (MOE) {
      // units run through the column blocks of one row block, then the next
      u.rb = __builtin_amdgcn_readfirstlane(id / nblk);
      u.nb = id - u.rb * nblk;
      const int e = __builtin_amdgcn_readfirstlane(p.block_expert[u.rb]);
      if (e < 0 || e >= p.n_experts) return u;  // no expert: skipped, nothing written
      u.e = e;
      u.nks = 4 * KB;
      u.t = (uint32_t)((uint64_t)e * expert_bytes + (uint64_t)u.nb * 8 * (TILE_DW * 4));
      int shard = 0;
      while (shard + 1 < p.n_shards && u.nb >= p.shard_end_blk[shard]) ++shard;
      u.a = xrot + ((int64_t)shard * M * K + (int64_t)u.rb * 16 * 32) * 2;
      return u;
    }
    // the divisions run on the vector unit: keep their (wave-uniform)
    // results in scalar registers, so the addresses built from them are too
    u.nb = __builtin_amdgcn_readfirstlane(slab ? id / NU : id);
    u.slab = slab ? id - u.nb * NU : 0;
    u.part = u.slab * p.unit;
    u.kb_begin = __builtin_amdgcn_readfirstlane((int)((int64_t)u.part * KB / P));
    const int kb_end = __builtin_amdgcn_readfirstlane((int)((int64_t)(u.part + p.unit) * KB / P));
    u.nks = 4 * (kb_end - u.kb_begin);
    int shard = 0;
    while (shard + 1 < p.n_shards && u.nb >= p.shard_end_blk[shard]) ++shard;
    u.t = (uint32_t)(((int64_t)u.kb_begin * 8 * NT + u.nb * 8) * (TILE_DW * 4));
    u.a = xrot + ((int64_t)shard * M * K + (int64_t)u.kb_begin * 4 * M * 32) * 2;
    return u;
  };

  // ---- per-lane window: the lane's states v0 .. v0+15 of its tile, v0 =
  // 32*(j&7) + 16*(g&1), start bit v0*BITS (a multiple of 16); the tile is
  // k-tile (g>>1) of the k-step, n-tile 2tw + (j>>3) of the block.  The
  // window is NX dwords from dword d of the tile, read as one load; on the
  // lanes where it runs past the tile's end (the stream is circular) its
  // last dword is the tile's first, read by a second load.  Slot sl of a
  // group of DEPTH k-steps is k-step sl after the group's first: the
  // offsets include sl k-steps, so a group's loads share one scalar offset.
  uint32_t t_win[DEPTH], t_first[DEPTH], a_off[DEPTH][MT];
  uint32_t sel;
  bool wraps;
  {
    const int o = (32 * (j & 7) + 16 * (g & 1)) * BITS;
    const int d = o >> 5;
    const uint32_t tile = (uint32_t)((g >> 1) * NT + 2 * tw + (j >> 3)) * (TILE_DW * 4);
    wraps = d + NX > TILE_DW;
#pragma unroll
    for (int sl = 0; sl < DEPTH; ++sl) {
      t_win[sl] = tile + 4u * d + (uint32_t)(sl * tsb);
      t_first[sl] = tile + (uint32_t)(sl * tsb);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // row 16*mt + j; rows past the launch's last read that row (finite;
        // their results are never stored)
        const int row = 16 * mt + j < rows ? 16 * mt + j : rows - 1;
        a_off[sl][mt] = (uint32_t)((p.row_base + row) * 64 + 16 * g) + (uint32_t)(sl * asb);
      }
    }
    // raw dwords hold two stream words swapped; a start on a dword boundary
    // swaps them back, a start mid-dword takes the high word of X[i] and the
    // low word of X[i+1]
    sel = (o & 31) ? 0x03020504u : 0x01000302u;
  }

  uint32_t X[DEPTH][NX];
  uint32_t T0[DEPTH];
  half8_t A[DEPTH][MT];

  // (The empty asm keeps the x~ offset next to its load, so the load takes
  // the scalar-base + 32-bit-offset form instead of a 64-bit address built
  // per lane.)
  auto load_slot = [&](auto slot_c, uint32_t to, const char *ap) __attribute__((always_inline)) {
    constexpr int sl = decltype(slot_c)::value;
    if constexpr (NX == 2) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(trs, t_win[sl], to, 0);
      X[sl][0] = v.x;
      X[sl][1] = v.y;
    } else if constexpr (NX == 3) {
      typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
      const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(trs, t_win[sl], to, 0);
      X[sl][0] = v.x;
      X[sl][1] = v.y;
      X[sl][2] = v.z;
    } else {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(trs, t_win[sl], to, 0);
      X[sl][0] = v.x;
      X[sl][1] = v.y;
      X[sl][2] = v.z;
      X[sl][3] = v.w;
      if constexpr (NX == 5) X[sl][4] = __builtin_amdgcn_raw_buffer_load_b32(trs, t_win[sl] + 16u, to, 0);
    }
    T0[sl] = __builtin_amdgcn_raw_buffer_load_b32(trs, t_first[sl], to, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      asm volatile("" : "+v"(a_off[sl][mt]));
      A[sl][mt] = *(const half8_t *)(ap + a_off[sl][mt]);
    }
  };

  TblUnit cu = make_unit(0);
  TblUnit nu = make_unit(1);
  // a team without units still loads (unit 0's address, never used) so
  // that every slot is defined
  static_for<0, DEPTH>([&](auto sc) { load_slot(sc, cu.t, cu.a); });

  // ---- the table, two states per thread and store (overlaps the first loads)
  for (int s2 = tid; s2 < 32768; s2 += 256 * TEAMS) lds[s2] = decode_pair<CB>(2 * s2, 2 * s2 + 1);
  barrier_lds();

  for (int r = 0; r < rounds; ++r) {
    float4_t acc0[MT], acc1[MT], tot0[MT], tot1[MT], gs0[MT], gs1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc0[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
      acc1[mt] = acc0[mt];
      tot0[mt] = acc0[mt];
      tot1[mt] = acc0[mt];
      gs0[mt] = acc0[mt];
      gs1[mt] = acc0[mt];
    }
    if (cu.nks > 0) {
      // fold at every part end (first part copied, later parts added in
      // part order); part q ends at block floor((q+1)*KB/P)
      int fold_part = cu.part;
      int fold_ks = 4 * ((int)((int64_t)(fold_part + 1) * KB / P) - cu.kb_begin);
      // refills: k-steps ks0+DEPTH.. of this unit, else the next unit's
      // first DEPTH, else (no next unit) this group again, unused
      uint32_t rt = cu.t;
      const char *ra = cu.a;
      for (int ks0 = 0; ks0 < cu.nks; ks0 += DEPTH) {
        if (ks0 + DEPTH < cu.nks) {
          rt += (uint32_t)(DEPTH * tsb);
          ra += DEPTH * asb;
        } else if (nu.nks > 0) {
          rt = nu.t;
          ra = nu.a;
        }
        static_for<0, DEPTH>([&](auto sc) {
          constexpr int sl = decltype(sc)::value;
          uint32_t W[NX];
#pragma unroll
          for (int i = 0; i < NX; ++i) W[i] = X[sl][i];
          W[NX - 1] = wraps ? T0[sl] : W[NX - 1];
          uint32_t Y[NY];
#pragma unroll
          for (int i = 0; i < NY; ++i) {
            if constexpr (BITS % 2) Y[i] = __builtin_amdgcn_perm(W[i + 1], W[i], sel);
            else Y[i] = __builtin_amdgcn_alignbit(W[i], W[i], 16);
          }
          u32x4_t f0, f1;
          table_pairs_of<BITS, TP, 0>(Y, table, f0);
          table_pairs_of<BITS, TP, 1>(Y, table, f1);
          alu_pairs<BITS, CB, TP, 0>(Y, f0);
          alu_pairs<BITS, CB, TP, 1>(Y, f1);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            acc0[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[sl][mt], __builtin_bit_cast(half8_t, f0), acc0[mt], 0,
                                                              0, 0);
            acc1[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[sl][mt], __builtin_bit_cast(half8_t, f1), acc1[mt], 0,
                                                              0, 0);
          }
          load_slot(sc, rt, ra);
        });
        if (ks0 + DEPTH == fold_ks) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if constexpr (MOE) {
              const int q = p.fold_q;
              const int qi = fold_part % q;
              if (qi == 0) {
                gs0[mt] = acc0[mt];
                gs1[mt] = acc1[mt];
              } else {
                gs0[mt] = gs0[mt] + acc0[mt];
                gs1[mt] = gs1[mt] + acc1[mt];
              }
              if (qi == q - 1) {
                if (fold_part == q - 1) {
                  tot0[mt] = gs0[mt];
                  tot1[mt] = gs1[mt];
                } else {
                  tot0[mt] = tot0[mt] + gs0[mt];
                  tot1[mt] = tot1[mt] + gs1[mt];
                }
              }
            } else if (fold_part == cu.part) {
              tot0[mt] = acc0[mt];
              tot1[mt] = acc1[mt];
            } else {
              tot0[mt] = tot0[mt] + acc0[mt];
              tot1[mt] = tot1[mt] + acc1[mt];
            }
            acc0[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
            acc1[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
          }
          ++fold_part;
          fold_ks = 4 * ((int)((int64_t)(fold_part + 1) * KB / P) - cu.kb_begin);
        }
      }
    }
    if (slab && !MOE) {
      if (cu.nks > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          store_partial(p.slabs, cu.slab, rows, N, 16 * mt + 4 * g, cu.nb * 128 + lane_col(tw, j, 0), tot0[mt]);
          store_partial(p.slabs, cu.slab, rows, N, 16 * mt + 4 * g, cu.nb * 128 + lane_col(tw, j, 1), tot1[mt]);
        }
      }
    } else {
      // output transform of the team's block through its LDS rows, 16 rows
      // at a time; every wave of the workgroup takes part in the barriers
      float *const zb = zbuf_all + team * (16 * 128);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          zb[(4 * g + i) * 128 + lane_col(tw, j, 0)] = tot0[mt][i];
          zb[(4 * g + i) * 128 + lane_col(tw, j, 1)] = tot1[mt][i];
        }
        barrier_lds();
        if (cu.nks > 0 && tw < 2 && 16 * mt + 8 * tw < rows) {
          uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
          // grouped calls: the block's expert's svh and bias, its 16 rows
          const uint16_t *const svh = MOE ? p.svh + (int64_t)cu.e * N : p.svh;
          const uint16_t *const bias = MOE && p.bias != nullptr ? p.bias + (int64_t)cu.e * N : p.bias;
          const int64_t rbase = MOE ? (int64_t)p.row_base + 16 * cu.rb : (int64_t)p.row_base;
          const int64_t rlim = MOE ? rbase + 16 : (int64_t)p.row_base + rows;
          const OutWords16 ow = out_words16(svh, bias, cu.nb * 128, lane);
          const int64_t row0 = rbase + 16 * mt + 8 * tw;
          if (p.out_bf16)
            output_rows8<true>(zb, 128, 8 * tw, ow, bias != nullptr, y, row0, rlim, N, cu.nb * 128, lane);
          else
            output_rows8<false>(zb, 128, 8 * tw, ow, bias != nullptr, y, row0, rlim, N, cu.nb * 128, lane);
        }
        barrier_lds();
      }
    }
    cu = nu;
    nu = make_unit(r + 2);
  }
}

// Pairs of every half-fragment decoded by table (the other 4 - TP by the
// ALU).  Two balances the two pipes on gfx950: at 6 bits and one row, one
// pair is 4% slower (VALU-bound), three 8% and four 25% slower (LDS-bound:
// a random 16-bit gather costs about 7 LDS cycles, 5 of them bank
// conflicts).  EXL3_TABLE_PAIRS overrides it at build time for measurement.
#ifdef EXL3_TABLE_PAIRS
constexpr int table_pairs(int) { return EXL3_TABLE_PAIRS; }
#else
constexpr int table_pairs(int) { return 2; }
#endif

// One 16-row A fragment per decoded B operand up to 16 rows, two up to 32,
// four (two teams per workgroup) up to 64.
template <int BITS, uint32_t CB>
hipError_t launch_table_t(const GemmParams &p, int grid, hipStream_t s) {
  constexpr int TP = table_pairs(BITS);
  const int rows = p.row_end - p.row_base;
  if (p.block_expert != nullptr) {
    hipLaunchKernelGGL((gemm_table_kernel<BITS, CB, TP, 1, 4, true>), dim3(grid), dim3(TBL_THREADS), 0, s, p);
    return hipGetLastError();
  }
  if (rows <= 16) hipLaunchKernelGGL((gemm_table_kernel<BITS, CB, TP, 1>), dim3(grid), dim3(TBL_THREADS), 0, s, p);
  else if (rows <= 32) hipLaunchKernelGGL((gemm_table_kernel<BITS, CB, TP, 2>), dim3(grid), dim3(TBL_THREADS), 0, s, p);
  else if (rows <= 64) hipLaunchKernelGGL((gemm_table_kernel<BITS, CB, TP, 4, 2>), dim3(grid), dim3(512), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_table_bits(int cb, const GemmParams &p, int grid, hipStream_t s) {
  switch (cb) {
    case 0: return launch_table_t<BITS, CB_3INST>(p, grid, s);
    case 1: return launch_table_t<BITS, CB_MCG>(p, grid, s);
    case 2: return launch_table_t<BITS, CB_MUL1>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace exl3
