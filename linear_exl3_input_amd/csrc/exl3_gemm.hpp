// Trellis-decode + MFMA GEMM of the EXL3 linear for gfx950.
//
// One workgroup (4 waves) owns a BM-row x 128-column output tile (one
// Hadamard block of columns, so the output transform can be applied in the
// same kernel) and a range of K.  The trellis slice it needs is streamed from
// HBM once per M-tile (cuda-exl3 README, "Why custom kernels": a block owns
// BM rows x BN columns and reads its trellis slice once), 128 k at a time,
// through a two-stage LDS pipeline.  Each wave decodes the tiles of its two
// 16-column strips straight into the B operand of v_mfma_f32_16x16x32_f16;
// every trellis value is decoded exactly once per M-tile (cuda-exl3 README,
// "What profiling found": decoding each tile once was the small-batch win).
//
// Value placement.  A 16x16 tile lists its 256 values in the order of the B
// fragments of two m16n8k16 products (TensorFold PR "cuda: EXL3 projections
// behind qlinear", "Arithmetic" step 2): value v = 8t + 4h + i sits at row
// k = 2(t%4) + (i&1) + 8(i>>1), column n = t/4 + 8h.  One MFMA B operand is
// 32 k x 16 columns.  Lane (j = lane%16, g = lane/16) of MFMA "half" h takes
// column c = (j&7) + 8h of n-tile 2*wave + (j>>3) in k-tile g>>1, and the
// two runs of four consecutive states v0..v0+3 and v0+8..v0+11 with
// v0 = 32(j&7) + 4h + 16(g&1).  Those are rows 4(g&1) + {0,1,2,3,8,9,10,11}
// of the tile, so the lane's 8 k slots are that ascending list.  The A operand
// (rotated activations) is read at the same 8 k for row j; any k order works
// as long as A and B agree (the FP8 DenseMlp page makes the same point).
//
// Bit stream.  Tile words are MSB-first; value v's 16-bit state starts at
// bit v*bits and wraps around the tile (a run of eight 6-bit values spans a
// 58-bit window, cuda-exl3 README, "Where the time goes").  While staging,
// each 32-bit word is rotated by 16 so LDS holds the stream MSB-first per
// dword, and every tile is stored with 4 pad dwords on each side (copies of
// its last and first 4 dwords) so no lane's window wraps inside LDS.
//
// Summation structure (fixed by (K, N, bits), never by M): K is cut into P
// parts of whole 128-k blocks; each part is one MFMA chain in ascending k
// from zero; parts are added in part order, the first part copied, not added
// to zero (TensorFold PR, "Arithmetic": a number of parts fixed by the shape,
// added in part order).  In slab mode each workgroup runs one part and writes
// an fp32 partial (store_partial); otherwise one workgroup runs all parts and keeps the
// running sum in registers.  Both give the same bits for every row.
#pragma once

#include <type_traits>

#include "exl3_device.hpp"
#include "exl3_launch.hpp"

namespace exl3 {

constexpr int STAGE_KT = 8;      // k-tiles per pipeline stage (128 k)
constexpr int WG_NT = 8;         // n-tiles per workgroup (128 columns)
constexpr int WG_THREADS = 256;  // 4 waves
constexpr int A_ROW_DW = 68;     // staged x~ row: 128 fp16 (64 dwords) + 4 pad
constexpr int Z_ROW = 132;       // epilogue z row: 128 fp32 + 4 pad

template <int BITS>
struct Geom {
  static constexpr int TILE_DW = 8 * BITS;         // dwords per 16x16 tile
  static constexpr int STRIDE = TILE_DW + 8;       // LDS dwords per tile (4 + tile + 4)
  static constexpr int TILE_CHUNKS = 2 * BITS;     // 16-byte chunks per tile
  static constexpr int ROW_CHUNKS = WG_NT * TILE_CHUNKS;
  static constexpr int STAGE_CHUNKS = STAGE_KT * ROW_CHUNKS;
  static constexpr int T_ITERS = (STAGE_CHUNKS + WG_THREADS - 1) / WG_THREADS;
  static constexpr int T_MIN = STAGE_CHUNKS / WG_THREADS;  // loads every wave issues per stage
  static constexpr int STAGE_T_DW = STAGE_KT * WG_NT * STRIDE;
  // dwords a lane needs: 16 + 11*bits stream bits after a start offset in [1, 32]
  static constexpr int NY = (11 * BITS + 16 + 31) / 32;
  static constexpr int NX = NY + 1;
};

// ---------------------------------------------------------------- staging

template <int BITS>
__device__ __forceinline__ void load_trellis_stage(u32x4_t (&treg)[Geom<BITS>::T_ITERS],
                                                   const uint16_t *__restrict__ tr, int kb, int nb,
                                                   int NT, int tid) {
  using G = Geom<BITS>;
#pragma unroll
  for (int it = 0; it < G::T_ITERS; ++it) {
    const int c = tid + WG_THREADS * it;
    if (G::STAGE_CHUNKS % WG_THREADS == 0 || c < G::STAGE_CHUNKS) {
      const int r = c / G::ROW_CHUNKS;
      const int q = c - r * G::ROW_CHUNKS;
      const uint16_t *src = tr + ((int64_t)(STAGE_KT * kb + r) * NT + WG_NT * nb) * (16 * BITS) + q * 8;
      treg[it] = __builtin_nontemporal_load((const u32x4_t *)src);
    }
  }
}

__device__ __forceinline__ uint32_t rot16(uint32_t w) { return __builtin_amdgcn_alignbit(w, w, 16); }

template <int BITS>
__device__ __forceinline__ void store_trellis_stage(const u32x4_t (&treg)[Geom<BITS>::T_ITERS],
                                                    uint32_t *__restrict__ tb, int tid) {
  using G = Geom<BITS>;
#pragma unroll
  for (int it = 0; it < G::T_ITERS; ++it) {
    const int c = tid + WG_THREADS * it;
    if (G::STAGE_CHUNKS % WG_THREADS == 0 || c < G::STAGE_CHUNKS) {
      const int r = c / G::ROW_CHUNKS;
      const int q = c - r * G::ROW_CHUNKS;
      const int t = q / G::TILE_CHUNKS;
      const int u = q - t * G::TILE_CHUNKS;
      u32x4_t v = treg[it];
      v.x = rot16(v.x);
      v.y = rot16(v.y);
      v.z = rot16(v.z);
      v.w = rot16(v.w);
      uint32_t *dst = tb + (r * WG_NT + t) * G::STRIDE;
      *(u32x4_t *)(dst + 4 + 4 * u) = v;
      if (u == 0) *(u32x4_t *)(dst + 4 + G::TILE_DW) = v;
      if (u == G::TILE_CHUNKS - 1) *(u32x4_t *)(dst) = v;
    }
  }
}

// ----------------------------------------------------------------- decode

template <int D, int NY>
__device__ __forceinline__ uint32_t window16(const uint32_t (&Y)[NY]) {
  constexpr int a = D / 32;
  constexpr int s = D % 32;
  if constexpr (s <= 16) return Y[a] >> (16 - s);
  else return __builtin_amdgcn_alignbit(Y[a], Y[a + 1], 48 - s);
}

// Decode the lane's 8 values of one MFMA B operand from a staged tile.
// `tp` points at the tile's LDS slot; `xoff` is 4 + the first dword the lane
// needs and `sh` = 32 - (its bit offset in that dword, in 1..32).
template <int BITS, uint32_t CB>
__device__ __forceinline__ half8_t decode_frag(const uint32_t *__restrict__ tp, int xoff, int sh) {
  using G = Geom<BITS>;
  uint32_t X[G::NX];
#pragma unroll
  for (int i = 0; i < G::NX; ++i) X[i] = tp[xoff + i];
  uint32_t Y[G::NY];
#pragma unroll
  for (int i = 0; i < G::NY; ++i) Y[i] = __builtin_amdgcn_alignbit(X[i], X[i + 1], sh);
  const uint32_t s0 = window16<0, G::NY>(Y);
  const uint32_t s1 = window16<BITS, G::NY>(Y);
  const uint32_t s2 = window16<8 * BITS, G::NY>(Y);
  const uint32_t s3 = window16<9 * BITS, G::NY>(Y);
  const uint32_t s4 = window16<2 * BITS, G::NY>(Y);
  const uint32_t s5 = window16<3 * BITS, G::NY>(Y);
  const uint32_t s6 = window16<10 * BITS, G::NY>(Y);
  const uint32_t s7 = window16<11 * BITS, G::NY>(Y);
  const u32x4_t r = {decode_pair<CB>(s0, s1), decode_pair<CB>(s2, s3), decode_pair<CB>(s4, s5),
                     decode_pair<CB>(s6, s7)};
  return __builtin_bit_cast(half8_t, r);
}

// decode_frag in pieces, so that a caller can spread the work between
// matrix-core instructions: load the lane's dwords, normalize them, then
// produce one packed pair of values (k = 0..3) at a time.
template <int BITS>
__device__ __forceinline__ void frag_load(const uint32_t *__restrict__ tp, int xoff, uint32_t (&X)[Geom<BITS>::NX]) {
#pragma unroll
  for (int i = 0; i < Geom<BITS>::NX; ++i) X[i] = tp[xoff + i];
}

template <int BITS>
__device__ __forceinline__ void frag_normalize(const uint32_t (&X)[Geom<BITS>::NX], int sh,
                                               uint32_t (&Y)[Geom<BITS>::NY]) {
#pragma unroll
  for (int i = 0; i < Geom<BITS>::NY; ++i) Y[i] = __builtin_amdgcn_alignbit(X[i], X[i + 1], sh);
}

template <int BITS, uint32_t CB, int K>
__device__ __forceinline__ uint32_t frag_pair(const uint32_t (&Y)[Geom<BITS>::NY]) {
  // slot order of the lane's states: v0, v0+1, v0+8, v0+9, v0+2, v0+3, v0+10, v0+11
  constexpr int D0 = (K == 0 ? 0 : K == 1 ? 8 : K == 2 ? 2 : 10) * BITS;
  constexpr int D1 = D0 + BITS;
  return decode_pair<CB>(window16<D0, Geom<BITS>::NY>(Y), window16<D1, Geom<BITS>::NY>(Y));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Per-lane constants of decode_frag for column half h.
template <int BITS>
__device__ __forceinline__ void lane_window(int j, int g, int h, int &xoff, int &sh) {
  const int v0 = 32 * (j & 7) + 4 * h + 16 * (g & 1);
  const int o = v0 * BITS;
  const int d0 = (o + 31) / 32 - 1;  // so that o - 32*d0 is in 1..32
  xoff = 4 + d0;
  sh = 32 - (o - 32 * d0);
}

// Column (within the workgroup's 128) of the lane's B column / C column.
__device__ __forceinline__ int lane_col(int wave, int j, int h) {
  return 16 * (2 * wave + (j >> 3)) + (j & 7) + 8 * h;
}

// Workgroup barrier that waits only for this wave's LDS operations.
// __syncthreads() also drains every outstanding global load (the release
// fence of the memory model), which would cancel the direct-to-LDS prefetch
// that is meant to stay in flight across barriers; completion of those loads
// is tracked explicitly with wait_vmcnt.
// The wait is the builtin (s_waitcnt lgkmcnt(0), encoding 0xC07F) so the
// compiler's own wait insertion knows LDS results are in after it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ------------------------------------------------------------ raw tiles
//
// Trellis tiles loaded straight to LDS (global_load_lds_dwordx4) are stored
// raw: the 16-bit words as in memory, so each dword holds two stream words in
// swapped order.  Each tile gets one 16-byte pad chunk on each side (its last
// chunk before it, its first chunk after it), so no lane's window wraps.  A
// stage (128 k x 128 columns = 8 x 8 tiles, tile t = 8*ktile + ntile) is
// 64 * (2*BITS + 2) chunks.

template <int BITS>
struct RawGeom {
  static constexpr int TSTRIDE = 8 * BITS + 8;          // dwords per padded tile
  static constexpr int T_CHUNKS = 64 * (2 * BITS + 2);  // 16-byte chunks per padded stage
  static constexpr int TSLOT_DW = T_CHUNKS * 4;
  static constexpr int NY = Geom<BITS>::NY;
  static constexpr int NX = Geom<BITS>::NX;
  static constexpr bool PERM = BITS % 2 == 0;
};

// Source offset (16-bit words from the stage's first tile) of padded chunk
// q of a stage; q past the stage (surplus lanes of the last load) reads a
// chunk of tile 0 that lands in a scratch area.
// A stage is 8 k-tiles x NTS n-tiles (NTS = 8: 128 columns, 4: 64).
template <int BITS, int NTS = 8>
__device__ __forceinline__ uint32_t raw_chunk_src(int q, int NT) {
  constexpr int TC = 2 * BITS + 2;
  if (q >= 8 * NTS * TC) return (uint32_t)((q % (2 * BITS)) * 8);
  const int t = q / TC;
  const int c = q - t * TC;
  const int sc = c == 0 ? 2 * BITS - 1 : (c == 2 * BITS + 1 ? 0 : c - 1);
  return (uint32_t)(((t / NTS) * NT + (t % NTS)) * (16 * BITS) + sc * 8);
}

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

// Per-lane window constants for half h: start dword, perm selector (even
// widths) or alignbit shift (odd widths: each dword is rotated by 16 first).
template <int BITS>
__device__ __forceinline__ void raw_lane_window(int j, int g, int h, int &doff, uint32_t &sel, int &sh) {
  sel = 0;
  sh = 0;
  if constexpr (RawGeom<BITS>::PERM) lane_window_perm<BITS>(j, g, h, doff, sel);
  else lane_window<BITS>(j, g, h, doff, sh);
}

template <int BITS>
__device__ __forceinline__ void raw_normalize(const uint32_t (&X)[Geom<BITS>::NX], uint32_t sel, int sh,
                                              uint32_t (&Y)[Geom<BITS>::NY]) {
  using R = RawGeom<BITS>;
  if constexpr (R::PERM) {
#pragma unroll
    for (int i = 0; i < R::NY; ++i) Y[i] = __builtin_amdgcn_perm(X[i + 1], X[i], sel);
  } else {
    uint32_t Z[R::NX];
#pragma unroll
    for (int i = 0; i < R::NX; ++i) Z[i] = rot16(X[i]);
#pragma unroll
    for (int i = 0; i < R::NY; ++i) Y[i] = __builtin_amdgcn_alignbit(Z[i], Z[i + 1], sh);
  }
}

// The lane's 8 values of one B operand from a raw tile (tp = tile start +
// doff in LDS).
template <int BITS, uint32_t CB>
__device__ __forceinline__ u32x4_t raw_decode_frag(const uint32_t *__restrict__ tp, uint32_t sel, int sh) {
  uint32_t X[Geom<BITS>::NX], Y[Geom<BITS>::NY];
#pragma unroll
  for (int i = 0; i < Geom<BITS>::NX; ++i) X[i] = tp[i];
  raw_normalize<BITS>(X, sel, sh, Y);
  return u32x4_t{frag_pair<BITS, CB, 0>(Y), frag_pair<BITS, CB, 1>(Y), frag_pair<BITS, CB, 2>(Y),
                 frag_pair<BITS, CB, 3>(Y)};
}

// ------------------------------------------------------------------- GEMM

// One accumulator of a lane (slab rows row0 .. row0+3 of column col; row0 is
// a multiple of 4) into partial slab `slab`.  Slabs are laid out
// [slab][rows/4][N][4] (rows padded to a multiple of 4, padding rows hold
// finite values of clamped rows): a lane's four values are one 16-byte store
// and a wave's stores fill whole cache lines.
__device__ __forceinline__ void store_partial(float *__restrict__ slabs, int slab, int rows, int N, int row0, int col,
                                              float4_t v) {
  if (row0 < rows) {
    const int64_t M4 = (rows + 3) >> 2;
    *(float4_t *)(slabs + (((int64_t)slab * M4 + (row0 >> 2)) * N + col) * 4) = v;
  }
}

// ------------------------------------------------------------ finisher
//
// The last of a tile's workgroups to finish adds the tile's partial slabs in
// order and applies the output stage (TensorFold PR, "Arithmetic": the last
// part to finish adds the parts in part order).  No workgroup waits for
// another, so nothing can hang.
//
// Visibility across the GPU's L2 caches (one per XCD) without fences that
// write back and invalidate a whole L2 (measured at 10-30 us per call): the
// partials are written with device-coherent stores (sc1, the cache policy of
// an agent-scope atomic store) and every writer waits until its stores have
// completed (vmcnt 0) before the workgroup counts its arrival with an
// agent-scope atomic add; the last workgroup to arrive reads the partials
// with device-coherent loads (sc1).  Slab bytes stay below 2 GiB (32-bit
// buffer offsets; the host caps slabs far lower).

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const GemmParams &p) {
  const int rows = p.row_end - p.row_base;
  const uint32_t bytes = (uint32_t)((int64_t)gridDim.y * ((rows + 3) >> 2) * p.N * 16);
  return __builtin_amdgcn_make_buffer_rsrc(p.slabs, (short)0, (int)bytes, 0x00020000);
}

constexpr int CPOL_SC1 = 16;  // device-scope coherent access

// store_partial through the coherent path.
__device__ __forceinline__ void store_partial_coherent(__amdgpu_buffer_rsrc_t rs, int slab, int rows, int N,
                                                       int row0, int col, float4_t v) {
  if (row0 < rows) {
    const uint32_t M4 = (uint32_t)((rows + 3) >> 2);
    const uint32_t off = (((uint32_t)slab * M4 + (uint32_t)(row0 >> 2)) * (uint32_t)N + (uint32_t)col) * 16u;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rs, off, 0, CPOL_SC1);
  }
}

// The ordered sum (reduce_rows4's order: fold_q slabs per group, then the
// groups) of four rows of one 128-column block read through the coherent
// path, U slabs' loads in flight per round trip, then the output stage of
// the `rows` (<= 4) rows.  slab_stride: bytes per slab.
template <int U>
__device__ __forceinline__ void fold_rows4_coherent(__amdgpu_buffer_rsrc_t rs, int n_slabs, int fq,
                                                    uint32_t slab_stride, int N, int m4, int n0,
                                                    const GemmParams &p, OutWords ow, bool has_bias,
                                                    int64_t row0, int rows, int lane) {
  const uint32_t base = ((uint32_t)m4 * (uint32_t)N + (uint32_t)(n0 + 2 * lane)) * 16u;
  float4_t t0 = {0.f, 0.f, 0.f, 0.f}, t1 = t0, g0 = t0, g1 = t0;
  int iq = 0;
  for (int i0 = 0; i0 < n_slabs; i0 += U) {
    float4_t v0[U], v1[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u < n_slabs) {
        const uint32_t off = (uint32_t)(i0 + u) * slab_stride + base;
        v0[u] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CPOL_SC1));
        v1[u] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, CPOL_SC1));
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u < n_slabs) {
        if (iq == 0) {
          g0 = v0[u];
          g1 = v1[u];
        } else {
          g0 = g0 + v0[u];
          g1 = g1 + v1[u];
        }
        if (++iq == fq) {
          iq = 0;
          if (i0 + u + 1 == fq) {
            t0 = g0;
            t1 = g1;
          } else {
            t0 = t0 + g0;
            t1 = t1 + g1;
          }
        }
      }
  }
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < rows) {
      if (p.out_bf16) output_row_words<true>(t0[i], t1[i], ow, has_bias, y + (row0 + i) * N, n0, lane);
      else output_row_words<false>(t0[i], t1[i], ow, has_bias, y + (row0 + i) * N, n0, lane);
    }
}

// Arrival: every thread's stores have completed; one thread adds 1 to the
// tile's counter.  Returns true (uniformly) in the last of the tile's
// `arrivals` workgroups.
__device__ __forceinline__ bool arrive_last(const GemmParams &p, uint32_t tile, uint32_t arrivals) {
  __shared__ int s_last;
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             arrivals - 1;
  __syncthreads();
  return s_last != 0;
}

// The last workgroup's work on its tile (rows m0 .. m0+bm-1 of the launch,
// the 128 columns of block nb), with n_waves waves and `lds_bytes` of
// free LDS at `lds`.  The tile's slabs form G = n_slabs / fold_q groups of
// fold_q consecutive slabs.  Items (4-row group r, group gi) are dealt to the
// waves: each folds its group's slabs in slab order (first copied) into LDS,
// so all loads of a wave's item are in flight together and the waves' items
// overlap; then wave r folds the group sums of 4-row group r in group order
// (first copied) and writes the rows.  The same fp32 adds in the same order as
// reduce_rows4 (which serves when the items do not fit the LDS).  ow: the
// lane's svh and bias words of the block, loaded before the arrival.  The
// tile's counter is reset to zero for the next call.
__device__ __forceinline__ void finish_tile(const GemmParams &p, OutWords ow, bool has_bias, uint32_t tile, int nb,
                                            int m0, int bm, int wave_all, int n_waves, int lane, float *lds,
                                            int lds_bytes) {
  const int rows = p.row_end - p.row_base;
  const int M4 = (rows + 3) >> 2;
  const int N = p.N;
  const int n_slabs = gridDim.y;
  const int fq = p.fold_q;
  const int G = n_slabs / fq;
  const int rt = min(bm, p.row_end - m0);  // rows of this tile
  const int r4 = (rt + 3) >> 2;
  const int n0 = nb * 128;
  const int m4_0 = (m0 - p.row_base) >> 2;
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
  const __amdgpu_buffer_rsrc_t rs = slab_rsrc(p);
  const uint32_t slab_stride = (uint32_t)M4 * (uint32_t)N * 16u;  // bytes per slab
  auto load2 = [&](int slab, int m4, float4_t &a, float4_t &b) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)slab * slab_stride + ((uint32_t)m4 * (uint32_t)N + (uint32_t)(n0 + 2 * lane)) * 16u;
    a = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CPOL_SC1));
    b = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, CPOL_SC1));
  };
  if (r4 * G * 2048 <= lds_bytes && fq <= 4) {
    float4_t *const gs = reinterpret_cast<float4_t *>(lds);  // [r][gi][lane][2]
    int it = wave_all;
    if (fq == 1) {
      // one slab per item (its group sum): two items' loads per round trip
      for (; it + n_waves < r4 * G; it += 2 * n_waves) {
        const int ita = it, itb = it + n_waves;
        const int ra = ita / G, rb = itb / G;
        float4_t a0, a1, b0, b1;
        load2(ita - ra * G, m4_0 + ra, a0, a1);
        load2(itb - rb * G, m4_0 + rb, b0, b1);
        gs[(ita * 64 + lane) * 2] = a0;
        gs[(ita * 64 + lane) * 2 + 1] = a1;
        gs[(itb * 64 + lane) * 2] = b0;
        gs[(itb * 64 + lane) * 2 + 1] = b1;
      }
    }
    for (; it < r4 * G; it += n_waves) {
      const int r = it / G;
      const int gi = it - r * G;
      float4_t v0[4], v1[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < fq) load2(gi * fq + q, m4_0 + r, v0[q], v1[q]);
      float4_t g0 = v0[0], g1 = v1[0];
#pragma unroll
      for (int q = 1; q < 4; ++q)
        if (q < fq) {
          g0 = g0 + v0[q];
          g1 = g1 + v1[q];
        }
      gs[(it * 64 + lane) * 2] = g0;
      gs[(it * 64 + lane) * 2 + 1] = g1;
    }
    __syncthreads();
    for (int r = wave_all; r < r4; r += n_waves) {
      float4_t t0 = gs[(r * G * 64 + lane) * 2], t1 = gs[(r * G * 64 + lane) * 2 + 1];
      for (int gi = 1; gi < G; ++gi) {
        t0 = t0 + gs[((r * G + gi) * 64 + lane) * 2];
        t1 = t1 + gs[((r * G + gi) * 64 + lane) * 2 + 1];
      }
      const int r0 = m0 + 4 * r;
      const int nr = min(4, p.row_end - r0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nr) {
          if (p.out_bf16) output_row_words<true>(t0[i], t1[i], ow, has_bias, y + (int64_t)(r0 + i) * N, n0, lane);
          else output_row_words<false>(t0[i], t1[i], ow, has_bias, y + (int64_t)(r0 + i) * N, n0, lane);
        }
    }
  } else {
    // one wave per 4-row group, slabs in order (reduce_rows4's order)
    for (int r = wave_all; r < r4; r += n_waves)
      fold_rows4_coherent<4>(rs, n_slabs, fq, slab_stride, N, m4_0 + r, n0, p, ow, has_bias, m0 + 4 * r,
                             min(4, p.row_end - (m0 + 4 * r)), lane);
  }
  if (threadIdx.x == 0) __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS dwords of one stage slot of gemm_kernel (raw trellis tiles + x~) and of
// a quad's private area (NSLOT slots + the landing area of surplus loads).
// A quad is QW waves on 32*QW columns (QW = 4: a whole 128-column block;
// QW = 2: half of one).
template <int BITS, int MT, int QW>
struct SmallGeom {
  static constexpr int BM = 16 * MT;
  static constexpr int QT = 64 * QW;                        // threads per quad
  static constexpr int NTS = 2 * QW;                        // n-tiles per stage row
  static constexpr int TSTRIDE = 8 * BITS + 8;              // dwords per padded tile
  static constexpr int T_CHUNKS = 8 * NTS * (2 * BITS + 2);  // 16-byte chunks per padded stage
  static constexpr int TSLOT_DW = T_CHUNKS * 4;
  static constexpr int T_OPS = (T_CHUNKS + QT - 1) / QT;    // trellis loads per wave per stage
  static constexpr int JUNK = T_OPS * QT - T_CHUNKS;
  static constexpr int A_SLOT_DW = BM * 64;                 // x~: 4 k-steps x BM rows x 64 B
  static constexpr int A_OPS = 16 * BM / QT;                // x~ loads per wave per stage
  static constexpr int SLOT_DW = TSLOT_DW + A_SLOT_DW;
  static constexpr int OPS = T_OPS + A_OPS;                 // loads per wave per stage
  static constexpr int area(int nslot) { return nslot * SLOT_DW + JUNK * 4; }
  static_assert(16 * BM % QT == 0, "x~ loads divide evenly over the quad");
  static_assert(T_CHUNKS % 64 == 0, "each direct load lands whole in a slot or in the surplus area");
};

// BM = 16*MT rows (16, 32, 64) x 32*QW columns (QW = 4: one 128-column
// block; QW = 2: half of one, so that a layer with few tiles keeps twice the
// workgroups, slab mode only).  A workgroup is QD quads of QW waves; quad q
// computes K part (unit start + q) when QD > 1, or the whole unit (MULTI: its
// parts folded in order in registers) when QD == 1.  Wave w of a quad
// decodes n-tiles 2w, 2w+1 of its columns (both column halves) and
// multiplies them against all BM rows.  Both operands arrive by direct loads to LDS into the
// quad's stage slots (raw trellis tiles, and x~ in its k-step tile layout, 4
// k-steps x BM rows x 64 B per stage): two slots, the first two stages issued
// together, when QD quads of two slots fit in LDS, else one slot.  Barriers
// wait only for LDS operations; the loads are waited for by count.  The
// quads' part sums are then folded in part order through LDS.  Rows past the
// launch's last row load that row (finite, never stored).
template <int BITS, uint32_t CB, int MT, bool MULTI, int QD, int QW, bool MOE>
__global__ __launch_bounds__(64 * QW * QD) void gemm_kernel(const GemmParams p) {
  using S = SmallGeom<BITS, MT, QW>;
  constexpr int BM = S::BM;
  constexpr int QT = S::QT;
  constexpr int NTS = S::NTS;
  constexpr int T_OPS = S::T_OPS;
  constexpr int A_OPS = S::A_OPS;
  constexpr int OPS = S::OPS;
  constexpr int SLOT_DW = S::SLOT_DW;
  constexpr int TSTRIDE = S::TSTRIDE;
  constexpr int NSLOT = small_tile_slots(BITS, MT, QW, QD);
  static_assert(NSLOT == (QD * S::area(2) * 4 <= 152 * 1024 ? 2 : 1), "slot rule");
  constexpr int QUAD_DW = S::area(NSLOT);
  constexpr int MAIN_DW = QD * QUAD_DW;
  constexpr int Z_DW = BM * Z_ROW;
  constexpr int LDS_DW = MAIN_DW > Z_DW ? MAIN_DW : Z_DW;
  static_assert(!MULTI || QD == 1, "a quad computes one part when the workgroup has several");
  static_assert(LDS_DW * 4 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint32_t lds[LDS_DW];

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qd = wave_all / QW;
  const int wave = wave_all % QW;
  uint32_t *const qlds = lds + qd * QUAD_DW;
  uint32_t *const junk = qlds + NSLOT * SLOT_DW;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nb = QW == 4 ? (int)blockIdx.x : (int)blockIdx.x >> 1;  // 128-column block
  const int c0 = QW == 4 ? 0 : 64 * ((int)blockIdx.x & 1);         // first column of the slice in it
  const int m0 = p.row_base + blockIdx.z * BM;
  const int rend = p.row_end;
  const int M = p.M, K = p.K, N = p.N;
  const int NT = N >> 4;
  const int KB = K >> 7;

  // Grouped (MoE) calls: the row block's expert selects its trellis, svh
  // and bias (experts stacked at fixed strides); a block of no expert (-1)
  // has nothing to compute, for every workgroup of its tiles alike.
  const uint16_t *trellis = p.trellis, *svh = p.svh, *bias = p.bias;
  if constexpr (MOE) {
    const int e = __builtin_amdgcn_readfirstlane(p.block_expert[m0 / BM]);
    if (e < 0 || e >= p.n_experts) return;
    trellis += (int64_t)e * p.expert_trellis;
    svh += (int64_t)e * N;
    if (bias != nullptr) bias += (int64_t)e * N;
  }

  const int u0 = blockIdx.y * p.unit;  // first part of the workgroup's unit
  const int p_begin = QD > 1 ? u0 + qd : u0;
  const int p_end = QD > 1 ? p_begin + 1 : u0 + p.unit;
  const int kb_begin = (int)((int64_t)p_begin * KB / p.parts);
  const int kb_end = (int)((int64_t)p_end * KB / p.parts);
  const int nst = kb_end - kb_begin;

  int shard = 0;
  while (shard + 1 < p.n_shards && nb >= p.shard_end_blk[shard]) ++shard;
  const uint16_t *__restrict__ xs = p.x_rot + (int64_t)shard * M * K;

  // load sources: 16-bit word offsets from the stage bases
  const uint16_t *const t_base = trellis + ((int64_t)kb_begin * 8 * NT + nb * 8 + c0 / 16) * (16 * BITS);
  const int64_t t_stage = (int64_t)8 * NT * (16 * BITS);
  uint32_t t_src[T_OPS];
#pragma unroll
  for (int r = 0; r < T_OPS; ++r) t_src[r] = raw_chunk_src<BITS, NTS>(r * QT + wave * 64 + lane, NT);
  const uint16_t *const a_base = xs + (int64_t)kb_begin * 4 * M * 32;
  const int64_t a_stage = (int64_t)4 * M * 32;
  uint32_t a_src[A_OPS];
#pragma unroll
  for (int r = 0; r < A_OPS; ++r) {
    const int c = r * QT + wave * 64 + lane;  // chunk: k-step c/(4BM), row (c/4)%BM, 16 B piece c%4
    int row = m0 + (c >> 2) % BM;
    row = row < rend ? row : rend - 1;
    a_src[r] = (uint32_t)(((c / (4 * BM)) * M + row) * 32 + (c & 3) * 8);
  }
  // the rotated activations come from x_rot, or are rotated here (rot_in)
  const bool rot_in = !MOE && p.x_in != nullptr;
  auto issue_stage = [&](int stage, int slot) __attribute__((always_inline)) {
    uint32_t *const ts = qlds + slot * SLOT_DW;
#pragma unroll
    for (int r = 0; r < T_OPS; ++r) {
      const int q0 = r * QT + wave * 64;
      uint32_t *dst = q0 < S::T_CHUNKS ? ts + q0 * 4 : junk + (q0 - S::T_CHUNKS) * 4;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(t_base + stage * t_stage + t_src[r]),
                                       (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
    if (rot_in) return;
#pragma unroll
    for (int r = 0; r < A_OPS; ++r)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(a_base + stage * a_stage + a_src[r]),
                                       (__attribute__((address_space(3))) void *)(ts + S::TSLOT_DW + (r * QT + wave * 64) * 4),
                                       16, 0, 0);
  };

  int doff0, sh0, doff1, sh1;
  uint32_t sel0, sel1;
  raw_lane_window<BITS>(j, g, 0, doff0, sel0, sh0);
  raw_lane_window<BITS>(j, g, 1, doff1, sel1, sh1);
  const int tile_lane = ((g >> 1) * NTS + 2 * wave + (j >> 3)) * TSTRIDE;

  float4_t acc[MT][2];
  float4_t tot[MULTI ? MT : 1][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Every quad has the same number of stages (the host gives a several-quad
  // unit equal parts), so all waves meet the same barriers.
  issue_stage(0, 0);
  if (!rot_in) {
    if (NSLOT == 2 && nst > 1) {
      issue_stage(1, 1);
      wait_vmcnt<OPS>();  // stage 0 landed (stage 1's loads were issued after it)
    } else {
      wait_vmcnt<0>();
    }
  } else {
    // Rotation in the GEMM: every stage of the quad's K range has a slot
    // (the host's condition), so the loop below issues no further stage.
    // Each 16-lane group rotates one (stage, row) 128-block per pass, the
    // lane's piece straight into the slot's x~ area in the k-step tile
    // layout.  Only the tile's rows below the launch's last row are
    // rotated: a matrix-core product row depends on its own A row alone, so
    // whatever the other rows' x~ holds reaches only output rows that are
    // never stored.  The x loads of up to 8 passes are all issued before
    // the first rotation, so the passes share one load latency.
    if (NSLOT == 2 && nst > 1) issue_stage(1, 1);
    if constexpr (!MOE) {
      constexpr int RG = QW * 4;  // 16-lane groups in a quad
      constexpr int RB = (BM * NSLOT + RG - 1) / RG < 8 ? (BM * NSLOT + RG - 1) / RG : 8;
      const int L = lane & 15;
      const int kin = rotate_piece_k0(L);
      const int g0 = wave * 4 + (lane >> 4);
      const uint16_t *const suh_s = p.suh_in + (int64_t)shard * K + kb_begin * 128 + kin;
      uint32_t sw[NSLOT][4];  // the lane's suh words of each stage
#pragma unroll
      for (int st = 0; st < NSLOT; ++st) {
        if (st < nst) {
          const u32x2_t lo = *(const u32x2_t *)(suh_s + st * 128);
          const u32x2_t hi = *(const u32x2_t *)(suh_s + st * 128 + 8);
          sw[st][0] = lo.x, sw[st][1] = lo.y, sw[st][2] = hi.x, sw[st][3] = hi.y;
        } else {
          sw[st][0] = sw[st][1] = sw[st][2] = sw[st][3] = 0u;
        }
      }
      const int rows = rend - m0 < BM ? rend - m0 : BM;  // >= 1
      const int work = rows * nst;
      for (int b0 = 0; b0 < work; b0 += RB * RG) {
        u32x2_t xlo[RB], xhi[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int it = b0 + g0 + i * RG;
          if (it < work) {
            const int st = it / rows;
            const int r = it - st * rows;
            const uint16_t *const src = p.x_in + (int64_t)(m0 + r) * K + (kb_begin + st) * 128 + kin;
            xlo[i] = *(const u32x2_t *)src;
            xhi[i] = *(const u32x2_t *)(src + 8);
          }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int it = b0 + g0 + i * RG;
          if (it < work) {
            const int st = it / rows;
            const int r = it - st * rows;
            const uint32_t xw[4] = {xlo[i].x, xlo[i].y, xhi[i].x, xhi[i].y};
            float xv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              xv[2 * j] = p.x_in_bf16 ? bf16_bits_to_f32(xw[j] & 0xFFFFu) : f16_bits_to_f32(xw[j] & 0xFFFFu);
              xv[2 * j + 1] = p.x_in_bf16 ? bf16_bits_to_f32(xw[j] >> 16) : f16_bits_to_f32(xw[j] >> 16);
            }
            uint32_t sws[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sws[j] = NSLOT == 2 && st != 0 ? sw[NSLOT - 1][j] : sw[0][j];
            *(u32x4_t *)(qlds + st * SLOT_DW + S::TSLOT_DW + ((L >> 2) * BM + r) * 16 + 4 * (L & 3)) =
                rotate_piece(xv, sws, L);
          }
        }
      }
    }
    wait_vmcnt<0>();
  }
  barrier_lds();

  int s = 0;
  auto run_stages = [&](int s_end) __attribute__((always_inline)) {
    for (; s < s_end; ++s) {
      const uint32_t *const tb = qlds + (NSLOT == 2 ? (s & 1) : 0) * SLOT_DW;
      const uint32_t *const ab = tb + S::TSLOT_DW + 16 * j + 4 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half8_t a[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) a[mt] = *(const half8_t *)(ab + (ks * BM + mt * 16) * 16);
        const uint32_t *tp = tb + tile_lane + 2 * NTS * ks * TSTRIDE;
        const half8_t b0 = __builtin_bit_cast(half8_t, raw_decode_frag<BITS, CB>(tp + doff0, sel0, sh0));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], b0, acc[mt][0], 0, 0, 0);
        const half8_t b1 = __builtin_bit_cast(half8_t, raw_decode_frag<BITS, CB>(tp + doff1, sel1, sh1));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt], b1, acc[mt][1], 0, 0, 0);
      }
      barrier_lds();  // every wave is done with this slot
      if constexpr (NSLOT == 2) {
        if (s + 2 < nst) {
          issue_stage(s + 2, s & 1);
          wait_vmcnt<OPS>();  // stage s+1 landed
        } else {
          wait_vmcnt<0>();
        }
      } else if (s + 1 < nst) {
        issue_stage(s + 1, 0);
        wait_vmcnt<0>();
      }
      barrier_lds();
    }
  };

  if constexpr (MULTI) {
    // first part copied, later parts added in part order
    run_stages((int)((int64_t)(p_begin + 1) * KB / p.parts) - kb_begin);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        tot[mt][h] = acc[mt][h];
        acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
    for (int part = p_begin + 1; part < p_end; ++part) {
      run_stages((int)((int64_t)(part + 1) * KB / p.parts) - kb_begin);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          tot[mt][h] = tot[mt][h] + acc[mt][h];
          acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[mt][h] = tot[mt][h];
  } else {
    run_stages(nst);
  }
  wait_vmcnt<0>();

  // The quads' parts in part order through LDS (the stage slots are free:
  // the last stage ended with a barrier): z = part 0, z = z + part 1, ...;
  // the last quad adds its part in registers and holds the unit's sum.
  float *z = reinterpret_cast<float *>(lds);
  if constexpr (QD > 1) {
    for (int q = 0; q < QD - 1; ++q) {
      if (qd == q) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int col = lane_col(wave, j, h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float *zi = z + (mt * 16 + 4 * g + i) * Z_ROW + col;
              *zi = q == 0 ? acc[mt][h][i] : *zi + acc[mt][h][i];
            }
          }
      }
      barrier_lds();
    }
    if (qd == QD - 1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = lane_col(wave, j, h);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][h][i] = z[(mt * 16 + 4 * g + i) * Z_ROW + col] + acc[mt][h][i];
        }
    }
  }
  const bool writer = qd == QD - 1;

  if (p.slab_mode) {
    const int rows = rend - p.row_base;
    if (p.counters == nullptr) {
      if (writer) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            store_partial(p.slabs, blockIdx.y, rows, N, m0 - p.row_base + mt * 16 + 4 * g,
                          nb * 128 + c0 + lane_col(wave, j, h), acc[mt][h]);
      }
      return;
    }
    if (writer) {
      const __amdgpu_buffer_rsrc_t rs = slab_rsrc(p);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          store_partial_coherent(rs, blockIdx.y, rows, N, m0 - p.row_base + mt * 16 + 4 * g,
                                 nb * 128 + c0 + lane_col(wave, j, h), acc[mt][h]);
    }
    // The output stage's svh and bias words of the block, loaded now: the
    // arrival waits for them together with the slab stores, so the last
    // workgroup does not wait a round trip for them afterwards.
    const OutWords ow = out_words(svh, bias, nb * 128, lane);
    // the tile is the 128-column block: both halves' workgroups arrive
    const uint32_t tile = blockIdx.z * (gridDim.x * QW / 4) + nb;
    if (!arrive_last(p, tile, gridDim.y * (4 / QW))) return;
    finish_tile(p, ow, bias != nullptr, tile, nb, m0, BM, wave_all, QW * QD, lane, z, LDS_DW * 4);
    return;
  }

  // fused: the output stage needs the whole 128-column block (QW == 4)
  if constexpr (QW == 4) {
  if constexpr (QD == 1) barrier_lds();  // every wave is done with the stage slots
  if (writer) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = lane_col(wave, j, h);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[(mt * 16 + 4 * g + i) * Z_ROW + col] = acc[mt][h][i];
      }
  }
  const OutWords16 ow = out_words16(svh, bias, nb * 128, lane);
  barrier_lds();
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
  for (int r0 = 8 * wave_all; r0 < BM && m0 + r0 < rend; r0 += 8 * QW * QD) {
    if (p.out_bf16) output_rows8<true>(z, Z_ROW, r0, ow, bias != nullptr, y, m0 + r0, rend, N, nb * 128, lane);
    else output_rows8<false>(z, Z_ROW, r0, ow, bias != nullptr, y, m0 + r0, rend, N, nb * 128, lane);
  }
  }
}

// -------------------------------------------------------------- big GEMM
//
// For M around 128 with a unit of several K parts per workgroup (their sums
// folded in registers; one part per workgroup takes the 8-wave 128-row tile
// of gemm_wide_kernel): a BM = 16*MT row x 128 column tile (MT = 8) on 4 waves.
// As in gemm_kernel, wave w decodes the B operands of n-tiles 2w and 2w+1 and
// keeps them in registers, now against all BM rows, so each trellis value is
// decoded once per BM rows and feeds 2*MT MFMAs per lane-set.  The rotated
// activations go HBM/L2 -> LDS by direct loads (global_load_lds_dwordx4, no
// registers involved) into a ring of k-step slots, PF k-steps ahead; each
// 16-row fragment occupies 1 KB in exactly the lane order of the MFMA A
// operand (x~ is in fragment order), so reading it is one conflict-free
// ds_read_b128 per lane.  The decode of k-step i+1 is interleaved with the
// MFMAs of k-step i.  Rows past M load row M-1 (finite, discarded).  Same
// k slots, k-step order, parts and part fold as gemm_kernel: same bits.

template <int MT>
__device__ __forceinline__ void issue_a_dma(uint32_t *__restrict__ slot, const uint16_t *__restrict__ xs, int m0,
                                            int M, int rend, int k, int wave, int lane) {
  // wave w loads fragments w, w+4, ... of this k-step; lane L of a fragment
  // holds row (L & 15) and k-chunk (L >> 4)
#pragma unroll
  for (int t = 0; t < MT / 4; ++t) {
    const int mf = wave + 4 * t;
    int row = m0 + 16 * mf + (lane & 15);
    row = row < rend ? row : rend - 1;
    const uint16_t *src = xs + ((int64_t)(k >> 5) * M + row) * 32 + 8 * (lane >> 4);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)(slot + mf * 256), 16, 0, 0);
  }
}

template <int BITS, uint32_t CB, int MT, bool MULTI>
__global__ __launch_bounds__(WG_THREADS, 1) void gemm_big_kernel(const GemmParams p) {
  using G = Geom<BITS>;
  constexpr int BM = 16 * MT;
  constexpr int PF = 2;                 // A prefetch distance (k-steps)
  constexpr int NSLOT = 4;              // ring slots; a slot is rewritten 2 steps after its last read
  constexpr int ASLOT_DW = MT * 256;    // MT fragments x 64 lanes x 16 bytes
  constexpr int A_DW = NSLOT * ASLOT_DW;
  constexpr int MAIN_DW = A_DW + 2 * G::STAGE_T_DW;
  constexpr int ZROWS = 64;             // output stage: 64 rows per pass
  constexpr int Z_DW = ZROWS * Z_ROW;
  constexpr int LDS_DW = MAIN_DW > Z_DW ? MAIN_DW : Z_DW;
  constexpr int DMA_PER_STEP = MT / 4;  // direct loads per wave per k-step
  __shared__ __attribute__((aligned(16))) uint32_t lds[LDS_DW];
  uint32_t *const abuf = lds;
  uint32_t *const tbuf = lds + A_DW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nb = blockIdx.x;
  const int m0 = p.row_base + blockIdx.z * BM;
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

  int xoff0, sh0, xoff1, sh1;
  lane_window<BITS>(j, g, 0, xoff0, sh0);
  lane_window<BITS>(j, g, 1, xoff1, sh1);
  const int tile_lane = (g >> 1) * WG_NT + 2 * wave + (j >> 3);

  u32x4_t treg[G::T_ITERS];
  float4_t acc[MT][2];
  float4_t tot[MULTI ? MT : 1][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
  // prologue: A for the first PF k-steps, trellis stage 0 in LDS, stage 1 in
  // registers.  Prefetch indices past the end are clamped to the last stage or
  // k-step, so the loop below has no branches (the extra loads are in bounds
  // and their results unused).
#pragma unroll
  for (int i = 0; i < PF; ++i)
    issue_a_dma<MT>(abuf + i * ASLOT_DW, xs, m0, M, rend, k_begin + 32 * min(i, nks - 1), wave, lane);
  load_trellis_stage<BITS>(treg, p.trellis, kb_begin, nb, NT, tid);
  store_trellis_stage<BITS>(treg, tbuf, tid);
  load_trellis_stage<BITS>(treg, p.trellis, kb_begin + min(1, nst - 1), nb, NT, tid);
  __syncthreads();
  half8_t b0 = decode_frag<BITS, CB>(tbuf + tile_lane * G::STRIDE, xoff0, sh0);
  half8_t b1 = decode_frag<BITS, CB>(tbuf + tile_lane * G::STRIDE, xoff1, sh1);

  int st = 0;
  auto run_stages = [&](int st_end) {
    for (; st < st_end; ++st) {
      // stage st is in tbuf[st & 1]; store stage st+1 and start loading st+2
      uint32_t *const tcur = tbuf + (st & 1) * G::STAGE_T_DW;
      uint32_t *const tnxt = tbuf + ((st + 1) & 1) * G::STAGE_T_DW;
      store_trellis_stage<BITS>(treg, tnxt, tid);
      auto kstep = [&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        const int i = 4 * st + ks;
        issue_a_dma<MT>(abuf + ((i + PF) % NSLOT) * ASLOT_DW, xs, m0, M, rend, k_begin + 32 * min(i + PF, nks - 1),
                        wave, lane);
        asm volatile("" ::: "memory");  // keep the issue order the counts below assume
        // Vector-memory ops complete in issue order.  This wave's direct loads
        // for k-step i are done once no more than the ops issued after them
        // are outstanding: the PF later groups, plus the trellis loads issued
        // after k-step 0 of this stage while they are younger than group i.
        if constexpr (ks == 1 || ks == 2) wait_vmcnt<PF * DMA_PER_STEP + G::T_MIN>();
        else wait_vmcnt<PF * DMA_PER_STEP>();
        barrier_lds();  // the other waves' loads for k-step i, and the stores above
        if constexpr (ks == 0) {
          load_trellis_stage<BITS>(treg, p.trellis, kb_begin + min(st + 2, nst - 1), nb, NT, tid);
          asm volatile("" ::: "memory");
        }
        // The next k-step's B operands are decoded in 10 pieces (2 normalize,
        // 8 pairs) spread between this step's MFMA pairs; sched_barrier keeps
        // the interleaving, so the VALU work issues while the matrix core is
        // busy instead of before it.
        const uint32_t *tp = ks < 3 ? tcur + (tile_lane + 2 * WG_NT * (ks + 1)) * G::STRIDE
                                    : tnxt + tile_lane * G::STRIDE;
        uint32_t X0[G::NX], X1[G::NX], Y0[G::NY], Y1[G::NY];
        u32x4_t nb0, nb1;
        frag_load<BITS>(tp, xoff0, X0);
        frag_load<BITS>(tp, xoff1, X1);
        const uint32_t *as = abuf + (i % NSLOT) * ASLOT_DW + 4 * lane;
        half8_t a[3];
        a[0] = *(const half8_t *)(as);
        a[1] = *(const half8_t *)(as + 256);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, MT>([&](auto mt_c) {
          constexpr int mt = decltype(mt_c)::value;
          acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt % 3], b0, acc[mt][0], 0, 0, 0);
          acc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt % 3], b1, acc[mt][1], 0, 0, 0);
          if constexpr (mt + 2 < MT) a[(mt + 2) % 3] = *(const half8_t *)(as + (mt + 2) * 256);
          static_for<mt * 10 / MT, (mt + 1) * 10 / MT>([&](auto pc) {
            constexpr int piece = decltype(pc)::value;
            if constexpr (piece == 0) frag_normalize<BITS>(X0, sh0, Y0);
            else if constexpr (piece < 5) nb0[piece - 1] = frag_pair<BITS, CB, piece - 1>(Y0);
            else if constexpr (piece == 5) frag_normalize<BITS>(X1, sh1, Y1);
            else nb1[piece - 6] = frag_pair<BITS, CB, piece - 6>(Y1);
          });
          __builtin_amdgcn_sched_barrier(0);
        });
        const half8_t n0 = __builtin_bit_cast(half8_t, nb0);
        const half8_t n1 = __builtin_bit_cast(half8_t, nb1);
        b0 = n0;
        b1 = n1;
      };
      kstep(std::integral_constant<int, 0>{});
      kstep(std::integral_constant<int, 1>{});
      kstep(std::integral_constant<int, 2>{});
      kstep(std::integral_constant<int, 3>{});
    }
  };

  if constexpr (MULTI) {
    // first part copied, later parts added in part order
    run_stages((int)((int64_t)(p_begin + 1) * KB / p.parts) - kb_begin);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        tot[mt][h] = acc[mt][h];
        acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
      }
    for (int part = p_begin + 1; part < p_end; ++part) {
      run_stages((int)((int64_t)(part + 1) * KB / p.parts) - kb_begin);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          tot[mt][h] = tot[mt][h] + acc[mt][h];
          acc[mt][h] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[mt][h] = tot[mt][h];
  } else {
    run_stages(nst);
  }
  wait_vmcnt<0>();  // the clamped tail loads land before LDS is reused

  if (p.slab_mode) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        store_partial(p.slabs, blockIdx.y, rend - p.row_base, N, m0 - p.row_base + mt * 16 + 4 * g,
                      nb * 128 + lane_col(wave, j, h), acc[mt][h]);
    return;
  }

  // output transform, 64 rows at a time through LDS
  float *z = reinterpret_cast<float *>(lds);
  uint16_t *__restrict__ y = reinterpret_cast<uint16_t *>(p.y);
  const OutWords16 ow = out_words16(p.svh, p.bias, nb * 128, lane);
#pragma unroll
  for (int pass = 0; pass < MT / 4; ++pass) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mt = 4 * pass + q;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = lane_col(wave, j, h);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[(q * 16 + 4 * g + i) * Z_ROW + col] = acc[mt][h][i];
      }
    }
    __syncthreads();
    for (int r0 = 8 * wave; r0 < ZROWS && m0 + pass * ZROWS + r0 < rend; r0 += 32) {
      if (p.out_bf16)
        output_rows8<true>(z, Z_ROW, r0, ow, p.bias != nullptr, y, m0 + pass * ZROWS + r0, rend, N, nb * 128, lane);
      else
        output_rows8<false>(z, Z_ROW, r0, ow, p.bias != nullptr, y, m0 + pass * ZROWS + r0, rend, N, nb * 128, lane);
    }
  }
}

// Decode-only kernel for tests: the same staging and decode_frag as the GEMM,
// storing each lane's 8 values at their (k, n) instead of multiplying.
template <int BITS, uint32_t CB>
__global__ __launch_bounds__(WG_THREADS) void debug_decode_kernel(const DecodeParams p) {
  using G = Geom<BITS>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[G::STAGE_T_DW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x, kb = blockIdx.y;
  u32x4_t treg[G::T_ITERS];
  load_trellis_stage<BITS>(treg, p.trellis, kb, nb, p.N >> 4, tid);
  store_trellis_stage<BITS>(treg, lds, tid);
  __syncthreads();
  const int tile_lane = (g >> 1) * WG_NT + 2 * wave + (j >> 3);
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t *tp = lds + (tile_lane + 2 * WG_NT * ks) * G::STRIDE;
    for (int h = 0; h < 2; ++h) {
      int xoff, sh;
      lane_window<BITS>(j, g, h, xoff, sh);
      // Read the halves through a u32x4: extracting _Float16 elements of the
      // half8 vector and bit-casting them one by one miscompiles (every
      // element came out equal to element 0).
      const u32x4_t b = __builtin_bit_cast(u32x4_t, decode_frag<BITS, CB>(tp, xoff, sh));
      const int n = nb * 128 + lane_col(wave, j, h);
      const int k0 = kb * 128 + 32 * ks + 16 * (g >> 1) + 4 * (g & 1);
      const int koff[8] = {0, 1, 2, 3, 8, 9, 10, 11};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p.wq[(int64_t)(k0 + koff[e]) * p.N + n] = (uint16_t)(b[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Dequantize to B fragments: the whole W_q once, in the order the matrix
// core reads it, for the dense GEMM of large batches.  Fragment f = 2w + h
// of 32-k step ks and 128-column block nb is the B operand wave w of a tile
// kernel decodes for column half h (n-tiles 2w, 2w+1): lane L holds its 8
// fp16 values as 16 contiguous bytes, so
//   wf[((ks * nblk + nb) * 8 + f) * 64 + L]  (16 bytes each)
// and one k-step of a block is 8 KB.  The same staging and decode_frag as
// the tile kernels, so the same fp16 values.  One workgroup per 128 k x 128
// columns.
template <int BITS, uint32_t CB>
__global__ __launch_bounds__(WG_THREADS) void dequant_kernel(const DecodeParams p) {
  using G = Geom<BITS>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[G::STAGE_T_DW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x, kb = blockIdx.y;
  const int nblk = p.N >> 7;
  u32x4_t treg[G::T_ITERS];
  load_trellis_stage<BITS>(treg, p.trellis, kb, nb, p.N >> 4, tid);
  store_trellis_stage<BITS>(treg, lds, tid);
  __syncthreads();
  const int tile_lane = (g >> 1) * WG_NT + 2 * wave + (j >> 3);
  u32x4_t *const wf = reinterpret_cast<u32x4_t *>(p.wq);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t *tp = lds + (tile_lane + 2 * WG_NT * ks) * G::STRIDE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int xoff, sh;
      lane_window<BITS>(j, g, h, xoff, sh);
      const u32x4_t b = __builtin_bit_cast(u32x4_t, decode_frag<BITS, CB>(tp, xoff, sh));
      wf[(((int64_t)(4 * kb + ks) * nblk + nb) * 8 + 2 * wave + h) * 64 + lane] = b;
    }
  }
}

// Decode-rate ruler: the same trellis staging and decode as the tile kernels
// for one 128 x 128 block per workgroup, with no matrix-core work and no
// weight stores: the 4-byte words of every decoded fragment are XOR-reduced
// into one word per block, out[kb * nblk + nb].  The low half of that word
// is the XOR of the block's fp16 values at even k, the high half at odd k
// (a fragment's words pair k offsets 0-1, 2-3, 8-9, 10-11).  Its time is the
// fastest any decoding kernel can stream the trellis (decode-VALU roof).
template <int BITS, uint32_t CB>
__global__ __launch_bounds__(WG_THREADS) void decode_rate_kernel(const DecodeParams p) {
  using G = Geom<BITS>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[G::STAGE_T_DW];
  __shared__ uint32_t red[WG_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x, kb = blockIdx.y;
  const int nblk = p.N >> 7;
  u32x4_t treg[G::T_ITERS];
  load_trellis_stage<BITS>(treg, p.trellis, kb, nb, p.N >> 4, tid);
  store_trellis_stage<BITS>(treg, lds, tid);
  __syncthreads();
  const int tile_lane = (g >> 1) * WG_NT + 2 * wave + (j >> 3);
  uint32_t x = 0;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t *tp = lds + (tile_lane + 2 * WG_NT * ks) * G::STRIDE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int xoff, sh;
      lane_window<BITS>(j, g, h, xoff, sh);
      const u32x4_t b = __builtin_bit_cast(u32x4_t, decode_frag<BITS, CB>(tp, xoff, sh));
      x ^= b[0] ^ b[1] ^ b[2] ^ b[3];
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d, 64);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < WG_THREADS / 64; ++w) t ^= red[w];
    reinterpret_cast<uint32_t *>(p.wq)[kb * nblk + nb] = t;
  }
}

// ---------------------------------------------------------------- launchers

// One small-tile instance; the grouped (MoE) variant when the call routes
// row blocks to experts.
template <int BITS, uint32_t CB, int MT, bool MULTI, int QD, int QW>
void launch_small(const GemmParams &p, dim3 grid, hipStream_t s) {
  if (p.block_expert != nullptr)
    hipLaunchKernelGGL((gemm_kernel<BITS, CB, MT, MULTI, QD, QW, true>), grid, dim3(64 * QW * QD), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_kernel<BITS, CB, MT, MULTI, QD, QW, false>), grid, dim3(64 * QW * QD), 0, s, p);
}

// quads > 1: one part per quad (no register fold); otherwise `multi` folds
// the workgroup's parts in registers.  half: 64-column workgroups (quads of
// two waves; slab mode only, no register fold).
template <int BITS, uint32_t CB, int MT>
hipError_t launch_gemm_t(int quads, bool half, bool multi, const GemmParams &p, dim3 grid, hipStream_t s) {
  if (half) {
    if (multi || !p.slab_mode) return hipErrorInvalidValue;
    switch (quads) {
      case 1: launch_small<BITS, CB, MT, false, 1, 2>(p, grid, s); break;
      case 2: launch_small<BITS, CB, MT, false, 2, 2>(p, grid, s); break;
      case 4: launch_small<BITS, CB, MT, false, 4, 2>(p, grid, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (quads) {
    case 1:
      if (multi) launch_small<BITS, CB, MT, true, 1, 4>(p, grid, s);
      else launch_small<BITS, CB, MT, false, 1, 4>(p, grid, s);
      break;
    case 2: launch_small<BITS, CB, MT, false, 2, 4>(p, grid, s); break;
    case 4: launch_small<BITS, CB, MT, false, 4, 4>(p, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 128-row tiles of a unit of several parts (folded in registers)
template <int BITS, uint32_t CB, int MT>
hipError_t launch_big_t(const GemmParams &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((gemm_big_kernel<BITS, CB, MT, true>), grid, dim3(WG_THREADS), 0, s, p);
  return hipGetLastError();
}

template <int BITS, uint32_t CB>
hipError_t launch_wide_t(int bm, bool multi, const GemmParams &p, dim3 grid, hipStream_t s);

// bm = rows per M-tile: 16/32/64 -> gemm_kernel, 128 -> gemm_wide_kernel
// with 64-row waves (one part per workgroup) or gemm_big_kernel (a unit of
// several parts), 256/512 -> gemm_wide_kernel (512 threads; 512 for a single
// part per workgroup only).
template <int BITS, uint32_t CB>
hipError_t launch_gemm_cb(int bm, int quads, bool half, bool multi, const GemmParams &p, dim3 grid, hipStream_t s) {
  if (bm > 64 && (quads != 1 || half)) return hipErrorInvalidValue;
  switch (bm) {
    case 16: return launch_gemm_t<BITS, CB, 1>(quads, half, multi, p, grid, s);
    case 32: return launch_gemm_t<BITS, CB, 2>(quads, half, multi, p, grid, s);
    case 64: return launch_gemm_t<BITS, CB, 4>(quads, half, multi, p, grid, s);
    case 128:
      // one part per workgroup: the 8-wave tile with 64-row waves, two
      // workgroups per CU; a unit of several parts folded in registers: the
      // 4-wave tile
      if (!multi) return launch_wide_t<BITS, CB>(128, false, p, grid, s);
      return launch_big_t<BITS, CB, 8>(p, grid, s);
    case 256:
    case 512: return launch_wide_t<BITS, CB>(bm, multi, p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t launch_gemm_bits(int cb, int bm, int quads, bool half, bool multi, const GemmParams &p, dim3 grid,
                            hipStream_t s) {
  switch (cb) {
    case 0: return launch_gemm_cb<BITS, CB_3INST>(bm, quads, half, multi, p, grid, s);
    case 1: return launch_gemm_cb<BITS, CB_MCG>(bm, quads, half, multi, p, grid, s);
    case 2: return launch_gemm_cb<BITS, CB_MUL1>(bm, quads, half, multi, p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t launch_dequant_bits(int cb, const DecodeParams &p, hipStream_t s) {
  const dim3 grid(p.N / 128, p.K / 128);
  switch (cb) {
    case 0: hipLaunchKernelGGL((dequant_kernel<BITS, CB_3INST>), grid, dim3(WG_THREADS), 0, s, p); break;
    case 1: hipLaunchKernelGGL((dequant_kernel<BITS, CB_MCG>), grid, dim3(WG_THREADS), 0, s, p); break;
    case 2: hipLaunchKernelGGL((dequant_kernel<BITS, CB_MUL1>), grid, dim3(WG_THREADS), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_decode_rate_bits(int cb, const DecodeParams &p, hipStream_t s) {
  const dim3 grid(p.N / 128, p.K / 128);
  switch (cb) {
    case 0: hipLaunchKernelGGL((decode_rate_kernel<BITS, CB_3INST>), grid, dim3(WG_THREADS), 0, s, p); break;
    case 1: hipLaunchKernelGGL((decode_rate_kernel<BITS, CB_MCG>), grid, dim3(WG_THREADS), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_rate_kernel<BITS, CB_MUL1>), grid, dim3(WG_THREADS), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_decode_bits(int cb, const DecodeParams &p, hipStream_t s) {
  const dim3 grid(p.N / 128, p.K / 128);
  switch (cb) {
    case 0: hipLaunchKernelGGL((debug_decode_kernel<BITS, CB_3INST>), grid, dim3(WG_THREADS), 0, s, p); break;
    case 1: hipLaunchKernelGGL((debug_decode_kernel<BITS, CB_MCG>), grid, dim3(WG_THREADS), 0, s, p); break;
    case 2: hipLaunchKernelGGL((debug_decode_kernel<BITS, CB_MUL1>), grid, dim3(WG_THREADS), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace exl3

#define EXL3_DEFINE_BITS(B)                                                                        \
  namespace exl3 {                                                                                 \
  hipError_t launch_gemm_b##B(int cb, int bm, int quads, bool half, bool multi, const GemmParams &p, \
                              dim3 grid, hipStream_t s) {                                          \
    return launch_gemm_bits<B>(cb, bm, quads, half, multi, p, grid, s);                            \
  }                                                                                                \
  hipError_t launch_table_b##B(int cb, const GemmParams &p, int grid, hipStream_t s) {             \
    return launch_table_bits<B>(cb, p, grid, s);                                                   \
  }                                                                                                \
  hipError_t launch_debug_decode_b##B(int cb, const DecodeParams &p, hipStream_t s) {              \
    return launch_decode_bits<B>(cb, p, s);                                                        \
  }                                                                                                \
  hipError_t launch_dequant_b##B(int cb, const DecodeParams &p, hipStream_t s) {                   \
    return launch_dequant_bits<B>(cb, p, s);                                                       \
  }                                                                                                \
  hipError_t launch_decode_rate_b##B(int cb, const DecodeParams &p, hipStream_t s) {               \
    return launch_decode_rate_bits<B>(cb, p, s);                                                   \
  }                                                                                                \
  }
