// Device-side building blocks of the EXL3 linear for gfx950 (CDNA4).
//
// Everything here runs on a 64-wide wavefront.  The arithmetic follows the
// TensorFold PR "cuda: EXL3 projections behind qlinear", section
// "Arithmetic": fp32 Hadamard butterflies with a fixed add order, one fp16
// rounding of the rotated activations, fp16 products with fp32 sums, and one
// rounding of the output.  The codebooks follow the cuda-exl3 README, "What
// is supported" (3inst, mcg, mul1; mcg multiplier 0xCBAC1FED from its
// "GLM-5.3-Flash" section); the pages print no other constants, so 3inst and
// mul1 use the constants below, and both rotations use butterfly strides
// 1, 2, ..., 64 in ascending order.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace exl3 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int HBLOCK = 128;  // Hadamard block

// ------------------------------------------------------------ conversions

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
// Round to nearest even (the default rounding mode of v_cvt_f16_f32).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __hip_bfloat16 h = __float2bfloat16(f);
  return __builtin_bit_cast(uint16_t, h);
}

// ------------------------------------------------------------- codebooks
//
// A state is the low 16 bits of a 32-bit register (higher bits are ignored).
// mcg:   u = s * 0xCBAC1FED (mod 2^32), then the pair sum P(u)
// 3inst: u = s * 0x2C9277B5 + 0x3C6EF372, then P(u)
// P(u):  u' = (u & 0x8FFF8FFF) | 0x30003000 -> two fp16 halves in
//        +-[0.125, 2); value = lo + hi, one fp16 rounding
// mul1:  u = s * 0x9E3779B1, t = sum of u's bytes, value = t*alpha + beta in
//        one fp16 fused multiply-add (alpha = 0x1EEE, beta = 0xC2E8).  It is
//        evaluated as (1024 + t) * alpha + (beta - 1024 * alpha): the fp16
//        0x6400 | t is exactly 1024 + t, and beta - 1024 * alpha = -10.3828125
//        (0xC931) is an fp16, so the fused sum and its one rounding are the
//        same.

constexpr uint32_t CB_3INST = 0, CB_MCG = 1, CB_MUL1 = 2;

// 16-bit x 16-bit products in full-rate VALU ops.  v_mad_u32_u16 and the
// packed 16-bit ops read only the low halves they are told to, so a state may
// carry garbage above bit 15.  (Written as inline asm: the compiler otherwise
// masks the state and uses the quarter-rate v_mul_lo_u32.)
__device__ __forceinline__ uint32_t mad_u32_u16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
// {lo: 0, hi: (a[15:0] * kh) mod 2^16} for k = kh << 16.
__device__ __forceinline__ uint32_t pk_mul_lo_u16_dup(uint32_t a, uint32_t k) {
  uint32_t d;
  asm("v_pk_mul_lo_u16 %0, %1, %2 op_sel_hi:[0,1]" : "=v"(d) : "v"(a), "v"(k));
  return d;
}
// {lo: c[15:0], hi: (a[15:0] * kh + c[31:16]) mod 2^16} for k = kh << 16.
__device__ __forceinline__ uint32_t pk_mad_u16_dup(uint32_t a, uint32_t k, uint32_t c) {
  uint32_t d;
  asm("v_pk_mad_u16 %0, %1, %2, %3 op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(k), "v"(c));
  return d;
}

// (s mod 2^16) * C + B  (mod 2^32) in two full-rate ops:
//   t = {B_lo, (s * C_hi + B_hi) mod 2^16};  u = s * C_lo + t.
template <uint32_t C, uint32_t B>
__device__ __forceinline__ uint32_t mul16_const(uint32_t s) {
  const uint32_t kh = C & 0xFFFF0000u;
  uint32_t t;
  if constexpr (B == 0) t = pk_mul_lo_u16_dup(s, kh);
  else t = pk_mad_u16_dup(s, kh, B);
  return mad_u32_u16(s, C & 0xFFFFu, t);
}

template <uint32_t CB>
__device__ __forceinline__ uint32_t cb_hash(uint32_t s) {
  if constexpr (CB == CB_3INST) return mul16_const<0x2C9277B5u, 0x3C6EF372u>(s);
  else if constexpr (CB == CB_MCG) return mul16_const<0xCBAC1FEDu, 0u>(s);
  else return mul16_const<0x9E3779B1u, 0u>(s);
}

// P(u) for two words: lo half = P(u0), hi half = P(u1).  Each fp16 add reads
// the two halves of one masked word (SDWA selects) and writes one half of the
// result, the other half preserved.  The result usually feeds a matrix-core
// instruction, which must not read a VGPR sooner than two wait states after a
// VALU instruction wrote it; the compiler cannot see writes made inside asm
// and so does not count them, hence the s_nop 1 after the last add (without
// it an MFMA one instruction later read a stale operand).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(o));
  return d;
}

__device__ __forceinline__ uint32_t pair_sum2(uint32_t u0, uint32_t u1) {
  const uint32_t m0 = and_or(u0, 0x8FFF8FFFu, 0x30003000u);
  const uint32_t m1 = and_or(u1, 0x8FFF8FFFu, 0x30003000u);
  uint32_t r;
  asm("v_add_f16_sdwa %0, %1, %1 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:WORD_1"
      : "=v"(r) : "v"(m0));
  asm("v_add_f16_sdwa %0, %1, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_0 src1_sel:WORD_1\n\t"
      "s_nop 1"
      : "+v"(r) : "v"(m1));
  return r;
}

// Two states -> two fp16 values packed in one register (s0 low, s1 high).
template <uint32_t CB>
__device__ __forceinline__ uint32_t decode_pair(uint32_t s0, uint32_t s1) {
  if constexpr (CB == CB_MUL1) {
    // 0x6400 + the sum of the hash's four bytes, for both states, packed as
    // two fp16 bit patterns: v_sad_u8 adds the byte sum of state 0 (sum of
    // |byte - 0|, at most 1020, so no carry leaves the low half) and
    // v_sad_hi_u8 adds the byte sum of state 1 shifted into the high half.
    // (v_dot4_u32_u8 computes the same sums but runs ~2x slower while
    // another wave on the SIMD issues MFMAs.)
    const uint32_t d0 = __builtin_amdgcn_sad_u8(cb_hash<CB>(s0), 0u, 0x64006400u);
    const uint32_t d01 = __builtin_amdgcn_sad_hi_u8(cb_hash<CB>(s1), 0u, d0);
    const half2_t h = __builtin_bit_cast(half2_t, d01);
    const half2_t alpha = {__builtin_bit_cast(_Float16, (uint16_t)0x1EEE),
                           __builtin_bit_cast(_Float16, (uint16_t)0x1EEE)};
    const half2_t c = {__builtin_bit_cast(_Float16, (uint16_t)0xC931),
                       __builtin_bit_cast(_Float16, (uint16_t)0xC931)};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h, alpha, c));
  } else {
    return pair_sum2(cb_hash<CB>(s0), cb_hash<CB>(s1));
  }
}

// Keep an fp32 value as an fp32 register value: stops the compiler from
// fusing the product that produced it into a mixed-precision convert (which
// would round once instead of rounding to fp32 and then to the output type).
__device__ __forceinline__ float keep_f32(float v) {
  asm("" : "+v"(v));
  return v;
}

// ----------------------------------------------- rotated-activation layout
//
// x~ is stored in "fragment order": inside every aligned group of 32 k, the
// 4-element chunks are stored in the order 0, 2, 1, 3, 4, 6, 5, 7 (chunk
// index bits b2 b1 b0 stored at b2 b0 b1).  Lane group g of an MFMA operand
// holds k = 16(g>>1) + 4(g&1) + {0,1,2,3,8,9,10,11}, which is then the
// contiguous run 8g..8g+7.  The values are those of the natural order.
__device__ __forceinline__ int frag_order_k(int k) {
  const int c = (k >> 2) & 7;
  const int cs = (c & 4) | ((c & 1) << 1) | ((c >> 1) & 1);
  return (k & ~31) | (cs << 2) | (k & 3);
}

// ------------------------------------------- input rotation, one piece
//
// x~[m][:] = fp16_rne(2^-4 * H128(x[m][:] * suh[:])) per 128-block, on
// sixteen lanes per (row, block): lane L holds the 8 values that one 16-byte
// piece of the k-step tile layout stores, of 32-group j = L/4 and piece
// q = L%4, k = 32j + 16(q/2) + 4(q%2) + {0,1,2,3, 8,9,10,11} (the fragment
// order of frag_order_k).  The butterfly strides 1, 2 and 8 pair values
// inside the lane; strides 4, 16, 32 and 64 pair lane L with L^1, L^2, L^4
// and L^8 (within its 16-lane DPP row), whose values arrive by DPP lane
// moves.  The stages run in the fixed order 1, 2, 4, ..., 64, each pair
// (a, b) -> (a + b, a - b) one fp32 add each, so any caller gets the same
// bits; x * suh is exact in fp32.

// Lane value of lane^1, ^2, ^4, ^8 (within 16 lanes) by DPP: quad_perm
// [1,0,3,2]; quad_perm [2,3,0,1]; half-row mirror (i -> 7-i) then quad_perm
// [3,2,1,0] (7 - (i^3) = i^4 for i < 8); row rotate by 8.
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
  const int b = __builtin_bit_cast(int, v);
  int r;
  if constexpr (X == 1) r = __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false);
  else if constexpr (X == 2) r = __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, false);
  else if constexpr (X == 4)
    r = __builtin_amdgcn_update_dpp(0, __builtin_amdgcn_update_dpp(0, b, 0x141, 0xF, 0xF, false), 0x1B, 0xF, 0xF,
                                    false);
  else r = __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false);
  return __builtin_bit_cast(float, r);
}

// One cross-lane butterfly stage: the lane whose bit is clear keeps a + b
// (its value a, the partner's b), the other keeps b' - a' with its partner
// a' = the clear lane's value: the same two fp32 operations as in-lane.
template <int X>
__device__ __forceinline__ void xstage(float (&t)[8], bool upper) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = lane_xor<X>(t[e]);
    t[e] = upper ? p - t[e] : t[e] + p;
  }
}

// In-lane stage: pairs (e, e + d) for e with bit d clear.
template <int D>
__device__ __forceinline__ void lstage(float (&t)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if ((e & D) == 0) {
      const float a = t[e], b = t[e + D];
      t[e] = a + b;
      t[e + D] = a - b;
    }
}

// The lane's piece: xv its 8 x values (fp32; t[0..3] = k0 + 0..3, t[4..7] =
// k0 + 8..11), sw the suh words at the same k (two fp16 each), L the lane
// within its 16.  Returns the 8 rotated fp16 values as one 16-byte piece.
__device__ __forceinline__ u32x4_t rotate_piece(const float (&xv)[8], const uint32_t (&sw)[4], int L) {
  float t[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t[2 * i] = xv[2 * i] * f16_bits_to_f32(sw[i] & 0xFFFFu);
    t[2 * i + 1] = xv[2 * i + 1] * f16_bits_to_f32(sw[i] >> 16);
  }
  lstage<1>(t);                // stride 1
  lstage<2>(t);                // stride 2
  xstage<1>(t, (L & 1) != 0);  // stride 4: piece q ^ 1
  lstage<4>(t);                // stride 8: the lane's two runs
  xstage<2>(t, (L & 2) != 0);  // stride 16: piece q ^ 2
  xstage<4>(t, (L & 4) != 0);  // stride 32: group j ^ 1
  xstage<8>(t, (L & 8) != 0);  // stride 64: group j ^ 2
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_f16_bits(t[2 * i] * 0.0625f) | (f32_to_f16_bits(t[2 * i + 1] * 0.0625f) << 16);
  return o;
}

// First k of lane L's piece within its 128-block.
__device__ __forceinline__ int rotate_piece_k0(int L) { return 32 * (L >> 2) + 16 * ((L & 3) >> 1) + 4 * (L & 1); }

// ------------------------------------------------ wavefront Hadamard (fp32)
//
// Lane l holds elements 2l and 2l+1 of one 128-element block.  Stage s pairs
// elements e and e + 2^s (e with bit s clear) into (a + b, a - b); stage 0 is
// inside the lane, stage s >= 1 pairs lane l with lane l ^ 2^(s-1).
__device__ __forceinline__ void hadamard128_wave(float &x0, float &x1, int lane) {
  float a = x0 + x1;
  float b = x0 - x1;
#pragma unroll
  for (int s = 1; s < 7; ++s) {
    const int mask = 1 << (s - 1);
    const float pa = __shfl_xor(a, mask, WAVE);
    const float pb = __shfl_xor(b, mask, WAVE);
    if (lane & mask) {
      a = pa - a;
      b = pb - b;
    } else {
      a = a + pa;
      b = b + pb;
    }
  }
  x0 = a;
  x1 = b;
}

// The output stage's svh and bias words of lane l (columns n0 + 2l,
// n0 + 2l + 1).  Without a bias svh's word is loaded in its place (a line
// already on its way) and never used.
struct OutWords {
  uint32_t sv, bv;
};
__device__ __forceinline__ OutWords out_words(const uint16_t *__restrict__ svh, const uint16_t *__restrict__ bias,
                                              int n0, int lane) {
  return OutWords{*(const uint32_t *)(svh + n0 + 2 * lane),
                  *(const uint32_t *)((bias != nullptr ? bias : svh) + n0 + 2 * lane)};
}

// Output stage for one 128-column block of one row, on one wave:
// y = rne_out(svh * 2^-3 * H128(z) [+ bias]), the bias (fp16, optional)
// added in fp32 before the one rounding; lane l owns columns n0 + 2l,
// n0 + 2l + 1, whose svh and bias words are w.  Branch-free bias: without
// one, add -0.0, the exact identity of fp32 addition (+0 + -0 = +0,
// -0 + -0 = -0).
template <bool OUT_BF16>
__device__ __forceinline__ void output_row_words(float z0, float z1, OutWords w, bool has_bias,
                                                 uint16_t *__restrict__ yrow, int n0, int lane) {
  hadamard128_wave(z0, z1, lane);
  const float b0 = has_bias ? f16_bits_to_f32(w.bv & 0xFFFFu) : -0.0f;
  const float b1 = has_bias ? f16_bits_to_f32(w.bv >> 16) : -0.0f;
  const float y0 = keep_f32(keep_f32((z0 * 0.125f) * f16_bits_to_f32(w.sv & 0xFFFFu)) + b0);
  const float y1 = keep_f32(keep_f32((z1 * 0.125f) * f16_bits_to_f32(w.sv >> 16)) + b1);
  uint32_t packed;
  if constexpr (OUT_BF16) packed = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
  else packed = f32_to_f16_bits(y0) | (f32_to_f16_bits(y1) << 16);
  *(uint32_t *)(yrow + n0 + 2 * lane) = packed;
}

// The same with the words loaded here, before the butterfly so that their
// latency overlaps it.
template <bool OUT_BF16>
__device__ __forceinline__ void output_row(float z0, float z1, const uint16_t *__restrict__ svh,
                                           const uint16_t *__restrict__ bias, uint16_t *__restrict__ yrow, int n0,
                                           int lane) {
  output_row_words<OUT_BF16>(z0, z1, out_words(svh, bias, n0, lane), bias != nullptr, yrow, n0, lane);
}

// ---------------------------------------------- output stage, 8 rows a wave
//
// The same output stage on eight rows of a 128-column block at a time, with
// most of the butterfly inside each lane.  Lane L takes row ((L >> 2) & 1) +
// 2 (L >> 4) of the eight and the 16 consecutive columns 16q .. 16q + 15,
// q = (L & 3) | (((L >> 3) & 1) << 2), so column bits 0-3 are the lane's
// register index and column bits 4, 5 and 6 are lane bits 0, 1 and 3.  The
// strides 1, 2, 4 and 8 are lane-local adds; 16, 32 and 64 pair lanes that
// differ in bit 0, 1 or 3, whose values arrive by DPP moves (quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_ror:8) with no LDS round trip.  The
// stage order and every add are those of output_row_words, so the bits are
// the same: the lane holding the upper element of a pair adds its negation
// to the lower element (a + (-b), exactly a - b), the lower lane adds the
// upper element to its own (b + a = a + b).
struct OutWords16 {
  u32x4_t sv[2], bv[2];  // fp16 svh and bias pairs of the lane's 16 columns
};
__device__ __forceinline__ int rows8_group(int lane) { return (lane & 3) | (((lane >> 3) & 1) << 2); }
__device__ __forceinline__ int rows8_row(int lane) { return ((lane >> 2) & 1) + 2 * (lane >> 4); }

__device__ __forceinline__ OutWords16 out_words16(const uint16_t *__restrict__ svh, const uint16_t *__restrict__ bias,
                                                  int n0, int lane) {
  const int c = n0 + 16 * rows8_group(lane);
  const uint16_t *b = bias != nullptr ? bias : svh;
  OutWords16 w;
  w.sv[0] = *(const u32x4_t *)(svh + c);
  w.sv[1] = *(const u32x4_t *)(svh + c + 8);
  w.bv[0] = *(const u32x4_t *)(b + c);
  w.bv[1] = *(const u32x4_t *)(b + c + 8);
  return w;
}

template <int CTRL>
__device__ __forceinline__ void hadamard_lane_stage(float (&v)[16], bool upper) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float other = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[i]), CTRL, 0xF, 0xF, false));
    v[i] = other + (upper ? -v[i] : v[i]);
  }
}

// v: the lane's 16 values of its row (columns 16q .. 16q + 15 of the block),
// yrow: the row of y, n0: the block's first column.
template <bool OUT_BF16>
__device__ __forceinline__ void output_row16(float (&v)[16], const OutWords16 &w, bool has_bias,
                                             uint16_t *__restrict__ yrow, int n0, int lane) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int bit = 1 << s;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!(i & bit)) {
        const float a = v[i], b = v[i | bit];
        v[i] = a + b;
        v[i | bit] = a - b;
      }
  }
  hadamard_lane_stage<0xB1>(v, (lane & 1) != 0);   // quad_perm [1,0,3,2]: stride 16
  hadamard_lane_stage<0x4E>(v, (lane & 2) != 0);   // quad_perm [2,3,0,1]: stride 32
  hadamard_lane_stage<0x128>(v, (lane & 8) != 0);  // row_ror:8: stride 64
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sv = w.sv[i >> 2][i & 3], bv = w.bv[i >> 2][i & 3];
    const float b0 = has_bias ? f16_bits_to_f32(bv & 0xFFFFu) : -0.0f;
    const float b1 = has_bias ? f16_bits_to_f32(bv >> 16) : -0.0f;
    const float y0 = keep_f32(keep_f32((v[2 * i] * 0.125f) * f16_bits_to_f32(sv & 0xFFFFu)) + b0);
    const float y1 = keep_f32(keep_f32((v[2 * i + 1] * 0.125f) * f16_bits_to_f32(sv >> 16)) + b1);
    if constexpr (OUT_BF16) packed[i] = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
    else packed[i] = f32_to_f16_bits(y0) | (f32_to_f16_bits(y1) << 16);
  }
  uint16_t *dst = yrow + n0 + 16 * rows8_group(lane);
  *(u32x4_t *)dst = u32x4_t{packed[0], packed[1], packed[2], packed[3]};
  *(u32x4_t *)(dst + 8) = u32x4_t{packed[4], packed[5], packed[6], packed[7]};
}

// Eight rows r0 .. r0+7 of z (LDS, rows of `stride` floats, 16-byte
// aligned) through the output stage into y rows row0 .. row0+7; rows at or
// past rend are skipped.  The DPP partners of a lane always work on the same
// row (they differ in lane bits 0, 1 and 3 only), so skipping whole rows
// leaves every partner of a working lane active.
template <bool OUT_BF16>
__device__ __forceinline__ void output_rows8(const float *z, int stride, int r0, const OutWords16 &w, bool has_bias,
                                             uint16_t *__restrict__ y, int64_t row0, int64_t rend, int N, int n0,
                                             int lane) {
  const int r = rows8_row(lane);
  if (row0 + r >= rend) return;
  const float *src = z + (r0 + r) * stride + 16 * rows8_group(lane);
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4_t t = *(const float4_t *)(src + 4 * i);
    v[4 * i] = t[0];
    v[4 * i + 1] = t[1];
    v[4 * i + 2] = t[2];
    v[4 * i + 3] = t[3];
  }
  output_row16<OUT_BF16>(v, w, has_bias, y + (row0 + r) * N, n0, lane);
}

// Ordered sum of K-part partials for four rows of one 128-column block, then
// the output stage of those rows.  Slabs are [n_slabs][M4][N][4] fp32 (the
// four rows of a column are 16 contiguous bytes); lane l holds columns
// n0 + 2l, n0 + 2l + 1.  The sum is the shape-fixed two-level order: each run
// of fold_q consecutive slabs (one group of parts) is folded in order, the
// first slab copied, and the group sums are folded in group order, the first
// copied (TensorFold PR, "Arithmetic": a shape-fixed number of parts added in
// part order, so a row's bits do not depend on the batch).  With fold_q = 1
// it is the plain fold ((s0 + s1) + s2) + ...  Loads are issued U slabs at
// a time before their adds.
template <bool OUT_BF16, int U = 8>
__device__ __forceinline__ void reduce_rows4(const float *__restrict__ slabs, int n_slabs, int fold_q,
                                             int64_t slab_floats, int N, int64_t m4, int n0,
                                             const uint16_t *__restrict__ svh, const uint16_t *__restrict__ bias,
                                             uint16_t *__restrict__ y, int64_t row0, int rows, int lane) {
  const float4_t *src = reinterpret_cast<const float4_t *>(slabs + (m4 * N + n0 + 2 * lane) * 4);
  const int64_t st = slab_floats / 4;  // float4s per slab
  float4_t t0 = {0.f, 0.f, 0.f, 0.f}, t1 = t0, g0 = t0, g1 = t0;
  int iq = 0;  // position of slab i inside its group
  for (int i0 = 0; i0 < n_slabs; i0 += U) {
    float4_t v0[U], v1[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u < n_slabs) {
        v0[u] = src[(i0 + u) * st];
        v1[u] = src[(i0 + u) * st + 1];
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
        if (++iq == fold_q) {
          iq = 0;
          if (i0 + u + 1 == fold_q) {
            t0 = g0;
            t1 = g1;
          } else {
            t0 = t0 + g0;
            t1 = t1 + g1;
          }
        }
      }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (r < rows) output_row<OUT_BF16>(t0[r], t1[r], svh, bias, y + (row0 + r) * N, n0, lane);
}

}  // namespace exl3
