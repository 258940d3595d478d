"""EXL3 trellis format, decoded the plain way (oracle; test infrastructure).

What the pages fix
------------------
* A weight matrix is stored as 16x16 tiles, ``trellis[K/16][N/16][16*bits]``
  int16 words; each tile carries 256 weights at ``bits`` bits each (1..8),
  and each weight is decoded from a 16-bit state (TensorFold PR "cuda: EXL3
  projections behind qlinear", "What it adds"; cuda-exl3 page, "What is
  supported").
* Decoding a run of consecutive values reads a sliding window over the tile's
  bit stream: eight 6-bit values need a 58-bit window, i.e. 7*6+16 bits
  (cuda-exl3 page, "Where the time goes", the list of rejected changes), so
  value v's state is the 16 bits that start v*bits bits into the stream.
* Three procedural codebooks map a state to fp16: 3inst, mcg and mul1; the
  codebook id is all the decoder needs (cuda-exl3, "What is supported").
  mcg's multiplier is 0xCBAC1FED (cuda-exl3, "GLM-5.3-Flash").  mul1 is one
  fused fp16 multiply-add of an exact sum, the format's single rounding
  (TensorFold PR, "Arithmetic" step 2).
* A tile's 256 values are in the order of the B fragments of two
  mma.m16n8k16 (TensorFold PR, "Arithmetic" step 2).

Readings taken where the pages are silent
-----------------------------------------
R1  Bit order: stream bit i is bit (15 - i%16) of word i//16 (MSB first in
    each 16-bit word, words in ascending order).
R2  Window anchor: state_v = stream bits [v*bits, v*bits+16), taken
    circularly modulo the tile's 256*bits bits.
R3  Value order: value v = 8*t + 4*h + i (t = fragment lane 0..31, h = which
    of the two m16n8k16 products, i = fragment element 0..3) sits at tile row
    k = 2*(t%4) + (i&1) + 8*(i>>1) and column n = t//4 + 8*h, which is the
    public PTX ISA layout of the m16n8k16 f16 B fragment.
R4  3inst: u = (s*0x2C9277B5 + 0x3C6EF372) mod 2**32, then the pair-sum map
    P(u) below (an LCG followed by mask/xor into two fp16 halves that are
    added, in the manner of QTIP's 3INST code).
R5  mcg: u = (s*0xCBAC1FED) mod 2**32 (the page's multiplier), then P(u).
R6  P(u): u' = (u & 0x8FFF8FFF) ^ 0x30003000; value = fp16 round-to-nearest
    -even of (fp16(u'[15:0]) + fp16(u'[31:16])).  The two halves lie in
    +-[0.125, 2), their sum is exact in fp64, so there is one rounding.
R7  mul1: u = (s*0x9E3779B1) mod 2**32, t = sum of u's four bytes (0..1020,
    exact in fp16), value = fp16 RNE of t*alpha + beta with alpha = fp16
    0x1EEE and beta = fp16 0xC2E8: one fused multiply-add, one rounding.

Parity status: every function here is pinned by tests/test_oracle_format.py
(closed forms, brute force over single tiles, hand-worked values from the
page's mcg multiplier, the PTX fragment layout, and whole-table invariants).
Compatibility with real ExLlamaV3 checkpoints is parity unpinned: no
checkpoint and no format source is available to check R1-R7 against.
"""
from __future__ import annotations

import numpy as np

CB_3INST, CB_MCG, CB_MUL1 = 0, 1, 2
CODEBOOK_NAMES = {CB_3INST: "3inst", CB_MCG: "mcg", CB_MUL1: "mul1"}

_MASK32 = 0xFFFFFFFF


def _f16_of_bits(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> float64 values (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _bits_of_f64_as_f16(values: np.ndarray) -> np.ndarray:
    """Round float64 to fp16 (nearest, ties to even) and return the bits."""
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def pair_sum(u: np.ndarray) -> np.ndarray:
    """Reading R6: mask/xor a 32-bit word into two fp16 halves and add them.

    Returns fp16 bits.  Both halves have biased exponents 12..15, so each is
    in +-[0.125, 2); their sum is exact in float64 and rounded once to fp16.
    """
    u = np.asarray(u, dtype=np.uint64) & _MASK32
    m = (u & 0x8FFF8FFF) ^ 0x30003000
    lo = _f16_of_bits((m & 0xFFFF).astype(np.uint16))
    hi = _f16_of_bits((m >> 16).astype(np.uint16))
    return _bits_of_f64_as_f16(lo + hi)


MUL1_ALPHA_BITS = 0x1EEE
MUL1_BETA_BITS = 0xC2E8


def codebook(cb: int, states: np.ndarray) -> np.ndarray:
    """Decode 16-bit states to fp16 bits with codebook ``cb`` (R4-R7)."""
    s = np.asarray(states, dtype=np.uint64) & 0xFFFF
    if cb == CB_3INST:
        return pair_sum((s * 0x2C9277B5 + 0x3C6EF372) & _MASK32)
    if cb == CB_MCG:
        return pair_sum((s * 0xCBAC1FED) & _MASK32)
    if cb == CB_MUL1:
        u = (s * 0x9E3779B1) & _MASK32
        t = (u & 0xFF) + ((u >> 8) & 0xFF) + ((u >> 16) & 0xFF) + ((u >> 24) & 0xFF)
        alpha = _f16_of_bits(np.array(MUL1_ALPHA_BITS, dtype=np.uint16))
        beta = _f16_of_bits(np.array(MUL1_BETA_BITS, dtype=np.uint16))
        # t*alpha + beta is exact in float64 (t < 2**10, alpha has 11
        # significant bits); the conversion to fp16 is the single rounding.
        return _bits_of_f64_as_f16(t.astype(np.float64) * alpha + beta)
    raise ValueError(f"unknown codebook id {cb}")


def codebook_table(cb: int) -> np.ndarray:
    """All 65,536 states of one codebook, as fp16 bits."""
    return codebook(cb, np.arange(65536, dtype=np.uint64))


# ---------------------------------------------------------------------------
# Tile unpacking (R1, R2)
# ---------------------------------------------------------------------------

def tile_stream_bits(words: np.ndarray, bits: int) -> np.ndarray:
    """Reading R1: the tile's bit stream, one uint8 (0/1) per bit.

    ``words`` has shape [..., 16*bits] (uint16).  Result [..., 256*bits].
    """
    w = np.asarray(words, dtype=np.uint16)
    assert w.shape[-1] == 16 * bits, (w.shape, bits)
    big_endian = w.astype(">u2")  # most significant byte first
    raw = big_endian.view(np.uint8).reshape(w.shape[:-1] + (32 * bits,))
    return np.unpackbits(raw, axis=-1)  # MSB of each byte first


def tile_states(words: np.ndarray, bits: int) -> np.ndarray:
    """Reading R2: state_v = 16 stream bits starting at v*bits, circular.

    ``words`` [..., 16*bits] -> states [..., 256] (uint16), value order v.
    """
    if not 1 <= bits <= 8:
        raise ValueError(f"bits must be 1..8, got {bits}")
    stream = tile_stream_bits(words, bits)
    length = 256 * bits
    v = np.arange(256)[:, None]
    j = np.arange(16)[None, :]
    idx = (v * bits + j) % length  # [256, 16]
    window = stream[..., idx]  # [..., 256, 16], first stream bit first
    packed = np.packbits(window, axis=-1)  # [..., 256, 2], first bit -> MSB
    return (packed[..., 0].astype(np.uint16) << 8) | packed[..., 1].astype(np.uint16)


# ---------------------------------------------------------------------------
# In-tile value order (R3)
# ---------------------------------------------------------------------------

def value_position(v: int) -> tuple[int, int]:
    """Reading R3: (row k, column n) of value v inside its 16x16 tile."""
    t, rem = divmod(v, 8)
    h, i = divmod(rem, 4)
    k = 2 * (t % 4) + (i & 1) + 8 * (i >> 1)
    n = t // 4 + 8 * h
    return k, n


VALUE_K = np.array([value_position(v)[0] for v in range(256)], dtype=np.int64)
VALUE_N = np.array([value_position(v)[1] for v in range(256)], dtype=np.int64)


def tile_grid(values: np.ndarray) -> np.ndarray:
    """Place 256 per-tile values (value order) into a [..., 16, 16] k x n grid."""
    vals = np.asarray(values)
    out = np.zeros(vals.shape[:-1] + (16, 16), dtype=vals.dtype)
    out[..., VALUE_K, VALUE_N] = vals
    return out


# ---------------------------------------------------------------------------
# Whole-matrix decode
# ---------------------------------------------------------------------------

def unpack_states(trellis: np.ndarray, bits: int) -> np.ndarray:
    """trellis [K/16, N/16, 16*bits] -> state matrix [K, N] (uint16)."""
    tr = np.asarray(trellis, dtype=np.uint16)
    kt, nt, w = tr.shape
    assert w == 16 * bits
    out = np.empty((kt * 16, nt * 16), dtype=np.uint16)
    for r in range(kt):  # one row of tiles at a time bounds the memory used
        grid = tile_grid(tile_states(tr[r], bits))  # [nt, 16, 16]
        out[16 * r:16 * r + 16] = grid.transpose(1, 0, 2).reshape(16, nt * 16)
    return out


def dequantize_bits(trellis: np.ndarray, bits: int, cb: int) -> np.ndarray:
    """W_q as fp16 bits [K, N]: W_q[16*kt + k][16*nt + n] = cb(state)."""
    return codebook(cb, unpack_states(trellis, bits))


def dequantize(trellis: np.ndarray, bits: int, cb: int) -> np.ndarray:
    """W_q as float64 [K, N] (every value is an fp16, so this is exact)."""
    return _f16_of_bits(dequantize_bits(trellis, bits, cb))
