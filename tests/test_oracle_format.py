"""Pins for oracle.format: codebooks, tile unpacking and the in-tile value order.

Each check reaches the oracle's answer by another route than the oracle's
own code: values worked by hand from the page's constants, closed forms,
brute force over single tiles with Python integers and strings, CPython's
own fp16 rounding (struct 'e'), and the public PTX fragment layout.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import format as fmt

CBS = (fmt.CB_3INST, fmt.CB_MCG, fmt.CB_MUL1)


def f16_bits_of_exact(q: Fraction) -> int:
    """fp16 round-to-nearest-even of an exact rational, via CPython's packer."""
    # float(q) is exact for every q below (at most 22 significant bits).
    assert Fraction(float(q)) == q
    return struct.unpack("<H", struct.pack("<e", float(q)))[0]


def f16_value(bits: int) -> Fraction:
    return Fraction(struct.unpack("<e", struct.pack("<H", bits))[0])


# ---------------------------------------------------------------------------
# codebooks
# ---------------------------------------------------------------------------

def test_mcg_worked_by_hand():
    # The page's mcg multiplier is 0xCBAC1FED ("GLM-5.3-Flash").
    # s = 0: u = 0 -> masked halves 0x3000, 0x3000 = 0.125 + 0.125 = 0.25.
    # s = 1: u = 0xCBAC1FED.  hi 0xCBAC & 0x8FFF = 0x8BAC, ^0x3000 -> 0xBBAC
    #        = -(1 + 940/1024) * 2**-1 = -0.958984375;
    #        lo 0x1FED & 0x8FFF = 0x0FED, ^0x3000 -> 0x3FED = 1 + 1005/1024
    #        = 1.9814453125.  Sum 1.0224609375 = 1 + 23/1024 -> 0x3C17.
    # s = 2: u = 0x197583FDA mod 2**32 = 0x97583FDA.  hi 0x9758 -> 0x8758 ->
    #        0xB758 = -(1 + 856/1024) / 4 = -0.458984375; lo 0x3FDA -> 0x0FDA
    #        -> 0x3FDA = 1 + 986/1024 = 1.962890625.  Sum 1.50390625
    #        = 1 + 516/1024 -> 0x3E04.
    got = fmt.codebook(fmt.CB_MCG, np.array([0, 1, 2]))
    assert [int(v) for v in got] == [0x3400, 0x3C17, 0x3E04]


def test_3inst_worked_by_hand():
    # s = 0: u = 0x3C6EF372.  hi 0x3C6E & 0x8FFF = 0x0C6E -> 0x3C6E
    # = 1 + 110/1024 = 1.107421875; lo 0xF372 & 0x8FFF = 0x8372 -> 0xB372
    # = -(1 + 882/1024) / 8 = -0.232666015625.  Sum 0.874755859375 =
    # (1 + 767.5/1024) / 2: a tie between mantissas 767 and 768, so round to
    # even 768 -> 0x3800 | 0x300 = 0x3B00.
    got = fmt.codebook(fmt.CB_3INST, np.array([0]))
    assert int(got[0]) == 0x3B00


def test_mul1_worked_by_hand():
    # s = 0: t = 0, value = beta = fp16 0xC2E8 exactly.
    # s = 1: u = 0x9E3779B1, bytes 158 + 55 + 121 + 177 = 511;
    #   511 * alpha + beta = 511 * 0.00676727294921875 - 3.453125
    #   = 0.00495147705078125 = 2**-8 * (1 + 274/1024) -> 0x1C00 | 274 = 0x1D12.
    got = fmt.codebook(fmt.CB_MUL1, np.array([0, 1]))
    assert [int(v) for v in got] == [0xC2E8, 0x1D12]
    assert f16_value(fmt.MUL1_ALPHA_BITS) == Fraction(1774, 262144)  # 0x1EEE = 2**-8 * (1 + 750/1024)
    assert f16_value(fmt.MUL1_BETA_BITS) == Fraction(-221, 64)       # 0xC2E8


@pytest.mark.parametrize("cb", CBS)
def test_every_state_decodes_finite(cb):
    # The pages: every one of the 65,536 codes decodes finite in every codebook.
    tab = fmt.codebook_table(cb)
    vals = tab.view(np.float16).astype(np.float64)
    assert tab.shape == (65536,)
    assert np.all(np.isfinite(vals))
    # distribution sanity: centred, unit-order variance
    assert abs(vals.mean()) < 0.05
    assert 0.5 < vals.var() < 2.0


@pytest.mark.parametrize("cb", (fmt.CB_3INST, fmt.CB_MCG))
def test_pair_sum_codebooks_against_cpython_rounding(cb):
    # Recompute a sample of states with exact rationals and CPython's fp16
    # packer (independent of numpy's float -> half conversion).
    mult, add = (0x2C9277B5, 0x3C6EF372) if cb == fmt.CB_3INST else (0xCBAC1FED, 0)
    rng = np.random.default_rng(5)
    states = rng.integers(0, 65536, size=3000)
    got = fmt.codebook(cb, states)
    for s, g in zip(states.tolist(), got.tolist()):
        u = (s * mult + add) % 2 ** 32
        m = (u & 0x8FFF8FFF) ^ 0x30003000
        q = f16_value(m & 0xFFFF) + f16_value(m >> 16)
        assert abs(q) < 4
        assert g == f16_bits_of_exact(q), (hex(s), hex(g))


def test_mul1_is_one_rounding_of_an_exact_sum():
    rng = np.random.default_rng(6)
    states = rng.integers(0, 65536, size=3000)
    got = fmt.codebook(fmt.CB_MUL1, states)
    alpha = f16_value(fmt.MUL1_ALPHA_BITS)
    beta = f16_value(fmt.MUL1_BETA_BITS)
    for s, g in zip(states.tolist(), got.tolist()):
        u = (s * 0x9E3779B1) % 2 ** 32
        t = sum(u.to_bytes(4, "little"))
        assert g == f16_bits_of_exact(t * alpha + beta)
    # at most 1021 distinct values, monotone in the byte sum
    tab = fmt.codebook_table(fmt.CB_MUL1)
    assert len(np.unique(tab)) <= 1021


def test_gpu_fma_form_of_mul1_is_exact():
    # The decoder may evaluate t*alpha + beta as (1024 + t)*alpha + c with
    # c = beta - 1024*alpha; that is the same exact sum provided c is an fp16.
    alpha = f16_value(fmt.MUL1_ALPHA_BITS)
    beta = f16_value(fmt.MUL1_BETA_BITS)
    c = beta - 1024 * alpha
    assert f16_value(f16_bits_of_exact(c)) == c


# ---------------------------------------------------------------------------
# unpacking
# ---------------------------------------------------------------------------

def brute_states(words, bits):
    """Brute force with strings: the tile's bits as '0'/'1', MSB first."""
    stream = "".join(format(int(w), "016b") for w in words)
    assert len(stream) == 256 * bits
    ring = stream + stream
    return [int(ring[v * bits:v * bits + 16], 2) for v in range(256)]


@pytest.mark.parametrize("bits", range(1, 9))
def test_unpack_brute_force(bits):
    rng = np.random.default_rng(100 + bits)
    for _ in range(3):
        words = rng.integers(0, 65536, size=16 * bits, dtype=np.uint16)
        assert fmt.tile_states(words, bits).tolist() == brute_states(words, bits)


@pytest.mark.parametrize("bits", range(1, 9))
def test_unpack_constant_tiles(bits):
    zeros = np.zeros(16 * bits, dtype=np.uint16)
    ones = np.full(16 * bits, 0xFFFF, dtype=np.uint16)
    assert np.all(fmt.tile_states(zeros, bits) == 0)
    assert np.all(fmt.tile_states(ones, bits) == 0xFFFF)


@pytest.mark.parametrize("bits", range(1, 9))
def test_unpack_single_bit(bits):
    length = 256 * bits
    for p in (0, 1, 15, 16, 17, length // 2 + 3, length - 16, length - 1):
        words = np.zeros(16 * bits, dtype=np.uint16)
        words[p // 16] = 1 << (15 - p % 16)  # stream bit p (MSB first)
        st = fmt.tile_states(words, bits)
        for v in range(256):
            d = (p - v * bits) % length
            want = (1 << (15 - d)) if d < 16 else 0
            assert st[v] == want, (bits, p, v)


def test_unpack_8bit_is_byte_pairs():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 65536, size=128, dtype=np.uint16)
    byts = [b for w in words.tolist() for b in (w >> 8, w & 0xFF)]  # MSB first
    st = fmt.tile_states(words, 8)
    assert st.tolist() == [(byts[v] << 8) | byts[(v + 1) % 256] for v in range(256)]


@pytest.mark.parametrize("bits", range(1, 9))
def test_unpack_shift_register(bits):
    rng = np.random.default_rng(200 + bits)
    words = rng.integers(0, 65536, size=16 * bits, dtype=np.uint16)
    st = fmt.tile_states(words, bits).astype(np.int64)
    stream = fmt.tile_stream_bits(words, bits)
    for v in range(255):
        nxt = 0
        for j in range(bits):
            nxt = (nxt << 1) | int(stream[(v * bits + 16 + j) % (256 * bits)])
        assert st[v + 1] == ((st[v] << bits) | nxt) & 0xFFFF


# ---------------------------------------------------------------------------
# value order
# ---------------------------------------------------------------------------

def test_value_order_matches_ptx_b_fragment():
    # PTX ISA, mma.m16n8k16 with .f16 B (16x8): thread `lane` holds b0..b3 at
    # row = (lane % 4) * 2 + (i & 1) (+ 8 for b2, b3), col = lane // 4.  The
    # tile's second 8 columns are the second product.  Value v = 8*lane +
    # 4*h + i.  Hand-derived points:
    cases = {0: (0, 0), 1: (1, 0), 2: (8, 0), 3: (9, 0), 4: (0, 8), 7: (9, 8),
             8: (2, 0), 26: (14, 0), 27: (15, 0), 31: (15, 8), 32: (0, 1), 36: (0, 9),
             254: (14, 15), 255: (15, 15)}
    for v, kn in cases.items():
        assert fmt.value_position(v) == kn, v
    pos = {fmt.value_position(v) for v in range(256)}
    assert len(pos) == 256  # a bijection onto the 16 x 16 tile


@pytest.mark.parametrize("bits,cb", [(2, fmt.CB_3INST), (5, fmt.CB_MCG), (8, fmt.CB_MUL1)])
def test_dequantize_tile_placement(bits, cb):
    # A 32 x 48 matrix (2 x 3 tiles), decoded tile by tile with the brute
    # force unpacker and placed by hand.
    rng = np.random.default_rng(300 + bits)
    tr = rng.integers(0, 65536, size=(2, 3, 16 * bits), dtype=np.uint16)
    got = fmt.dequantize_bits(tr, bits, cb)
    assert got.shape == (32, 48)
    for kt in range(2):
        for nt in range(3):
            st = brute_states(tr[kt, nt], bits)
            vals = fmt.codebook(cb, np.array(st))
            for v in range(256):
                k, n = fmt.value_position(v)
                assert got[16 * kt + k, 16 * nt + n] == vals[v]
