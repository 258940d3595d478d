"""Pins for oracle.moe: the alignment by hand and the combine by closed forms."""
import numpy as np

from oracle import moe
from oracle import transform as tf


def test_align_worked_example():
    # pairs p = t*2 + j: experts 0,1 | 1,2 | 0,0 ; 3 experts, blocks of 16
    ids = np.array([[0, 1], [1, 2], [0, 0]])
    rows, runs, be = moe.align_runs(ids, 3, 16)
    assert rows == 64  # 6 pairs + 3 experts x 15 padding = 51 -> 64
    assert runs[0][0] == 0 and list(runs[0][1]) == [0, 4, 5]
    assert runs[1][0] == 16 and list(runs[1][1]) == [1, 2]
    assert runs[2][0] == 32 and list(runs[2][1]) == [3]
    assert list(be) == [0, 1, 2, -1]


def test_align_drops_unknown_experts_and_skips_empty_ones():
    ids = np.array([[5, -1], [2, 2]])  # 5 and -1 are not experts of 4
    rows, runs, be = moe.align_runs(ids, 4, 16)
    assert len(runs[0][1]) == 0 and len(runs[1][1]) == 0 and list(runs[2][1]) == [2, 3]
    assert runs[2][0] == 0 and list(be[:1]) == [2] and np.all(be[1:] == -1)


def test_combine_closed_forms():
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((8, 6)) * 4).astype(np.float32)
    yb = tf.f32_to_bf16_bits(y)
    pair_row = np.array([3, 0, -1, 5])  # T=2, k=2; token 1's first pair dropped
    w = np.array([[1.0, 0.0], [2.0, 0.5]], np.float32)
    out = moe.combine_bits(yb, "bf16", pair_row, w)
    yv = tf.bf16_bits_to_f32(yb)
    assert np.array_equal(out[0], tf.f32_to_bf16_bits(yv[3] + np.float32(0) * yv[0]))  # 1*y + 0*y
    assert np.array_equal(out[1], tf.f32_to_bf16_bits((np.float32(0.5) * yv[5]).astype(np.float32)))
    # two terms: fp32(w0*y0) + fp32(w1*y1) rounded once (not twice)
    a, b = np.float32(1.0), np.float32(2.0 ** -9)
    yy = tf.f32_to_bf16_bits(np.array([[a], [b]], np.float32))
    out2 = moe.combine_bits(yy, "bf16", np.array([0, 1]), np.array([[1.0, 1.0]], np.float32))
    assert tf.bf16_bits_to_f32(out2)[0, 0] == np.float32(1.0)  # 1 + 2^-9 rounds to 1 in bf16 once
    # 1 + 3 * 2^-9 = 1 + 0.75 bf16 ulp in fp32, rounded once: 1 + 2^-7 (each
    # add rounded to bf16 would stay at 1)
    out3 = moe.combine_bits(yy, "bf16", np.array([0, 1, 1, 1]), np.array([[1.0, 1.0, 1.0, 1.0]], np.float32))
    assert tf.bf16_bits_to_f32(out3)[0, 0] == np.float32(1.0 + 2.0 ** -7)
