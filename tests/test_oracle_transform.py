"""Pins for oracle.transform: the Hadamard, both rotations and the roundings."""
import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import transform as tf


def test_sylvester_matches_scipy_and_is_orthogonal():
    h = tf.sylvester()
    assert np.array_equal(h, scipy.linalg.hadamard(128).astype(np.float64))
    assert np.array_equal(h @ h, 128 * np.eye(128))


def test_butterfly_is_the_hadamard_product():
    h = scipy.linalg.hadamard(128).astype(np.float64)
    for j in (0, 1, 5, 64, 127):
        e = np.zeros(128)
        e[j] = 1.0
        assert np.array_equal(tf.butterfly(e), h[:, j])  # one-hot closed form
    rng = np.random.default_rng(1)
    v = rng.standard_normal((3, 384))
    want = (v.reshape(3, 3, 128) @ h).reshape(3, 384)  # block diagonal
    assert np.allclose(tf.butterfly(v), want, rtol=0, atol=1e-12)


def test_butterfly_float32_add_order():
    # Strides ascend: with t = [1, 0, 2**-24, 2**-24, 0, ...] stage 0 forms
    # t2 + t3 = 2**-23 first, and stage 1 adds it to t0 + t1 = 1 exactly:
    # out[0] = 1 + 2**-23.  With descending strides t0 would meet t2 first and
    # 1 + 2**-24 rounds (ties to even) to 1, twice: out[0] = 1.
    t = np.zeros(128, dtype=np.float32)
    t[0], t[2], t[3] = 1.0, 2.0 ** -24, 2.0 ** -24
    out = tf.butterfly(t)
    assert out.dtype == np.float32 and out[0] == np.float32(1.0 + 2.0 ** -23)


def test_rotate_one_hot_closed_form():
    # x = e_j (bf16 1.0 = 0x3F80), suh = 1: x~ = +-2**-4 (fp16 0x2C00 / 0xAC00)
    # following the signs of Hadamard column j.
    h = scipy.linalg.hadamard(128)
    for j in (0, 3, 77, 127):
        x = np.zeros((1, 128), dtype=np.uint16)
        x[0, j] = 0x3F80
        suh = np.full((1, 128), 0x3C00, dtype=np.uint16)
        xr = tf.rotate_input(x, suh, "bf16")[0, 0]
        want = np.where(h[:, j] > 0, 0x2C00, 0xAC00).astype(np.uint16)
        assert np.array_equal(xr, want)


def test_rotate_replay_within_one_ulp_of_exact():
    rng = np.random.default_rng(2)
    x = tf.f32_to_bf16_bits(rng.standard_normal((9, 512)).astype(np.float32))
    suh = (np.where(rng.integers(0, 2, (2, 512)) == 1, -1.0, 1.0)
           * np.exp2(rng.uniform(-2, 2, (2, 512)))).astype(np.float16).view(np.uint16)
    xr = tf.f16_from_bits(tf.rotate_input(x, suh)).astype(np.float64)
    ex = tf.rotate_input_f64(x, suh)
    ulp = np.spacing(np.abs(ex).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(xr - ex) <= ulp)
    # and the suh scale really is applied per shard
    assert not np.array_equal(xr[0], xr[1])


def test_rotate_block_diagonal():
    # Splitting K at a multiple of 128 is exact (the pages' tensor-parallel note).
    rng = np.random.default_rng(3)
    x = tf.f32_to_bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    suh = np.full((1, 256), 0xBC00, dtype=np.uint16)
    whole = tf.rotate_input(x, suh)
    left = tf.rotate_input(x[:, :128], suh[:, :128])
    right = tf.rotate_input(x[:, 128:], suh[:, 128:])
    assert np.array_equal(whole, np.concatenate([left, right], axis=-1))


def test_rotate_fp16_input():
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 5] = 0x4000  # fp16 2.0
    suh = np.full((1, 128), 0x3800, dtype=np.uint16)  # 0.5
    xr = tf.rotate_input(x, suh, "f16")[0, 0]
    h = scipy.linalg.hadamard(128)
    assert np.array_equal(xr, np.where(h[:, 5] > 0, 0x2C00, 0xAC00).astype(np.uint16))


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_output_one_hot_closed_form(out_dtype):
    # z = e_j in one 128-column block: y = +-(1/8) * svh, exactly representable.
    h = scipy.linalg.hadamard(128)
    rng = np.random.default_rng(4)
    svh = (np.where(rng.integers(0, 2, 256) == 1, -1.0, 1.0) * 2.0 ** rng.integers(-3, 3, 256))
    svh_bits = svh.astype(np.float16).view(np.uint16)
    z = np.zeros((1, 256), dtype=np.float32)
    z[0, 128 + 9] = 1.0
    y = tf.output_transform_f32(z, svh_bits, out_dtype)
    want = np.zeros(256)
    want[128:] = h[:, 9] * svh[128:] / 8
    got = (tf.bf16_bits_to_f32(y) if out_dtype == "bf16" else tf.f16_from_bits(y)).astype(np.float64)
    assert np.array_equal(got[0], want)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    a = rng.standard_normal(100000).astype(np.float32) * np.float32(1e3)
    # explicit ties: low 16 bits exactly 0x8000, both parities of bit 16
    # values in [1, 2) whose low 16 bits are exactly half a bf16 ulp
    ties = ((rng.integers(0, 128, 256, dtype=np.uint32) << 16) | 0x3F808000).view(np.float32)
    a = np.concatenate([a, ties, -ties, np.array([0.0, -0.0], np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tf.f32_to_bf16_bits(a), want)


def test_f16_rounding_matches_torch():
    rng = np.random.default_rng(6)
    a = rng.standard_normal(100000).astype(np.float32) * np.float32(30)
    want = torch.from_numpy(a).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tf.f32_to_f16_bits(a), want)


def test_reduce_parts_is_left_to_right():
    # ((1 + 2**-24) + 2**-24) = 1 in float32 (ties to even twice), while
    # 1 + (2**-24 + 2**-24) = 1 + 2**-23: the order is observable.
    parts = np.array([1.0, 2.0 ** -24, 2.0 ** -24], dtype=np.float32).reshape(3, 1, 1)
    assert tf.reduce_parts_f32(parts)[0, 0] == np.float32(1.0)
    # the first part is copied, not added to +0: -0.0 survives
    neg = np.array([-0.0], dtype=np.float32).reshape(1, 1, 1)
    assert np.signbit(tf.reduce_parts_f32(neg)[0, 0])


def test_reduce_parts_grouped_tree():
    # Groups of two: (1 + 2**-24) = 1 (tie to even) and (2**-24 + 2**-24) =
    # 2**-23 exactly, so the grouped total is 1 + 2**-23, while the flat
    # left-to-right fold absorbs every 2**-24 into 1 and stays at 1.
    parts = np.array([1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24], dtype=np.float32).reshape(4, 1, 1)
    assert tf.reduce_parts_f32(parts)[0, 0] == np.float32(1.0)
    assert tf.reduce_parts_f32(parts, groups=4)[0, 0] == np.float32(1.0)
    assert tf.reduce_parts_f32(parts, groups=1)[0, 0] == np.float32(1.0)
    assert tf.reduce_parts_f32(parts, groups=2)[0, 0] == np.float32(1.0 + 2.0 ** -23)
    with pytest.raises(ValueError):
        tf.reduce_parts_f32(parts, groups=3)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_output_bias_closed_forms(out_dtype):
    """The bias (reading R16): z = 0 gives rne_out(bias) exactly; a one-hot z
    of value v in a block gives rne_out(fp32(+-v * 2**-3 * svh) + bias) in
    every column of the block, the sign that of the Hadamard column."""
    rng = np.random.default_rng(7)
    N = 256
    svh = (np.where(rng.integers(0, 2, N) == 1, -1.0, 1.0) * np.exp2(rng.uniform(-2, 2, N))).astype(np.float16)
    bias = (rng.standard_normal(N) * 3).astype(np.float16)
    rnd = tf.f32_to_bf16_bits if out_dtype == "bf16" else tf.f32_to_f16_bits
    zero = tf.output_transform_f32(np.zeros((2, N), np.float32), svh.view(np.uint16), out_dtype, bias.view(np.uint16))
    assert np.array_equal(zero, np.broadcast_to(rnd(bias.astype(np.float32)), (2, N)))
    h = scipy.linalg.hadamard(128)
    z = np.zeros((1, N), np.float32)
    z[0, 128 + 5] = v = np.float32(3.75)
    got = tf.output_transform_f32(z, svh.view(np.uint16), out_dtype, bias.view(np.uint16))
    sgn = np.concatenate([np.zeros(128), h[:, 5]])
    want = np.empty(N, np.float32)
    for n in range(N):
        a = np.float32(np.float32(np.float32(sgn[n]) * v) * np.float32(0.125)) * np.float32(svh[n])
        want[n] = np.float32(a + np.float32(bias[n]))
    assert np.array_equal(got[0], rnd(want))
    # without a bias the old result
    assert np.array_equal(tf.output_transform_f32(z, svh.view(np.uint16), out_dtype),
                          rnd((np.float32(0.125) * np.float32(3.75) * sgn.astype(np.float32)
                               * svh.astype(np.float32)).astype(np.float32))[None])


def test_exp_f32_against_the_exponential():
    """Reading R17's exp: within 2 ulp of float64 e^x over the whole finite
    range, exact at 0, overflow to inf and underflow to 0 past +-104."""
    x = np.linspace(-87, 88, 100001).astype(np.float32)
    e = tf.exp_f32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    assert np.all(np.abs(e - ref) <= 2 * np.spacing(ref.astype(np.float32)).astype(np.float64))
    edge = tf.exp_f32(np.array([0.0, 200.0, -200.0], np.float32))
    assert edge[0] == 1.0 and np.isinf(edge[1]) and edge[2] == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_swiglu_against_float64(dtype):
    """act = rne(silu(g) * u): within one output ulp of the float64 value for
    every pair (the fp32 steps round at most a few fp32 ulps), and equal to
    the float64 value's rounding for nearly all; silu(0) = 0 exactly and the
    sign of u carries through."""
    rng = np.random.default_rng(11)
    M, K = 64, 512
    f = (rng.standard_normal((M, 2 * K)) * np.exp2(rng.uniform(-6, 4, (M, 2 * K)))).astype(np.float32)
    bits = tf.f32_to_bf16_bits(f) if dtype == "bf16" else tf.f32_to_f16_bits(f)
    act = tf.swiglu_bits(bits, dtype)
    to64 = (lambda b: tf.bf16_bits_to_f32(b).astype(np.float64)) if dtype == "bf16" else \
        (lambda b: tf.f16_from_bits(b).astype(np.float64))
    g, u = to64(bits[:, :K]), to64(bits[:, K:])
    exact = g / (1.0 + np.exp(-g)) * u
    rnd = tf.f32_to_bf16_bits if dtype == "bf16" else tf.f32_to_f16_bits
    want = rnd(exact.astype(np.float32))
    assert np.mean(act == want) > 0.999
    off = act != want  # anywhere else: the neighbouring code of the same sign (one output ulp)
    assert np.all(np.abs(act[off].astype(np.int32) - want[off].astype(np.int32)) == 1)
    zero = np.zeros((1, 256), np.uint16)
    assert np.all(tf.swiglu_bits(zero, dtype) == 0)
