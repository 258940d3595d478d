"""GPU: edge cases of the method's arithmetic, through the C ABI.

* Rotated activations in fp16's subnormal range: the format rounds x~ to fp16
  once (TensorFold PR "cuda: EXL3 projections behind qlinear", "Arithmetic"
  step 1) and reading R10 keeps subnormals; the rotation is bit-exact and
  the linear within the oracle's bound, which treats them exactly.
* x~ within a factor of two of fp16's largest finite value.
* Non-finite inputs (reading R18): IEEE propagation through both rotations
  and the products: a row holding a NaN or an infinity has a wholly
  non-finite output row, and every other row keeps its bits.
* The most shards a weight view takes (16), against the oracle and against
  sixteen one-shard calls with the same part tree (cuda-exl3 README, "One op
  per layer": all shards in one GEMM, only the activation slice differs)."""
import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from oracle import linear as olin
from oracle import transform as otf
from gpu_util import banner, bits16, dev16, rot_layout, weight, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ex.load()
    torch.cuda.init()


def _run(w, x_bits, out=torch.bfloat16, **force):
    xr = ex.input_transform(x_dev(x_bits), w.suh)
    y = ex.linear(w, xr, out, **force)
    torch.cuda.synchronize()
    return bits16(xr), bits16(y)


@pytest.mark.parametrize("M", [5, 40, 300])
def test_subnormal_rotated_activations(M):
    """x scaled by 2**-15: most of x~ is fp16-subnormal (below 2**-14)."""
    lay = wl.small_layer("subn", 1024, (256, 128), 5, "mcg", (300,), seed=801)
    t = wl.gen_all(lay)
    x = otf.f32_to_bf16_bits(otf.bf16_bits_to_f32(t.x[:M]) * np.float32(2.0 ** -15))
    want_rot = otf.rotate_input(x, t.suh, "bf16")
    frac = np.mean((want_rot & 0x7C00) == 0)
    assert frac > 0.5, f"only {frac:.2f} of x~ subnormal or zero"
    xr, y = _run(weight(t), x)
    assert np.array_equal(xr, rot_layout(want_rot))
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, x)
    res = olin.check(y, ref, t.svh, lay.K, "bf16")
    banner(f"subnormal x~ M={M} ({frac:.2f} subnormal): {res}")
    assert res.ok, str(res)


def test_rotated_activations_near_fp16_max():
    """Rows aligned with Hadamard rows: x~ reaches 2**15 = 32768, within a
    factor of two of 65504; the rotation is exact and the linear (fp32 sums)
    within the bound."""
    lay = wl.small_layer("big", 512, (256,), 6, "mul1", (8,), seed=802)
    t = wl.gen_all(lay)
    h = otf.sylvester()
    x = np.zeros((8, 512), np.float32)
    for r in range(8):
        x[r] = np.tile(h[r * 7 % 128] * 4096.0, 4)  # x~[r, 128b + r'] = 2**-4 * 128 * 4096 = 32768
    suh = np.full((1, 512), 0x3C00, np.uint16)
    xb = otf.f32_to_bf16_bits(x)
    tw = wl.Tensors(lay, t.trellis, suh, t.svh, xb)
    want_rot = otf.rotate_input(xb, suh, "bf16")
    assert np.max(np.abs(otf.f16_from_bits(want_rot).astype(np.float64))) == 32768.0
    xr, y = _run(weight(tw), xb)
    assert np.array_equal(xr, rot_layout(want_rot))
    ref = olin.reference(t.trellis, suh, t.svh, lay.shards, lay.bits, lay.cb, xb)
    res = olin.check(y, ref, t.svh, lay.K, "bf16")
    banner(f"x~ near fp16 max: {res}")
    assert res.ok, str(res)


@pytest.mark.parametrize("M,force", [(6, {}), (6, {"decoder": ex.EXL3_DECODER_TABLE}), (70, {}), (70, {"bm": 128}),
                                     (300, {}), (300, {"decoder": ex.EXL3_DECODER_DENSE})])
def test_non_finite_inputs_propagate(M, force):
    lay = wl.small_layer("nonfinite", 1024, (256, 128), 4, "3inst", (300,), seed=803)
    t = wl.gen_all(lay)
    w = weight(t)
    x = t.x[:M].copy()
    bad = {1: 0x7FC0, 3: 0x7F80, 4: 0xFF80}  # bf16 NaN, +inf, -inf
    for r, v in bad.items():
        x[r, 37 * r + 5] = v
    _, y = _run(w, x, **force)
    _, y_clean = _run(w, t.x[:M], **force)
    yf = otf.bf16_bits_to_f32(y)
    for r in bad:
        assert not np.any(np.isfinite(yf[r])), f"row {r} has finite outputs"
    good = [r for r in range(M) if r not in bad]
    assert np.array_equal(y[good], y_clean[good])
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[:M][good])
    res = olin.check(y[good], ref, t.svh, lay.K, "bf16")
    assert res.ok, str(res)


@pytest.mark.parametrize("M", [3, 130])
def test_sixteen_shards(M):
    shards = tuple([128] * 12 + [256, 128, 384, 128])
    lay = wl.small_layer("s16", 512, shards, 3, "mul1", (130,), seed=804)
    assert lay.n_shards == ex.MAX_SHARDS
    t = wl.gen_all(lay, magnitudes=True)
    w = weight(t)
    _, y = _run(w, t.x[:M])
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[:M])
    res = olin.check(y, ref, t.svh, lay.K, "bf16")
    banner(f"16 shards M={M}: {res}")
    assert res.ok, str(res)
    pl = ex.plan(w, M)
    c0 = 0
    for s, n in enumerate(shards):
        ws = ex.Exl3Weight(dev16(np.ascontiguousarray(t.trellis[:, c0 // 16:(c0 + n) // 16])),
                           dev16(np.ascontiguousarray(t.suh[s:s + 1]), torch.float16),
                           dev16(np.ascontiguousarray(t.svh[c0:c0 + n]), torch.float16), lay.bits, lay.codebook, (n,))
        _, ys = _run(ws, t.x[:M], parts=pl["parts"], groups=pl["groups"])
        assert np.array_equal(ys, y[:, c0:c0 + n]), f"shard {s}"
        c0 += n
