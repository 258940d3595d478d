"""GPU: the fused activation and the bias.

SwiGLU folded into the down projection's input transform (cuda-exl3 README,
"MoE throughput"; reading R17): bit-exact against the oracle's act followed
by its rotation.  The layer's bias (README "VRAM"; reading R16): bit-exact in
the output stage given z, the same bits from every kernel family, and within
the oracle's bound for the whole linear."""
import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from oracle import linear as olin
from oracle import transform as otf
from gpu_util import banner, bits16, dev16, rot_layout, slab_layout, weight, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ex.load()
    torch.cuda.init()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,K,S", [(1, 128, 1), (7, 384, 2), (130, 1024, 1), (517, 4096, 2), (3, 640, 2)])
def test_swiglu_transform_bit_exact(dtype, M, K, S):
    banner(f"swiglu transform {dtype} M={M} K={K} S={S}")
    rng = np.random.default_rng(600 + M + K + S)
    f = (rng.standard_normal((M, 2 * K)) * np.exp2(rng.uniform(-8, 6, (M, 2 * K)))).astype(np.float32)
    f[:, :8] = [0.0, -0.0, 40.0, -40.0, 90.0, -90.0, 1e-3, -1e-3]  # saturating and tiny gates
    gu = otf.f32_to_bf16_bits(f) if dtype == "bf16" else otf.f32_to_f16_bits(f)
    suh = (np.where(rng.integers(0, 2, (S, K)) == 1, -1.0, 1.0) * np.exp2(rng.uniform(-2, 2, (S, K)))
           ).astype(np.float16).view(np.uint16)
    got = bits16(ex.input_transform_swiglu(x_dev(gu, dtype), dev16(suh, torch.float16)))
    want = rot_layout(otf.rotate_input(otf.swiglu_bits(gu, dtype), suh, dtype))
    assert got.shape == want.shape
    bad = np.argwhere(got != want)
    assert bad.shape[0] == 0, f"{bad.shape[0]} values differ, first {bad[:4].tolist()}"


def _bias(N, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(N) * 2).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_bias_output_stage_bit_exact(out_dtype):
    P, G, M, N = 8, 2, 9, 256
    rng = np.random.default_rng(610)
    z = (rng.standard_normal((P, M, N)) * np.exp2(rng.integers(-6, 6, (P, M, N)))).astype(np.float32)
    svh = (np.where(rng.integers(0, 2, N) == 1, -1.0, 1.0) * np.exp2(rng.uniform(-2, 2, N))
           ).astype(np.float16).view(np.uint16)
    bias = _bias(N, 611)
    trellis = np.zeros((8, N // 16, 64), dtype=np.uint16)
    suh = np.full((1, 128), 0x3C00, dtype=np.uint16)
    w = ex.Exl3Weight(dev16(trellis), dev16(suh, torch.float16), dev16(svh, torch.float16), 4, "mcg", (N,),
                      bias=dev16(bias, torch.float16))
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float16
    got = bits16(ex.debug_epilogue(w, torch.from_numpy(slab_layout(z)).cuda(), M, dt, groups=G))
    want = otf.output_transform_f32(otf.reduce_parts_f32(z, G), svh, out_dtype, bias)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [5, 40, 300])
def test_bias_every_kernel_family(M):
    """Tile kernels (16-64 rows, with and without the finishing workgroup,
    half-width workgroups), 128/256/512-row kernels, table and dense
    decoders: one set of bits with a bias, equal to the output stage applied
    to the GEMM stage's parts, and within the oracle's bound."""
    lay = wl.small_layer("bias", 1024, (256, 384), 5, "mul1", (300,), seed=612)
    t = wl.gen_all(lay)
    bias = _bias(lay.N, 613)
    w = ex.Exl3Weight(dev16(t.trellis), dev16(t.suh, torch.float16), dev16(t.svh, torch.float16), lay.bits,
                      lay.codebook, lay.shards, bias=dev16(bias, torch.float16))
    xr = ex.input_transform(x_dev(t.x[:M]), w.suh)
    outs = {"auto": bits16(ex.linear(w, xr, torch.bfloat16))}
    pl = ex.plan(w, M)
    tree = dict(parts=pl["parts"], groups=pl["groups"])
    scheds = [dict(tree, bm=b, mode=ex.EXL3_MODE_SLABS) for b in (16, 64, 128, 256)]
    scheds += [dict(tree, bm=16, mode=ex.EXL3_MODE_SLABS, wg_cols=64, unit=1),
               dict(tree, decoder=ex.EXL3_DECODER_DENSE, mode=ex.EXL3_MODE_SLABS)]
    if M <= 64:
        scheds.append(dict(tree, decoder=ex.EXL3_DECODER_TABLE))
    for f in scheds:
        outs[str(f)] = bits16(ex.linear(w, xr, torch.bfloat16, **f))
    first = outs["auto"]
    for k, y in outs.items():
        assert np.array_equal(y, first), f"schedule {k}"
    z = ex.debug_parts(w, xr)
    assert np.array_equal(bits16(ex.debug_epilogue(w, z, M, groups=pl["groups"])), first)
    assert len(outs) >= 7
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[:M], "bf16", bias_bits=bias)
    res = olin.check(first, ref, t.svh, lay.K, "bf16")
    banner(f"bias M={M} ({len(outs)} schedules): {res}")
    assert res.ok, str(res)
