"""GPU: the fused activation and the bias.

SwiGLU folded into the down projection's input transform (cuda-exl3 README,
"MoE throughput"; reading R17): against float64 silu(g) * u (the act within
one output ulp, the rotated act within a bound derived from the rounding
steps), and bit-exact against the oracle's fp32 act followed by its rotation
(which checks reading R17's fixed exp sequence).  The layer's bias (README "VRAM"; reading R16): bit-exact in
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


def _silu_times_u_f64(gu_bits, dtype):
    K = gu_bits.shape[1] // 2
    to64 = (lambda b: otf.bf16_bits_to_f32(b).astype(np.float64)) if dtype == "bf16" else \
        (lambda b: otf.f16_from_bits(b).astype(np.float64))
    g, u = to64(gu_bits[:, :K]), to64(gu_bits[:, K:])
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u, u


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_swiglu_act_against_float64(dtype):
    """The fused transform's act against float64 silu(g) * u, within one
    output ulp.  One nonzero u per 128-block makes the block's rotation
    exact (every entry is +-act * suh * 2**-4, a dtype value times a power
    of two, representable in fp16 in the range used), so the kernel's act is
    read back from x~.  Gates span the saturating ends (the exp argument is
    clamped at +-104)."""
    rng = np.random.default_rng(620)
    M, K = 64, 512
    nblk = K // 128
    gmax = 90.0 if dtype == "bf16" else 10.0
    g = rng.uniform(-gmax, gmax, (M, K)).astype(np.float32)
    g[:, :6] = [0.0, -0.0, gmax, -gmax, 1e-3, -1e-3]
    rnd = otf.f32_to_bf16_bits if dtype == "bf16" else otf.f32_to_f16_bits
    to64 = (lambda b: otf.bf16_bits_to_f32(b).astype(np.float64)) if dtype == "bf16" else \
        (lambda b: otf.f16_from_bits(b).astype(np.float64))
    gb = rnd(g)
    g64 = to64(gb)
    silu = g64 / (1.0 + np.exp(-g64))
    pos = rng.integers(0, 128, (M, nblk))
    u = np.zeros((M, K), np.float32)
    for b in range(nblk):
        j = 128 * b + pos[:, b]
        target = np.exp2(rng.uniform(-4, 6, M)) * np.where(rng.integers(0, 2, M) == 1, -1.0, 1.0)
        s = silu[np.arange(M), j]
        umax = 1e38 if dtype == "bf16" else 6e4
        u[np.arange(M), j] = np.clip(np.where(s != 0, target / np.where(s != 0, s, 1.0), 1.0), -umax, umax)
    gu = np.concatenate([gb, rnd(u)], axis=1)
    suh = np.full((1, K), 0x3C00, np.uint16)
    got = bits16(ex.input_transform_swiglu(x_dev(gu, dtype), dev16(suh, torch.float16)))
    xr = got.reshape(1, K // 32, M, 32).transpose(0, 2, 1, 3).reshape(M, K // 32, 32)
    exact, _ = _silu_times_u_f64(gu, dtype)
    for b in range(nblk):
        j = 128 * b + pos[:, b]
        # stored position 0 of the block's first k-step is natural k = 128b
        act_gpu = 16.0 * otf.f16_from_bits(xr[:, 4 * b, 0]).astype(np.float64)
        want = exact[np.arange(M), j]
        mant, emin = (7, -126) if dtype == "bf16" else (10, -14)
        e = np.maximum(np.floor(np.log2(np.maximum(np.abs(want), 1e-300))), emin)
        ulp = np.exp2(e - mant)
        err = np.abs(act_gpu - want)
        assert np.all(err <= ulp), f"block {b}: worst {np.max(err / ulp):.2f} ulp"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_swiglu_transform_within_float64_bound(dtype):
    """The fused transform on general inputs against float64: x~* = 2**-4 *
    H128(silu(g) * u * suh), exact.  Bound per element: the act carries at
    most u_d + 2**-20 relative error (the dtype's rounding, and a few fp32
    roundings in exp, the add, the divide and the product) plus an absolute
    a_d + 2**-120 |u| (the dtype's subnormal half-spacing; silu underflows to
    zero below g = -88.7, where |silu| < 2**-121); the fp32 butterfly adds
    g_7 of the block's sum of |act * suh|; the fp16 rounding adds u_16 |x~*|
    and 2**-25."""
    rng = np.random.default_rng(630)
    M, K, S = 33, 1024, 2
    f = (rng.standard_normal((M, 2 * K)) * np.exp2(rng.uniform(-8, 6, (M, 2 * K)))).astype(np.float32)
    f[:, :8] = [0.0, -0.0, 40.0, -40.0, 95.0, -95.0, 1e-3, -1e-3]
    if dtype == "f16":
        f = np.clip(f, -60000, 60000)
    rnd = otf.f32_to_bf16_bits if dtype == "bf16" else otf.f32_to_f16_bits
    gu = rnd(f)
    suh = (np.where(rng.integers(0, 2, (S, K)) == 1, -1.0, 1.0) * np.exp2(rng.uniform(-2, 2, (S, K)))
           ).astype(np.float16).view(np.uint16)
    got = bits16(ex.input_transform_swiglu(x_dev(gu, dtype), dev16(suh, torch.float16)))
    got = got.reshape(S, K // 32, M, 32).transpose(0, 2, 1, 3)  # [S, M, K/32, 32] stored order
    perm = np.array([0, 2, 1, 3, 4, 6, 5, 7])
    nat = got.reshape(S, M, K // 32, 8, 4)[..., np.argsort(perm), :].reshape(S, M, K)
    act64, u64 = _silu_times_u_f64(gu, dtype)
    u_d = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    a_d = 2.0 ** -134 if dtype == "bf16" else 2.0 ** -25
    g7 = olin.gamma(7, 2.0 ** -24)
    for s in range(S):
        sv = otf.f16_from_bits(suh[s]).astype(np.float64)
        t = act64 * sv
        xstar = otf.butterfly(t) * 2.0 ** -4
        e_act = ((u_d + 2.0 ** -20) * np.abs(act64) + a_d + 2.0 ** -120 * np.abs(u64)) * np.abs(sv)
        blk = lambda a: np.repeat(a.reshape(M, K // 128, 128).sum(axis=-1), 128, axis=1)
        b = (1 + 2.0 ** -11) * 2.0 ** -4 * (blk(e_act) + g7 * blk(np.abs(t) + e_act)) \
            + 2.0 ** -11 * np.abs(xstar) + 2.0 ** -25
        x = otf.f16_from_bits(nat[s]).astype(np.float64)
        r = np.abs(x - xstar) / b
        assert np.all(np.isfinite(x)) and np.max(r) <= 1.0, f"shard {s}: {np.max(r):.3f} of the bound"


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
    ystar, bnd = olin.output_stage_reference(z, svh, out_dtype, bias)
    ratio = np.max(np.abs(olin.out_bits_to_f64(got, out_dtype) - ystar) / bnd)
    assert ratio <= 1.0, f"output stage with bias {ratio:.3f} of the fp64 bound"
    want = otf.output_transform_f32(otf.reduce_parts_f32(z, G), svh, out_dtype, bias)  # reading R15's order
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
    scheds += [dict(tree, bm=512, mode=ex.EXL3_MODE_SLABS, unit=1),
               dict(tree, bm=16, mode=ex.EXL3_MODE_SLABS, wg_cols=64, unit=1),
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
    # one part: the output stage inside every tile kernel (fused), fp16 out
    one = {b: bits16(ex.linear(w, xr, torch.float16, parts=1, mode=ex.EXL3_MODE_FUSED, bm=b))
           for b in (16, 64, 128, 256, 512)}
    for b, y in one.items():
        assert np.array_equal(y, one[16]), f"one part, bm={b}"
    res1 = olin.check(one[16], ref, t.svh, lay.K, "f16")
    banner(f"bias M={M} one part, fp16 out: {res1}")
    assert res1.ok, str(res1)
