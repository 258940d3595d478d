"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact where the format fixes every rounding (codebooks, unpacking, the
input rotation, the output stage given z); within the rounding-order bound of
the oracle (and worst-column relative error <= 5e-3) for the whole linear,
whose fp32 sums run inside the matrix unit in an order the pages leave open.
"""
import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from oracle import format as ofmt
from oracle import linear as olin
from oracle import transform as otf
from gpu_util import banner, bits16, dev16, rot_layout, slab_layout, weight, x_dev

pytestmark = pytest.mark.gpu

CB_NAMES = ("3inst", "mcg", "mul1")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ex.load()
    torch.cuda.init()


# ------------------------------------------------------------ bit-exact parts

@pytest.mark.parametrize("cb", CB_NAMES)
def test_codebook_every_state(cb):
    banner(f"codebook {cb}")
    got = bits16(ex.debug_codebook(cb))
    want = ofmt.codebook_table(wl.CB_ID[cb])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} states differ, first {bad[:5]}: {got[bad[:5]]} vs {want[bad[:5]]}"


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("cb", CB_NAMES)
def test_decode_every_width_and_codebook(bits, cb):
    banner(f"decode bits={bits} cb={cb}")
    lay = wl.small_layer(f"dec_b{bits}_{cb}", 256, (384,), bits, cb, (1,), seed=40 + bits)
    t = wl.gen_all(lay)
    got = bits16(ex.debug_decode(weight(t)))
    want = ofmt.dequantize_bits(t.trellis, bits, lay.cb)
    bad = np.argwhere(got != want)
    assert bad.shape[0] == 0, f"{bad.shape[0]} weights differ, first (k, n) {bad[:4].tolist()}"


@pytest.mark.parametrize("x_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,K,S", [(1, 128, 1), (7, 384, 3), (33, 1024, 2), (130, 256, 1), (517, 4096, 2), (3, 640, 2), (2, 4096, 1)])
def test_input_transform_bit_exact(x_dtype, M, K, S):
    banner(f"input transform {x_dtype} M={M} K={K} S={S}")
    rng = np.random.default_rng(1000 + M + K + S)
    xf = rng.standard_normal((M, K)).astype(np.float32) * 3
    x = otf.f32_to_bf16_bits(xf) if x_dtype == "bf16" else otf.f32_to_f16_bits(xf)
    suh = (np.where(rng.integers(0, 2, (S, K)) == 1, -1.0, 1.0) * np.exp2(rng.uniform(-2, 2, (S, K)))
           ).astype(np.float16).view(np.uint16)
    got = bits16(ex.input_transform(x_dev(x, x_dtype), dev16(suh, torch.float16)))
    want = rot_layout(otf.rotate_input(x, suh, x_dtype))
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_input_transform_one_hot_closed_form():
    import scipy.linalg
    h = scipy.linalg.hadamard(128)
    x = np.zeros((128, 128), dtype=np.uint16)
    x[np.arange(128), np.arange(128)] = 0x3F80  # row j = e_j (bf16 1.0)
    suh = np.full((1, 128), 0x3C00, dtype=np.uint16)
    got = bits16(ex.input_transform(x_dev(x), dev16(suh, torch.float16)))
    want = np.where(h.T > 0, 0x2C00, 0xAC00).astype(np.uint16)  # row j = signs of column j
    assert np.array_equal(got, rot_layout(want[None]))


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("P,G,M,N", [(1, 1, 3, 128), (3, 3, 17, 384), (8, 8, 64, 256), (8, 2, 9, 256),
                                     (12, 3, 5, 128), (16, 16, 7, 128), (17, 17, 1, 256), (20, 4, 64, 128),
                                     (24, 8, 65, 128), (17, 17, 300, 128), (10, 5, 129, 256)])
def test_output_stage_bit_exact(out_dtype, P, G, M, N):
    banner(f"epilogue {out_dtype} P={P} G={G} M={M} N={N}")
    rng = np.random.default_rng(2000 + P + M + N)
    z = (rng.standard_normal((P, M, N)) * np.exp2(rng.integers(-6, 6, (P, M, N)))).astype(np.float32)
    svh = (np.where(rng.integers(0, 2, N) == 1, -1.0, 1.0) * np.exp2(rng.uniform(-2, 2, N))
           ).astype(np.float16).view(np.uint16)
    lay = wl.small_layer("ep", 128, (N,), 4, "mcg")
    trellis = np.zeros((8, N // 16, 64), dtype=np.uint16)
    suh = np.full((1, 128), 0x3C00, dtype=np.uint16)
    w = ex.Exl3Weight(dev16(trellis), dev16(suh, torch.float16), dev16(svh, torch.float16), 4, "mcg", (N,))
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float16
    got = bits16(ex.debug_epilogue(w, torch.from_numpy(slab_layout(z)).cuda(), M, dt, groups=G))
    # against the plain definition: the fp64 sum of the parts through the
    # exact output transform, within the bound of any fp32 fold of P terms
    ystar, bnd = olin.output_stage_reference(z, svh, out_dtype)
    ratio = np.max(np.abs(olin.out_bits_to_f64(got, out_dtype) - ystar) / bnd)
    assert ratio <= 1.0, f"output stage {ratio:.3f} of the fp64 bound"
    # and bit for bit the library's fold order (reading R15: parts of a group
    # in order, then the groups in order)
    want = otf.output_transform_f32(otf.reduce_parts_f32(z, G), svh, out_dtype)
    assert np.array_equal(got, want)
    del lay


# ------------------------------------------------------- the whole linear

def _run(t, out_dtype="bf16", M=None, x_dtype="bf16", **force):
    x = t.x if M is None else t.x[:M]
    w = weight(t)
    xr = ex.input_transform(x_dev(x, x_dtype), w.suh)
    y = ex.linear(w, xr, torch.bfloat16 if out_dtype == "bf16" else torch.float16, **force)
    torch.cuda.synchronize()
    return bits16(y)


def _check(t, y, out_dtype="bf16", M=None, x_dtype="bf16"):
    lay = t.layer
    x = t.x if M is None else t.x[:M]
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, x, x_dtype)
    res = olin.check(y, ref, t.svh, lay.K, out_dtype)
    banner(f"{lay.name} M={x.shape[0]} {out_dtype}: {res}")
    assert res.ok, str(res)
    return res


SMALL = [wl.small_layer(f"lin_b{b}_{cb}", 256, (256,), b, cb, (5,), seed=60 + b) for b in range(1, 9)
         for cb in CB_NAMES]


@pytest.mark.parametrize("lay", SMALL, ids=lambda l: l.name)
def test_linear_every_width_and_codebook(lay):
    t = wl.gen_all(lay)
    _check(t, _run(t))


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("magnitudes", [False, True])
def test_linear_two_shards(out_dtype, magnitudes):
    lay = wl.small_layer("two_shards", 384, (128, 256), 6, "mul1", (33,), seed=7)
    t = wl.gen_all(lay, magnitudes=magnitudes)
    _check(t, _run(t, out_dtype), out_dtype)


def test_linear_fp16_activations():
    lay = wl.small_layer("f16x", 512, (256,), 5, "mcg", (9,), seed=8)
    t = wl.gen_all(lay)
    rng = np.random.default_rng(9)
    t.x = otf.f32_to_f16_bits(rng.standard_normal((9, 512)).astype(np.float32))
    _check(t, _run(t, x_dtype="f16"), x_dtype="f16")


@pytest.mark.parametrize("M", [1, 7, 16, 17, 33, 64, 65, 130, 257, 300])
def test_linear_ragged_rows(M):
    lay = wl.small_layer("ragged", 1024, (256,), 4, "3inst", (300,), seed=10)
    t = wl.gen_all(lay)
    _check(t, _run(t, M=M), M=M)


@pytest.mark.parametrize("parts", [1, 2, 4, 8])
def test_schedules_agree_bit_for_bit(parts):
    """mode and rows-per-tile never change a bit; every part count is in bound."""
    lay = wl.small_layer("sched", 1024, (128, 256), 6, "mul1", (70,), seed=11)
    t = wl.gen_all(lay)
    outs = {}
    for mode in (ex.EXL3_MODE_FUSED, ex.EXL3_MODE_SLABS):
        for bm in (16, 32, 64, 128, 256, 512):
            if bm == 512 and mode == ex.EXL3_MODE_FUSED and parts > 1:
                continue  # one accumulator set per 512-row workgroup
            outs[(mode, bm)] = _run(t, parts=parts, mode=mode, bm=bm)
            if mode == ex.EXL3_MODE_SLABS and parts > 1 and bm <= 64:
                outs[(mode, bm, 64)] = _run(t, parts=parts, mode=mode, bm=bm, wg_cols=64)
    first = next(iter(outs.values()))
    for key, y in outs.items():
        assert np.array_equal(y, first), f"schedule {key} differs"
    _check(t, first)


@pytest.mark.parametrize("bits,cb", [(6, "mul1"), (5, "3inst"), (8, "mcg"), (3, "mul1"), (1, "mcg"), (2, "3inst"),
                                     (4, "mul1"), (7, "mcg")])
@pytest.mark.parametrize("M", [300, 600])
def test_large_tiles_ragged(bits, cb, M):
    """The 128-, 256- and 512-row tiles on a ragged last tile: bit-identical
    to the 64-row tile, for one part and for slabs of two parts."""
    banner(f"large tiles {bits}-bit {cb} M={M}")
    lay = wl.small_layer("tall", 1024, (256,), bits, cb, (M,), seed=30 + bits)
    t = wl.gen_all(lay)
    for parts, mode in ((1, ex.EXL3_MODE_FUSED), (2, ex.EXL3_MODE_SLABS)):
        ref = _run(t, parts=parts, mode=mode, bm=64)
        for bm in (128, 256, 512):
            assert np.array_equal(_run(t, parts=parts, mode=mode, bm=bm), ref), f"bm={bm} parts={parts}"
    _check(t, ref)


TABLE_CASES = [(1, "3inst"), (2, "mul1"), (3, "mcg"), (4, "mcg"), (5, "mul1"), (6, "mul1"), (7, "3inst"),
               (8, "mul1")]


@pytest.mark.parametrize("bits,cb", TABLE_CASES)
@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 33, 64])
def test_table_decoder_matches_alu(bits, cb, M):
    """The table decoder against the ALU tile kernel: the same bits for one
    part, a fused multi-part fold, and slabs; two shards, ragged rows."""
    banner(f"table decoder {bits}-bit {cb} M={M}")
    lay = wl.small_layer(f"table_b{bits}_{cb}", 1024, (256, 384), bits, cb, (64,), seed=80 + bits)
    t = wl.gen_all(lay)
    y = None
    for parts, mode in ((1, ex.EXL3_MODE_FUSED), (2, ex.EXL3_MODE_FUSED), (4, ex.EXL3_MODE_SLABS),
                        (8, ex.EXL3_MODE_SLABS)):
        ref = _run(t, M=M, parts=parts, mode=mode, decoder=ex.EXL3_DECODER_ALU)
        y = _run(t, M=M, parts=parts, mode=mode, decoder=ex.EXL3_DECODER_TABLE)
        assert np.array_equal(y, ref), f"parts={parts} mode={mode}"
    _check(t, y, M=M)


@pytest.mark.parametrize("mode", [ex.EXL3_MODE_FUSED, ex.EXL3_MODE_SLABS])
def test_table_decoder_several_units_per_team(mode):
    """Slabs: 2048 units, more than the 4 teams of every CU, so each team
    streams two units back to back.  Fused: 8 parts folded per column block
    at K = 8192.  Both give the ALU kernel's bits; fp16 output."""
    banner(f"table decoder, many units, mode {mode}")
    lay = wl.small_layer("table_units", 8192, (4096,), 4, "mcg", (3,), seed=91)
    t = wl.gen_all(lay)
    parts = 64 if mode == ex.EXL3_MODE_SLABS else 8
    ref = _run(t, "f16", parts=parts, mode=mode, decoder=ex.EXL3_DECODER_ALU)
    y = _run(t, "f16", parts=parts, mode=mode, decoder=ex.EXL3_DECODER_TABLE)
    assert np.array_equal(y, ref)


DENSE_CASES = [(1, "mul1"), (2, "3inst"), (3, "mcg"), (4, "mcg"), (5, "mul1"), (6, "mul1"), (7, "3inst"), (8, "mcg")]


@pytest.mark.parametrize("bits,cb", DENSE_CASES)
@pytest.mark.parametrize("M", [1, 17, 256, 300, 600])
def test_dense_decoder_matches_alu(bits, cb, M):
    """Dequantize-then-GEMM against the ALU tile kernel: the same bits for
    one part, a register fold of 2 and of 3 unequal parts, one slab per part
    and grouped slabs; two shards, ragged rows past a 256-row tile."""
    banner(f"dense decoder {bits}-bit {cb} M={M}")
    lay = wl.small_layer(f"dense_b{bits}_{cb}", 1024, (256, 384), bits, cb, (600,), seed=120 + bits)
    t = wl.gen_all(lay)
    y = None
    for force in (dict(parts=1), dict(parts=2, mode=ex.EXL3_MODE_FUSED), dict(parts=3, mode=ex.EXL3_MODE_FUSED),
                  dict(parts=4, mode=ex.EXL3_MODE_SLABS), dict(parts=8, groups=2, mode=ex.EXL3_MODE_SLABS)):
        ref = _run(t, M=M, decoder=ex.EXL3_DECODER_ALU, **force)
        y = _run(t, M=M, decoder=ex.EXL3_DECODER_DENSE, **force)
        assert np.array_equal(y, ref), f"{force}"
    if M <= 300:
        _check(t, y, M=M)


# 288 column tiles of 256 x 256 with one 256-row tile: one round plus 32
# tiles on 256 CUs; odd_shards: 151 + 138 tiles (the first shard ends in a
# one-block tile), 33 past the round, the split inside the second shard
@pytest.mark.parametrize("shards", [(73728,), (128 * 301, 128 * 275)], ids=["one_shard", "odd_shards"])
def test_dense_split_last_round(shards):
    """The dense GEMM's 256 x 256 launch over whole rounds of the CUs and its
    256 x 128 launch over the column blocks after it: together the bits of
    the ALU decoder and within the oracle's bound; run apart through the
    hook, each writes exactly its own columns."""
    M = 200
    lay = wl.small_layer("dense_split", 256, shards, 4, "mcg", (M,), seed=140)
    t = wl.gen_all(lay)
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x[:M]), w.suh)
    nblk = w.N // 128
    pl = ex.plan(w, M, decoder=ex.EXL3_DECODER_DENSE)
    y_alu = bits16(ex.linear(w, xr, torch.bfloat16, decoder=ex.EXL3_DECODER_ALU))
    y_dense = bits16(ex.linear(w, xr, torch.bfloat16, decoder=ex.EXL3_DECODER_DENSE))
    assert np.array_equal(y_dense, y_alu)
    frags = ex.debug_dequant(w)
    fill = torch.full((M, w.N), -3.0, dtype=torch.bfloat16, device="cuda")
    mark = bits16(fill)[0, 0]
    y1, bulk = ex.debug_dense_gemm(w, frags, xr, which=1, out=fill.clone())
    y2, bulk2 = ex.debug_dense_gemm(w, frags, xr, which=2, out=fill.clone())
    y3, _ = ex.debug_dense_gemm(w, frags, xr, which=3)
    torch.cuda.synchronize()
    banner(f"dense split {shards}: {bulk} of {nblk} column blocks in 256 x 256 tiles, plan {pl}")
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert bulk == (512 if len(shards) == 1 else 511) and pl["launches"] == 3
    assert bulk == bulk2 and 0 < bulk <= nblk
    c = 128 * bulk
    b1, b2 = bits16(y1), bits16(y2)
    assert np.array_equal(b1[:, :c], y_alu[:, :c]) and (b1[:, c:] == mark).all()
    assert np.array_equal(b2[:, c:], y_alu[:, c:]) and (b2[:, :c] == mark).all()
    assert np.array_equal(bits16(y3), y_alu)
    _check(t, y_dense, M=M)


@pytest.mark.parametrize("decoder", [ex.EXL3_DECODER_ALU, ex.EXL3_DECODER_TABLE])
@pytest.mark.parametrize("parts", [1, 3, 8])
def test_part_sums_stage(decoder, parts):
    """The GEMM stage alone: every K part's fp32 sum within the rounding
    bound of its own length against the fp64 sum over that part's k range
    (3 parts of 8 blocks: 2, 3 and 3 blocks); and the output stage applied
    to those parts is bit for bit the whole linear."""
    banner(f"part sums, decoder {decoder}, {parts} parts")
    lay = wl.small_layer("parts", 1024, (256, 128), 5, "mcg", (13,), seed=95)
    t = wl.gen_all(lay)
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x), w.suh)
    z = ex.debug_parts(w, xr, parts=parts, decoder=decoder)
    torch.cuda.synchronize()
    M, N, K = t.x.shape[0], lay.N, lay.K
    zn = z.cpu().numpy().transpose(0, 1, 3, 2).reshape(parts, -1, N)[:, :M]  # [P, M, N]
    x64 = otf.f16_from_bits(otf.rotate_input(t.x, t.suh, "bf16")).astype(np.float64)  # [S, M, K]
    wq = ofmt.dequantize(t.trellis, lay.bits, lay.cb)  # [K, N]
    col_shard = olin.shard_of_columns(lay.shards)
    kb = K // 128
    for p in range(parts):
        k0, k1 = 128 * (p * kb // parts), 128 * ((p + 1) * kb // parts)
        for s in range(lay.n_shards):
            cols = np.nonzero(col_shard == s)[0]
            exact = x64[s][:, k0:k1] @ wq[k0:k1, cols]
            absd = np.abs(x64[s][:, k0:k1]) @ np.abs(wq[k0:k1, cols])
            err = np.abs(zn[p][:, cols] - exact)
            lim = olin.gamma(k1 - k0, olin.U_ACC) * absd
            assert np.all(err <= lim), f"part {p} shard {s}: worst {np.max(err - lim)} over the bound"
    y = bits16(ex.linear(w, xr, torch.bfloat16, parts=parts, decoder=decoder))
    y2 = bits16(ex.debug_epilogue(w, z, M))
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("M", [5, 40, 100, 300])
def test_grouped_tree_schedules_agree(M):
    """Eight one-block parts in two groups (the small-layer tree): quads of
    waves with the finishing workgroup (16-64 rows), register folds of a
    group (128-256 rows), one slab per part with the two-level output stage,
    and the GEMM stage + output stage hooks all give the same bits, within
    the bound of the oracle."""
    banner(f"grouped tree M={M}")
    lay = wl.small_layer("tree", 1024, (256, 128), 5, "mcg", (M,), seed=97)
    t = wl.gen_all(lay)
    outs = {}
    for bm in (16, 32, 64, 128, 256):
        if bm < M and bm < 64:
            continue
        for unit in (None, 1):
            outs[(bm, unit)] = _run(t, parts=8, groups=2, bm=bm, unit=unit, mode=ex.EXL3_MODE_SLABS)
            if bm <= 64:  # 64- and 128-column workgroups
                for cols in (64, 128):
                    outs[(bm, unit, cols)] = _run(t, parts=8, groups=2, bm=bm, unit=unit, mode=ex.EXL3_MODE_SLABS,
                                                  wg_cols=cols)
    if M <= 16:
        outs["table"] = _run(t, parts=8, groups=2, decoder=ex.EXL3_DECODER_TABLE)
        outs["table, part slabs"] = _run(t, parts=8, groups=2, decoder=ex.EXL3_DECODER_TABLE, unit=1)
    first = next(iter(outs.values()))
    for key, y in outs.items():
        assert np.array_equal(y, first), f"schedule {key} differs"
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x), w.suh)
    z = ex.debug_parts(w, xr, parts=8, groups=2)
    assert np.array_equal(bits16(ex.debug_epilogue(w, z, M, groups=2)), first)
    if M <= 64:
        z64 = ex.debug_parts(w, xr, parts=8, groups=2, bm=64, wg_cols=64)
        assert torch.equal(z64, z)
    zg = ex.debug_parts(w, xr, parts=8, groups=2, unit=4)
    assert np.array_equal(bits16(ex.debug_epilogue(w, zg, M)), first)
    _check(t, first)


@pytest.mark.parametrize("M", [70, 128, 200])
def test_one_part_schedules_agree(M):
    """One part over the whole K, fused (the tree of layers of 256+
    column blocks): 128-row tiles then run the 8-wave kernel with 64-row
    waves; it gives the bits of the 16-, 64- and 256-row tiles and of the
    dense decoder (ragged rows and two row tiles included), within the
    oracle's bound."""
    banner(f"one part M={M}")
    lay = wl.small_layer("onepart", 1024, (384, 256), 6, "mul1", (M,), seed=99)
    t = wl.gen_all(lay)
    outs = {bm: _run(t, parts=1, bm=bm, mode=ex.EXL3_MODE_FUSED) for bm in (16, 64, 128, 256)}
    outs["dense"] = _run(t, parts=1, decoder=ex.EXL3_DECODER_DENSE)
    for key, y in outs.items():
        assert np.array_equal(y, outs[128]), f"schedule {key} differs"
    _check(t, outs[128])


def test_grouped_tree_is_not_the_flat_fold():
    """The grouped tree and the flat fold of the same eight parts are both
    within the bound, and their bits differ somewhere (the tree is real)."""
    lay = wl.small_layer("tree2", 1024, (512,), 4, "mcg", (64,), seed=98)
    t = wl.gen_all(lay)
    flat = _run(t, parts=8)
    tree = _run(t, parts=8, groups=2)
    _check(t, flat)
    _check(t, tree)
    assert not np.array_equal(flat, tree)


def test_finisher_counters_stay_zero():
    """The finishing workgroup resets its tile's counter: after calls of
    several plans on one workspace the counter area is zero again, and a
    call after them gives the same bits as the first."""
    lay = wl.small_layer("fin", 2048, (512,), 4, "mcg", (64,), seed=99)
    t = wl.gen_all(lay)
    w = weight(t)
    assert ex.plan(w, 16)["launches"] == 1 and ex.plan(w, 16)["groups"] < ex.plan(w, 16)["parts"]
    first = _run(t, M=16)
    for M in (1, 7, 33, 64, 16):
        _run(t, M=M)
    torch.cuda.synchronize()
    ws = ex._workspaces[ex.workspace_key()]
    assert int(torch.count_nonzero(ws[:ex.COUNTER_BYTES])) == 0
    assert np.array_equal(_run(t, M=16), first)


def test_row_chunks():
    """4096 x 4096, 4 bits (32 column blocks x 4 groups of 4 parts) at 3200
    rows: the group slabs exceed 192 MiB, so the call runs in row chunks.
    Rows from both chunks equal the same rows computed alone, and sampled
    outputs are within the oracle's bound."""
    lay = wl.small_layer("chunks", 4096, (4096,), 4, "mcg", (3200,), seed=96)
    t = wl.gen_all(lay)
    w = weight(t)
    pl = ex.plan(w, 3200)
    banner(f"row chunks: plan {pl}")
    assert pl["mode"] == ex.EXL3_MODE_SLABS and pl["launches"] > 2
    xr = ex.input_transform(x_dev(t.x), w.suh)
    y = bits16(ex.linear(w, xr, torch.bfloat16))
    rows = [0, 1777, 3199]
    for r in rows:
        xr1 = ex.input_transform(x_dev(t.x[r:r + 1]), w.suh)
        assert np.array_equal(bits16(ex.linear(w, xr1, torch.bfloat16))[0], y[r]), f"row {r}"
    blocks = [0, 17, 31]
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[rows], col_blocks=blocks)
    res = olin.check(y[rows][:, ref.cols], ref, t.svh, lay.K, "bf16")
    banner(f"row chunks sampled: {res}")
    assert res.ok, str(res)


# ---------------------------------------------------------------- invariants

def test_row_alone_equals_row_in_batch():
    """A row's bytes are the same at every batch size (prefix rows)."""
    lay = wl.small_layer("inv", 2048, (512,), 4, "mcg", (96,), seed=12)
    t = wl.gen_all(lay)
    full = _run(t)
    for M in (1, 2, 15, 16, 17, 40, 64, 65, 95):
        part = _run(t, M=M)
        assert np.array_equal(part, full[:M]), f"M={M}"
    # and a single row moved to another position of a batch
    x = t.x.copy()
    x[50] = t.x[3]
    t2 = wl.Tensors(lay, t.trellis, t.suh, t.svh, x)
    assert np.array_equal(_run(t2)[50], full[3])


def test_repeat_runs_identical():
    lay = wl.small_layer("rep", 2048, (256,), 6, "mul1", (20,), seed=13)
    t = wl.gen_all(lay)
    a = _run(t)
    for _ in range(3):
        assert np.array_equal(_run(t), a)


def test_svh_sign_and_zero_columns():
    lay = wl.small_layer("svh", 512, (256,), 3, "3inst", (11,), seed=14)
    t = wl.gen_all(lay, magnitudes=True)
    y = _run(t)
    neg = wl.Tensors(lay, t.trellis, t.suh, t.svh ^ np.uint16(0x8000), t.x)
    assert np.array_equal(_run(neg), y ^ np.uint16(0x8000))
    svh = t.svh.copy()
    svh[[0, 77, 200]] = 0
    zero = wl.Tensors(lay, t.trellis, t.suh, svh, t.x)
    yz = _run(zero)
    assert np.all(yz[:, [0, 77, 200]] & np.uint16(0x7FFF) == 0)


def test_doubling_x_doubles_y():
    lay = wl.small_layer("dbl", 512, (128,), 5, "mul1", (8,), seed=15)
    t = wl.gen_all(lay)
    xr = otf.rotate_input(t.x, t.suh)
    assert np.all((xr & 0x7C00) != 0)  # no fp16 subnormal in x~, so scaling by 2 is exact
    y = _run(t)
    x2 = t.x + np.uint16(0x0080)  # bf16 exponent + 1 (no zeros / subnormals in x)
    assert np.all((t.x & 0x7F80) != 0)
    y2 = _run(wl.Tensors(lay, t.trellis, t.suh, t.svh, x2))
    f = lambda b: otf.bf16_bits_to_f32(b).astype(np.float64)
    assert np.array_equal(f(y2), 2.0 * f(y))


def test_two_shard_call_equals_two_single_calls():
    lay = wl.small_layer("i3", 512, (256, 128), 4, "mcg", (19,), seed=16)
    t = wl.gen_all(lay)
    fused = _run(t, parts=1)
    c0 = 0
    for s, n in enumerate(lay.shards):
        sub = wl.Layer("sub", lay.K, (n,), lay.bits, lay.codebook, lay.M_values, lay.seed_base)
        ts = wl.Tensors(sub, t.trellis[:, c0 // 16:(c0 + n) // 16].copy(), t.suh[s:s + 1].copy(),
                        t.svh[c0:c0 + n].copy(), t.x)
        assert np.array_equal(_run(ts, parts=1), fused[:, c0:c0 + n])
        c0 += n


def test_zero_rows_is_a_noop():
    lay = wl.small_layer("m0", 256, (128,), 2, "mul1", (1,), seed=17)
    t = wl.gen_all(lay)
    w = weight(t)
    xr = torch.empty(ex.rot_shape(1, 0, 256), dtype=torch.float16, device="cuda")
    y = ex.linear(w, xr)
    assert y.shape == (0, 128)


# ------------------------------------------------ measurement rulers

def test_stream_read_ruler_xor():
    """The streaming-read ruler reads every word once: the XOR of its output
    words is the XOR of the buffer (a ragged size: not a multiple of the
    grid's 4-load stride)."""
    rng = np.random.default_rng(301)
    host = rng.integers(0, 2**32, (1 << 20) + 12, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = ex.debug_stream_read(buf)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)


def test_mfma_loop_ruler_closed_form():
    """All-ones operands: every lane's 16 chains hold 32 * iters each."""
    out = ex.debug_mfma_loop(100)
    torch.cuda.synchronize()
    assert torch.all(out == 16 * 32 * 100)
    half = ex.debug_mfma_loop(3, one=0x3800)  # 0.5: 16 * 32 * 3 * 0.25
    assert torch.all(half == 16 * 32 * 3 * 0.25)


def _toggle_operands(tid):
    """The toggling ruler's operands of threads `tid` (its hash, restated):
    -> a, b [n, 2 sets, 8] float64."""
    t = tid.astype(np.uint64)
    a = np.zeros((len(tid), 2, 8))
    b = np.zeros((len(tid), 2, 8))
    m32 = np.uint64(0xFFFFFFFF)
    for s_ in range(2):
        for e in range(8):
            x = (t * np.uint64(0x9E3779B1) + np.uint64((s_ * 8 + e) * 0x85EBCA6B)) & m32
            x ^= x >> np.uint64(15)
            x = (x * np.uint64(0x2C1B3C6D)) & m32
            x ^= x >> np.uint64(12)
            a[:, s_, e] = ((x & np.uint64(0x83FF)) | np.uint64(0x3800)).astype(np.uint16).view(np.float16)
            b[:, s_, e] = (((x >> np.uint64(16)) & np.uint64(0x83FF)) | np.uint64(0x3800)).astype(np.uint16).view(
                np.float16)
    return a, b


def test_mfma_toggle_ruler_computes_its_products():
    """one = 0: two sets of hashed operands alternate.  Lane l of a wave
    holds A row l % 16 and B column l % 16 at k = 8 (l / 16) .. +7; its first
    accumulator element is C[4 (l / 16)][l % 16], so out = 8 iters (C_0 +
    C_1) at that position, against float64 within the fp32 accumulation's
    rounding (checked on the first 64 waves)."""
    iters = 5
    out = ex.debug_mfma_loop(iters, one=0).cpu().numpy()
    assert np.all(np.isfinite(out)) and np.all(np.abs(out) <= 512 * iters)
    want = np.zeros(64 * 64)
    for w in range(64):
        tid = np.arange(64 * w, 64 * w + 64)
        a, b = _toggle_operands(tid)
        for s_ in range(2):
            A = np.zeros((16, 32))
            B = np.zeros((32, 16))
            for l in range(64):
                A[l % 16, 8 * (l // 16):8 * (l // 16) + 8] = a[l, s_]
                B[8 * (l // 16):8 * (l // 16) + 8, l % 16] = b[l, s_]
            C = A @ B
            for l in range(64):
                want[64 * w + l] += 8 * iters * C[4 * (l // 16), l % 16]
    got = out[:64 * 64].astype(np.float64)
    assert np.allclose(got, want, rtol=1e-5, atol=1e-3), np.max(np.abs(got - want))


@pytest.mark.parametrize("bits,cb", [(2, "mul1"), (5, "3inst"), (7, "mcg")])
def test_dequant_fragments_layout(bits, cb):
    """The dense decoder's fragments are the oracle's W_q in the documented
    B-fragment order: [K/32][N/128][f = 2w + h][lane 16g + j][8] holds
    W_q[32ks + k][128nb + 16(2w + j/8) + j%8 + 8h] at the 8 k of piece g
    (4-element chunks c(2g), c(2g+1) of 0, 2, 1, 3, 4, 6, 5, 7)."""
    lay = wl.small_layer(f"dq_b{bits}_{cb}", 256, (384,), bits, cb, (1,), seed=330 + bits)
    t = wl.gen_all(lay)
    got = bits16(ex.debug_dequant(weight(t)))  # [K/32, N/128, 8, 64, 8]
    wq = ofmt.dequantize_bits(t.trellis, bits, lay.cb)  # [K, N]
    K, N = wq.shape
    chunk = np.array([0, 2, 1, 3, 4, 6, 5, 7])
    want = np.zeros_like(got)
    for f in range(8):
        w_, h = f // 2, f % 2
        for lane in range(64):
            g, j = lane // 16, lane % 16
            c = 16 * (2 * w_ + j // 8) + j % 8 + 8 * h
            ks = np.concatenate([4 * chunk[2 * g] + np.arange(4), 4 * chunk[2 * g + 1] + np.arange(4)])
            for kt in range(K // 32):
                for nb in range(N // 128):
                    want[kt, nb, f, lane] = wq[32 * kt + ks, 128 * nb + c]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bits,cb", [(1, "3inst"), (4, "mcg"), (6, "mul1"), (8, "3inst")])
def test_decode_rate_ruler_block_xor(bits, cb):
    """The decode ruler decodes every weight of every block: its block words
    are the XORs of the oracle's fp16 W_q bits at even (low half) and odd
    (high half) k of each 128 x 128 block."""
    lay = wl.small_layer(f"ruler_b{bits}_{cb}", 384, (256, 128), bits, cb, (1,), seed=310 + bits)
    t = wl.gen_all(lay)
    got = ex.debug_decode_rate(weight(t)).cpu().numpy().view(np.uint32)
    wq = ofmt.dequantize_bits(t.trellis, bits, lay.cb).astype(np.uint32)  # [K, N] fp16 bits
    blk = wq.reshape(lay.K // 128, 128, lay.N // 128, 128)
    lo = np.bitwise_xor.reduce(np.bitwise_xor.reduce(blk[:, 0::2], axis=1), axis=2)
    hi = np.bitwise_xor.reduce(np.bitwise_xor.reduce(blk[:, 1::2], axis=1), axis=2)
    assert np.array_equal(got, lo | (hi << 16))


# --------------------------------------------- full-size workloads, sampled

# Every (layer, M) point of the measured configurations except the bit-width
# sweep (which has its own test below): 33 points, 57 with the sweep.
FULL = [(lay.name, M) for lay in wl.LAYERS for M in lay.M_values]
_FULL_CACHE = {}


def _full_layer(name):
    """Seeded tensors of a full-size layer (x drawn for its largest M) and its
    device weight, kept for the points of the same layer."""
    if name not in _FULL_CACHE:
        _FULL_CACHE.clear()
        lay = wl.layer(name)
        t = wl.gen_all(lay)
        _FULL_CACHE[name] = (lay, t, weight(t))
    return _FULL_CACHE[name]


SWEEP = [(b, cb) for b in range(1, 9) for cb in ("3inst", "mcg", "mul1")]


@pytest.mark.parametrize("bits,cb", SWEEP, ids=[f"b{b}-{cb}" for b, cb in SWEEP])
def test_sweep_full_size_sampled(bits, cb):
    """The bit-width sweep at its real shape (K = N = 4096, 64 rows): the
    planner's call, the ALU and table decoders forced, and the first row
    alone give the same bits; sampled rows and column blocks are within the
    oracle's bound."""
    lay = wl.sweep_layer(bits, cb)
    banner(f"sweep {lay.name} M=64")
    t = wl.gen_all(lay, M=64)
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x), w.suh)
    y = bits16(ex.linear(w, xr, torch.bfloat16))
    for dec in (ex.EXL3_DECODER_ALU, ex.EXL3_DECODER_TABLE):
        assert np.array_equal(bits16(ex.linear(w, xr, torch.bfloat16, decoder=dec)), y), f"decoder {dec}"
    y1 = bits16(ex.linear(w, xr[:, :, :1].contiguous(), torch.bfloat16))
    assert np.array_equal(y1[0], y[0])
    rows, blocks = [0, 9, 18, 27, 36, 45, 54, 63], [0, 13, 31]
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[rows], col_blocks=blocks)
    res = olin.check(y[rows][:, ref.cols], ref, t.svh, lay.K, "bf16")
    banner(f"{lay.name}: {res}")
    assert res.ok, str(res)


@pytest.mark.parametrize("name,M", FULL, ids=[f"{f[0]}-M{f[1]}" for f in FULL])
def test_full_size_sampled(name, M):
    """A measured configuration at its real shape: the planner's call; the
    first row alone gives the same bits (batch invariance); the other
    decoders give the same bits (ALU and table up to 64 rows, ALU and dense
    from 512); sampled rows and column blocks (both shards' first blocks)
    within the oracle's bound."""
    lay, t, w = _full_layer(name)
    banner(f"full size {name} M={M} plan {ex.plan(w, M)}")
    x = t.x[:M]
    xr = ex.input_transform(x_dev(x), w.suh)
    y = bits16(ex.linear(w, xr, torch.bfloat16))
    # batch invariance at the real shape: the first row alone
    y1 = bits16(ex.linear(w, xr[:, :, :1].contiguous(), torch.bfloat16))
    assert np.array_equal(y1[0], y[0])
    if M <= 64 or M >= 512:  # the other decoders at the real shape
        for dec in (ex.EXL3_DECODER_ALU, ex.EXL3_DECODER_TABLE) if M <= 64 else (ex.EXL3_DECODER_ALU,
                                                                                ex.EXL3_DECODER_DENSE):
            assert np.array_equal(bits16(ex.linear(w, xr, torch.bfloat16, decoder=dec)), y), f"decoder {dec}"
    rows = sorted(set(np.linspace(0, M - 1, min(M, 8)).astype(int).tolist()))
    nblk = lay.N // 128
    blocks = sorted({0, nblk // 3, nblk - 1} | ({lay.shards[0] // 128} if lay.n_shards > 1 else set()))
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, x[rows], col_blocks=blocks)
    ysel = y[rows][:, ref.cols]
    res = olin.check(ysel, ref, t.svh, lay.K, "bf16")
    banner(f"{name} M={M} sampled rows {rows} blocks {blocks}: {res}")
    assert res.ok, str(res)
