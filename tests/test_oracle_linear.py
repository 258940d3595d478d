"""Pins for oracle.linear: the fp64 reference and the rounding-order bound."""
import numpy as np
import pytest

import workloads as wl
from oracle import format as fmt
from oracle import linear as ol
from oracle import transform as tf

SMALL = [
    wl.small_layer("s256_b4_mcg", 256, (256,), 4, "mcg", (1, 5, 16), seed=1),
    wl.small_layer("s384_b6_mul1_2sh", 384, (128, 256), 6, "mul1", (3, 16), seed=2),
    wl.small_layer("s128_b1_3inst", 128, (128,), 1, "3inst", (4,), seed=3),
    wl.small_layer("s256_b8_3inst", 256, (128,), 8, "3inst", (9,), seed=4),
]


def _ref(lay, M=None, magnitudes=False):
    t = wl.gen_all(lay, M, magnitudes)
    r = ol.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x)
    return t, r


@pytest.mark.parametrize("lay", SMALL, ids=lambda l: l.name)
def test_chain_equals_dense_reconstruction(lay):
    # y = x diag(suh) H W_q H diag(svh) / 128 through one numpy matmul per
    # shard, against the step-by-step chain with the exact (unrounded) x~.
    t = wl.gen_all(lay, magnitudes=True)
    xr64 = tf.rotate_input_f64(t.x, t.suh)  # [S, M, K]
    wq = fmt.dequantize(t.trellis, lay.bits, lay.cb)
    shard_col = ol.shard_of_columns(lay.shards)
    z = np.zeros((t.x.shape[0], lay.N))
    for s in range(lay.n_shards):
        cols = shard_col == s
        z[:, cols] = xr64[s] @ wq[:, cols]
    chain = tf.output_transform_f64(z, t.svh)
    dense = ol.dense_weight(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb)
    x64 = tf.bf16_bits_to_f32(t.x).astype(np.float64)
    direct = sum(x64 @ dense[s] for s in range(lay.n_shards))
    scale = np.max(np.abs(direct))
    assert np.max(np.abs(chain - direct)) <= 1e-12 * scale


def _f32_emulation(t, lay, ref, parts=1, out_dtype="bf16", reverse=False):
    """A float32 evaluation by another route: numpy float32 GEMMs over K parts."""
    wq = fmt.dequantize(t.trellis, lay.bits, lay.cb).astype(np.float32)
    xr = tf.f16_from_bits(ref.x_rot).astype(np.float32)
    shard_col = ol.shard_of_columns(lay.shards)
    bounds = np.linspace(0, lay.K, parts + 1).astype(int)
    partials = []
    for p in range(parts):
        k0, k1 = bounds[p], bounds[p + 1]
        zp = np.zeros((xr.shape[1], lay.N), dtype=np.float32)
        for s in range(lay.n_shards):
            cols = shard_col == s
            a = xr[s][:, k0:k1]
            b = wq[k0:k1][:, cols]
            if reverse:
                a, b = a[:, ::-1].copy(), b[::-1].copy()
            zp[:, cols] = a @ b
        partials.append(zp)
    z32 = tf.reduce_parts_f32(np.stack(partials))
    return tf.output_transform_f32(z32, t.svh, out_dtype)


@pytest.mark.parametrize("lay", SMALL, ids=lambda l: l.name)
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("parts,reverse", [(1, False), (3, False), (2, True)])
def test_float32_evaluations_lie_inside_the_bound(lay, out_dtype, parts, reverse):
    for magnitudes in (False, True):
        t, ref = _ref(lay, magnitudes=magnitudes)
        y = _f32_emulation(t, lay, ref, parts, out_dtype, reverse)
        res = ol.check(y, ref, t.svh, lay.K, out_dtype)
        assert res.ok, str(res)
        assert res.max_ratio < 0.9


def test_planted_mistakes_fall_outside_the_bound():
    lay = SMALL[0]
    t, ref = _ref(lay)
    good = _f32_emulation(t, lay, ref)
    assert ol.check(good, ref, t.svh, lay.K, "bf16").ok

    # (a) the 2**-3 output scale dropped
    y = tf.f32_to_bf16_bits(tf.bf16_bits_to_f32(good) * np.float32(8.0))
    assert not ol.check(y, ref, t.svh, lay.K, "bf16").ok
    # (b) one column's svh sign flipped
    svh = t.svh.copy()
    svh[37] ^= 0x8000
    y = tf.output_transform_f32(
        tf.f16_from_bits(ref.x_rot[0]).astype(np.float32) @ fmt.dequantize(t.trellis, lay.bits, lay.cb).astype(np.float32),
        svh, "bf16")
    assert not ol.check(y, ref, t.svh, lay.K, "bf16").ok
    # (c) tiles read transposed (kt <-> nt swapped)
    tr = t.trellis.transpose(1, 0, 2).copy()
    y = _f32_emulation(wl.Tensors(lay, tr, t.suh, t.svh, t.x), lay, ref)
    assert not ol.check(y, ref, t.svh, lay.K, "bf16").ok
    # (d) window anchored one value late (states shifted by one inside a tile)
    st = fmt.unpack_states(t.trellis, lay.bits)
    kt, nt = t.trellis.shape[:2]
    shifted = np.empty_like(st)
    for a in range(kt):
        for b in range(nt):
            words = t.trellis[a, b]
            s = np.roll(fmt.tile_states(words, lay.bits), -1)
            shifted[16 * a:16 * a + 16, 16 * b:16 * b + 16] = fmt.tile_grid(s)
    w = fmt.codebook(lay.cb, shifted).view(np.float16).astype(np.float32)
    y = tf.output_transform_f32(tf.f16_from_bits(ref.x_rot[0]).astype(np.float32) @ w, t.svh, "bf16")
    assert not ol.check(y, ref, t.svh, lay.K, "bf16").ok
    # (e) the input rotation skipped for one 128-block (x*suh*2**-4 only)
    xr = ref.x_rot.copy()
    raw = tf.bf16_bits_to_f32(t.x) * tf.f16_from_bits(t.suh[0]).astype(np.float32) * np.float32(2 ** -4)
    xr[0, :, :128] = tf.f32_to_f16_bits(raw[:, :128])
    y = tf.output_transform_f32(
        tf.f16_from_bits(xr[0]).astype(np.float32) @ fmt.dequantize(t.trellis, lay.bits, lay.cb).astype(np.float32),
        t.svh, "bf16")
    assert not ol.check(y, ref, t.svh, lay.K, "bf16").ok


def test_k_split_at_128_is_exact():
    # z over K equals the sum of z over K halves split at a multiple of 128.
    lay = SMALL[0]
    t, ref = _ref(lay)
    xr = tf.f16_from_bits(ref.x_rot[0]).astype(np.float64)
    wq = fmt.dequantize(t.trellis, lay.bits, lay.cb)
    halves = xr[:, :128] @ wq[:128] + xr[:, 128:] @ wq[128:]
    assert np.allclose(halves, ref.z, rtol=0, atol=1e-9 * np.max(np.abs(ref.z)))


def test_two_shards_equal_two_single_shard_layers():
    lay = SMALL[1]  # shards (128, 256)
    t, ref = _ref(lay)
    for s, (c0, c1) in enumerate([(0, 128), (128, 384)]):
        sub = wl.Layer("sub", lay.K, (c1 - c0,), lay.bits, lay.codebook, lay.M_values, lay.seed_base)
        r = ol.reference(t.trellis[:, c0 // 16:c1 // 16], t.suh[s:s + 1], t.svh[c0:c1], sub.shards,
                         lay.bits, lay.cb, t.x)
        assert np.array_equal(r.y, ref.y[:, c0:c1])


def test_column_block_selection_matches_full():
    lay = SMALL[0]
    t, ref = _ref(lay)
    part = ol.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x, col_blocks=[1])
    assert np.array_equal(part.y, ref.y[:, 128:256])
    assert np.array_equal(part.cols, np.arange(128, 256))


def test_bench_workloads_name_known_layers():
    """Every layer a bench workload names resolves, the bit-width sweep has all
    24 (bits, codebook) layers at K = N = 4096 with distinct seeds, and its
    first rows are the input recipe's (bf16 of standard normals)."""
    import bench
    for spec in bench.WORKLOADS.values():
        for n, Ms in spec:
            lay = wl.layer(n)
            assert max(Ms) <= lay.M_max
    # the default step holds every measured configuration: each (layer, M)
    # of the layer table and of the bit-width sweep
    default = {(n, M) for n, Ms in bench.WORKLOADS[bench.DEFAULT_WORKLOAD] for M in Ms}
    assert default == {(l.name, M) for l in wl.LAYERS + wl.SWEEP for M in l.M_values}
    assert len(default) == 57
    sweep = [wl.layer(n) for n, _ in bench.WORKLOADS["sweep_4096x4096_b1-8_all_cb"]]
    assert sorted((l.bits, l.codebook) for l in sweep) == sorted(
        (b, cb) for b in range(1, 9) for cb in ("3inst", "mcg", "mul1"))
    assert all(l.K == 4096 and l.N == 4096 and l.M_values == (64,) for l in sweep)
    assert len({l.seed_base for l in sweep}) == 24
    t = wl.gen_all(sweep[0], M=2)
    assert t.trellis.shape == (256, 256, 16) and t.x.shape == (2, 4096)


def _bits_to_f64(y, out_dtype):
    return ol.out_bits_to_f64(y, out_dtype)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("P", [1, 2, 5, 17])
def test_output_stage_bound_holds_for_fp32_folds(out_dtype, P):
    """The output stage's plain definition (fp64 sum of the parts, then
    H128 * 2**-3 * svh) with its bound: float32 folds of the parts in
    several orders (flat, reversed, grouped in two and four, pairwise),
    each followed by the float32 output stage, all lie inside; with a bias
    too."""
    rng = np.random.default_rng(700 + P)
    M, N = 9, 256
    z = (rng.standard_normal((P, M, N)) * np.exp2(rng.integers(-6, 6, (P, M, N)))).astype(np.float32)
    svh = (np.where(rng.integers(0, 2, N) == 1, -1.0, 1.0) * np.exp2(rng.uniform(-2, 2, N))
           ).astype(np.float16).view(np.uint16)
    bias = (rng.standard_normal(N) * 2).astype(np.float16).view(np.uint16)
    folds = [z.sum(axis=0, dtype=np.float32)]  # numpy's pairwise order
    for order in (list(range(P)), list(reversed(range(P)))):
        acc = z[order[0]].copy()
        for p in order[1:]:
            acc = (acc + z[p]).astype(np.float32)
        folds.append(acc)
    for G in (2, 4):
        if P % G == 0:
            folds.append(tf.reduce_parts_f32(z, G))
    for b in (None, bias):
        ystar, B = ol.output_stage_reference(z, svh, out_dtype, b)
        for f in folds:
            y = _bits_to_f64(tf.output_transform_f32(f, svh, out_dtype, b), out_dtype)
            r = np.abs(y - ystar) / B
            assert np.max(r) <= 1.0, f"fold outside the bound: {np.max(r)}"


def test_output_stage_bound_rejects_planted_mistakes():
    """A dropped part, a flipped svh, a dropped 2**-3 and one block left
    unrotated all fall outside the output stage's bound."""
    rng = np.random.default_rng(710)
    P, M, N = 4, 8, 256
    z = (rng.standard_normal((P, M, N))).astype(np.float32)
    svh = np.where(rng.integers(0, 2, N) == 1, 0xBC00, 0x3C00).astype(np.uint16)
    ystar, B = ol.output_stage_reference(z, svh, "bf16")
    full = tf.reduce_parts_f32(z)

    def bad(y_bits):
        return np.max(np.abs(_bits_to_f64(y_bits, "bf16") - ystar) / B) > 1.0

    assert not bad(tf.output_transform_f32(full, svh, "bf16"))
    assert bad(tf.output_transform_f32(tf.reduce_parts_f32(z[:3]), svh, "bf16"))
    flipped = svh.copy()
    flipped[5] ^= 0x8000
    assert bad(tf.output_transform_f32(full, flipped, "bf16"))
    y8 = tf.bf16_bits_to_f32(tf.output_transform_f32(full, svh, "bf16")) * np.float32(8)
    assert bad(tf.f32_to_bf16_bits(y8))
    raw = full * np.float32(0.125) * tf.f16_from_bits(svh).astype(np.float32)[None, :]
    y = tf.output_transform_f32(full, svh, "bf16")
    y[:, 128:] = tf.f32_to_bf16_bits(raw[:, 128:])
    assert bad(y)


def test_worst_column_limit_needs_enough_rows():
    """One row whose output in some column is near zero: the element-wise
    bound holds and the column-relative error is large, so the check uses
    the matrix-wide relative error there; from 8 rows the column limit
    applies."""
    lay = SMALL[0]
    t, ref = _ref(lay)
    good = _f32_emulation(t, lay, ref)
    r1 = ol.Reference(ref.x_rot[:, :1], ref.z[:1], ref.absdot[:1], ref.y[:1], ref.cols)
    res = ol.check(good[:1], r1, t.svh, lay.K, "bf16")
    assert res.max_ratio <= 1.0 and res.ok
    assert ref.y.shape[0] >= ol.MIN_ROWS_FOR_COLUMNS
    full = ol.check(good, ref, t.svh, lay.K, "bf16")
    assert full.ok and full.worst_col_rel <= 5e-3
