"""GPU: the single-GPU half of a column split, and padded layers.

Column split (cuda-exl3 README, "Tensor parallel" and "Notes on the format":
trellis and svh concatenate along the output dimension, so a GPU that owns
whole 128-column blocks runs its slice of the trellis, svh and shard map on
the replicated x): its columns have the bits of the full layer's when the
slice runs with the full layer's part tree (P and G come from the global
shape), which a forced plan carries, and they lie within the oracle's bound.

Padded layers (cuda-exl3 README, "Loading into a dim vLLM has padded"): whole
128-column blocks of output padding with svh zeroed come out exactly zero
whatever trellis is behind them, and the real columns are untouched; input
positions that carry zeros make suh there irrelevant, and a whole block of
them makes the trellis rows there irrelevant too."""
import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from oracle import linear as olin
from gpu_util import banner, bits16, dev16, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ex.load()
    torch.cuda.init()


def _weight(trellis, suh, svh, bits, cb, shards):
    return ex.Exl3Weight(dev16(trellis), dev16(suh, torch.float16), dev16(svh, torch.float16), bits, cb, shards)


def _slice(lay, t, c0, c1):
    """Columns [c0, c1) of a layer (whole 128-column blocks): trellis, svh,
    and the shard map and suh rows of the shards the range touches."""
    shards, rows, start = [], [], 0
    for s, n in enumerate(lay.shards):
        lo, hi = max(c0, start), min(c1, start + n)
        if lo < hi:
            shards.append(hi - lo)
            rows.append(s)
        start += n
    tr = np.ascontiguousarray(t.trellis[:, c0 // 16:c1 // 16])
    return _weight(tr, np.ascontiguousarray(t.suh[rows]), np.ascontiguousarray(t.svh[c0:c1]), lay.bits,
                   lay.codebook, shards)


@pytest.mark.parametrize("M", [1, 37, 300])
def test_column_slices_match_the_full_layer(M):
    # 8 parts in 8 groups for the whole layer; a slice of up to 1024 columns
    # alone would take 32 parts in 8 groups
    lay = wl.small_layer("colsplit", 4096, (3072, 2048, 3072), 5, "mul1", (300,), seed=401)
    t = wl.gen_all(lay)
    w = _weight(t.trellis, t.suh, t.svh, lay.bits, lay.codebook, lay.shards)
    x = x_dev(t.x[:M])
    y = bits16(ex.linear(w, ex.input_transform(x, w.suh), torch.bfloat16))
    pl = ex.plan(w, M)
    banner(f"column split M={M}: full plan {pl}")
    differs = False
    for c0, c1 in ((0, 256), (2944, 3328), (4864, 5888), (7936, 8192)):
        ws = _slice(lay, t, c0, c1)
        xr = ex.input_transform(x, ws.suh)
        got = bits16(ex.linear(ws, xr, torch.bfloat16, parts=pl["parts"], groups=pl["groups"]))
        assert np.array_equal(got, y[:, c0:c1]), f"columns {c0}:{c1}"
        own = ex.plan(ws, M)
        differs |= (own["parts"], own["groups"]) != (pl["parts"], pl["groups"])
    assert differs, "every slice's own plan has the full layer's tree: the forced tree was not exercised"
    # the slices' columns against the oracle (sampled rows)
    rows = sorted({0, M // 2, M - 1})
    blocks = [0, 2944 // 128, 4864 // 128, 7936 // 128, 8064 // 128]
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[rows], col_blocks=blocks)
    res = olin.check(y[rows][:, ref.cols], ref, t.svh, lay.K, "bf16")
    banner(f"column split M={M} vs oracle: {res}")
    assert res.ok, str(res)


@pytest.mark.parametrize("out", [torch.bfloat16, torch.float16])
def test_padded_output_blocks_are_exact_zeros(out):
    """384 real columns + one 128-column block of pad: svh zero there, the
    trellis behind it uninitialised (random words).  The pad is exactly zero
    and the real columns have the bits of the unpadded layer run with the
    padded layer's tree."""
    real = wl.small_layer("pad_real", 1024, (384,), 4, "3inst", (24,), seed=402)
    t = wl.gen_all(real)
    rng = np.random.default_rng(403)
    junk = rng.integers(0, 65536, (t.trellis.shape[0], 8, t.trellis.shape[2]), dtype=np.uint16)
    tr_pad = np.concatenate([t.trellis, junk], axis=1)
    svh_pad = np.concatenate([t.svh, np.zeros(128, dtype=np.uint16)])
    wp = _weight(tr_pad, t.suh, svh_pad, 4, "3inst", (512,))
    wr = _weight(t.trellis, t.suh, t.svh, 4, "3inst", (384,))
    for M in (1, 24):
        x = x_dev(t.x[:M])
        yp = ex.linear(wp, ex.input_transform(x, wp.suh), out)
        assert torch.all(yp[:, 384:].float() == 0), "pad columns not exactly zero"
        pl = ex.plan(wp, M)
        yr = ex.linear(wr, ex.input_transform(x, wr.suh), out, parts=pl["parts"], groups=pl["groups"])
        assert np.array_equal(bits16(yp[:, :384]), bits16(yr)), f"M={M}"
        od = "bf16" if out == torch.bfloat16 else "f16"
        ref = olin.reference(t.trellis, t.suh, t.svh, real.shards, real.bits, real.cb, t.x[:M])
        res = olin.check(bits16(yr), ref, t.svh, real.K, od)
        assert res.ok, f"M={M}: {res}"


def test_padded_input_positions():
    """x is zero at k >= 400 (the producing layer's pad).  Garbage suh there
    cannot reach the output (bit-identical to other garbage); over the whole
    pad block k >= 512 the trellis rows cannot either; and the result is
    within the oracle's bound."""
    lay = wl.small_layer("pad_in", 640, (256,), 6, "mcg", (17,), seed=404)
    t = wl.gen_all(lay)
    rng = np.random.default_rng(405)
    x = t.x.copy()
    x[:, 400:] = 0
    outs = []
    for trial in range(2):
        suh = t.suh.copy()
        suh[:, 400:] = rng.integers(0x3C00, 0x5000, (1, 240), dtype=np.uint16)  # positive finite fp16
        tr = t.trellis.copy()
        tr[512 // 16:] = rng.integers(0, 65536, tr[512 // 16:].shape, dtype=np.uint16)
        w = _weight(tr, suh, t.svh, lay.bits, lay.codebook, lay.shards)
        outs.append(bits16(ex.linear(w, ex.input_transform(x_dev(x), w.suh), torch.bfloat16)))
        ref = olin.reference(tr, suh, t.svh, lay.shards, lay.bits, lay.cb, x, "bf16")
        res = olin.check(outs[-1], ref, t.svh, lay.K, "bf16")
        assert res.ok, str(res)
    assert np.array_equal(outs[0], outs[1])
