"""GPU: seeded random layer shapes through every schedule the planner can
force on them.  Each case draws K, the shard widths, the width, the codebook
and the row count from a fixed seed; every forced tile size and fold mode
that the library accepts for the shape's own part tree must give the
automatic plan's bits (the tree fixes the arithmetic, the schedule only
orders the work), exl3_forward from x must give the same rows at the
case's M and at 1, 5 and 16 rows, and the automatic plan's output must sit
within the oracle's rounding bound.  Shapes stay small enough for the fp64
oracle."""
import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from oracle import linear as olin
from gpu_util import banner, bits16, weight, x_dev

pytestmark = pytest.mark.gpu

CB_NAMES = ("3inst", "mcg", "mul1")
N_CASES = 48


def _case(i):
    rng = np.random.default_rng(20270 + i)
    K = 128 * int(rng.integers(1, 17))
    n_shards = int(rng.integers(1, 4))
    shards = tuple(128 * int(rng.integers(1, 6)) for _ in range(n_shards))
    bits = int(rng.integers(1, 9))
    cb = CB_NAMES[int(rng.integers(0, 3))]
    M = int(rng.choice([1, 3, 16, 17, 40, 64, 100, 129, 200, 300, 520]))
    return K, shards, bits, cb, M


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_every_schedule(i):
    K, shards, bits, cb, M = _case(i)
    lay = wl.small_layer(f"rand{i}", K, shards, bits, cb, (M,), seed=700 + i)
    t = wl.gen_all(lay)
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x[:M]), w.suh)
    auto = ex.plan(w, M)
    first = bits16(ex.linear(w, xr, torch.bfloat16))
    tree = dict(parts=auto["parts"], groups=auto["groups"])
    ran = 0
    for bm in (16, 32, 64, 128, 256, 512):
        for mode in (ex.EXL3_MODE_FUSED, ex.EXL3_MODE_SLABS):
            for extra in ({}, dict(unit=1), dict(wg_cols=64)):
                f = dict(tree, bm=bm, mode=mode, **extra)
                try:
                    y = bits16(ex.linear(w, xr, torch.bfloat16, **f))
                except ex.Exl3Error as e:
                    assert e.status in (1, 2), f"{f}: {e}"  # refused: not a schedule for this tree
                    continue
                assert np.array_equal(y, first), f"case {i} {f}"
                ran += 1
    if M <= 64:
        try:
            y = bits16(ex.linear(w, xr, torch.bfloat16, decoder=ex.EXL3_DECODER_TABLE, **tree))
            assert np.array_equal(y, first), f"case {i} table"
            ran += 1
        except ex.Exl3Error as e:
            assert e.status in (1, 2)
    if M >= 100:
        try:
            y = bits16(ex.linear(w, xr, torch.bfloat16, decoder=ex.EXL3_DECODER_DENSE, **tree))
            assert np.array_equal(y, first), f"case {i} dense"
            ran += 1
        except ex.Exl3Error as e:
            assert e.status in (1, 2)
    # the whole layer from x (exl3_forward) at the case's M and at a few
    # rows, where the rotation runs inside the small-tile GEMM when it is
    # short: a row's bits are the same at every M, so each equals `first`'s
    fused = 0
    for Mf in sorted({1, 5, 16, M} & set(range(1, M + 1))):
        got = bits16(ex.forward(w, x_dev(t.x[:Mf]), torch.bfloat16))
        assert np.array_equal(got, first[:Mf]), f"case {i} forward M={Mf}"
        fused += ex.forward_workspace_bytes(w, Mf) == ex.plan(w, Mf)["workspace"]
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[:M], "bf16")
    res = olin.check(first, ref, t.svh, lay.K, "bf16")
    banner(f"random case {i}: K={K} shards={shards} {bits}-bit {cb} M={M} plan {auto}: {ran} schedules, "
           f"{fused} forward calls rotated in the GEMM, {res}")
    assert ran >= 4
    assert res.ok, str(res)
