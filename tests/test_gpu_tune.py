"""GPU: the schedule autotuner times the schedules of the shape's own part
tree and records the fastest; the output bits never change, the recorded
schedule is what later unforced calls run, and tuning is refused while the
stream is being captured into a graph (cuda-exl3 README, "Where the time
goes": tune once per shape in eager warm-up, the cost model under capture)."""
import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from oracle import linear as olin
from gpu_util import banner, bits16, weight, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ex.load()
    torch.cuda.init()
    yield
    ex.tune_clear()


CASES = [("small", 1), ("small", 100), ("small", 300), ("q_proj_5120x12288_b6_mul1", 128),
         ("q_proj_5120x12288_b6_mul1", 16)]


@pytest.mark.parametrize("name,M", CASES, ids=[f"{c[0]}-M{c[1]}" for c in CASES])
def test_tune_keeps_bits_and_is_used(name, M):
    lay = (wl.small_layer("tune_small", 2048, (256, 384), 5, "mcg", (300,), seed=501) if name == "small"
           else wl.layer(name))
    t = wl.gen_all(lay, M=M)
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x[:M]), w.suh)
    ex.tune_clear()
    planned = ex.plan(w, M)
    y0 = bits16(ex.linear(w, xr, torch.bfloat16))
    copies = [w] + [ex.Exl3Weight(w.trellis.clone(), w.suh, w.svh, w.bits, w.codebook, w.shard_n) for _ in range(2)]
    best = ex.tune(copies, xr, reps=3)
    banner(f"tune {name} M={M}: planner {planned} -> tuned {best}")
    assert (best["parts"], best["groups"]) == (planned["parts"], planned["groups"])
    now = ex.plan(w, M)
    for k in ("parts", "groups", "mode", "bm", "decoder", "unit", "wg_cols"):
        assert now[k] == best[k], k
    y1 = bits16(ex.linear(w, xr, torch.bfloat16))
    assert np.array_equal(y0, y1)
    # the tuned schedule's output against the oracle (sampled rows and blocks)
    rows = sorted(set(np.linspace(0, M - 1, min(M, 8)).astype(int).tolist()))
    nblk = lay.N // 128
    blocks = sorted({0, nblk // 2, nblk - 1})
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[rows], col_blocks=blocks)
    res = olin.check(y1[rows][:, ref.cols], ref, t.svh, lay.K, "bf16")
    banner(f"tuned {name} M={M} vs oracle: {res}")
    assert res.ok, str(res)
    ex.tune_clear()
    assert ex.plan(w, M) == planned


def test_tune_refused_under_capture():
    lay = wl.small_layer("tune_cap", 1024, (256,), 4, "mcg", (8,), seed=502)
    t = wl.gen_all(lay)
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x), w.suh)
    ex.tune(w, xr, reps=1)  # eager: sizes the workspace
    y = torch.empty((8, 256), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    caught = None
    with torch.cuda.graph(g, stream=side):
        try:
            ex.tune(w, xr, reps=1)
        except ex.Exl3Error as e:
            caught = e
        ex.linear(w, xr, torch.bfloat16, out=y)
    assert caught is not None and caught.status == 2 and "captured" in str(caught)
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits16(y), bits16(ex.linear(w, xr, torch.bfloat16)))
    ex.tune_clear()
