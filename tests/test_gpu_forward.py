"""GPU: exl3_forward (the whole layer from x in one call) gives exactly the
bits of exl3_input_transform followed by exl3_linear, both where the
rotation runs inside the small-tile GEMM (one launch) and where the call
falls back to the transform into its workspace; plus the oracle's bound on
one rotated-in-GEMM case."""
import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from oracle import linear as olin
from gpu_util import banner, bits16, dev16, weight, x_dev

pytestmark = pytest.mark.gpu


def _fused(w, M):
    """True when the call rotates inside the GEMM: its workspace is the
    plan's own (no room for x_rot)."""
    return ex.forward_workspace_bytes(w, M) == ex.plan(w, M)["workspace"]


# (name, K, shards, bits, cb, {M: rotation in the GEMM expected}); the
# rotation runs in the GEMM while a tile's rows times the stages of a quad
# stay within 16 (two stages a quad on the 4096 x 4096 layer: up to 8 rows)
CASES = [
    ("sweep_like", 4096, (4096,), 4, "mcg", {8: True, 5: True, 12: False, 40: False}),
    ("expert_like", 4096, (2048,), 4, "mcg", {1: True, 16: True, 7: True, 17: False}),
    ("small_like", 1024, (1024,), 4, "3inst", {1: True, 16: True}),
    ("two_shards", 1024, (256, 384), 6, "mul1", {5: True, 33: False, 50: False}),
    ("odd_width", 2048, (640,), 3, "mul1", {1: True, 17: False, 64: False}),
    # one part over all of K: eight stages a quad, more than its slots
    ("one_part", 1024, (32768,), 4, "mul1", {16: False, 128: False, 300: False}),
]


@pytest.mark.parametrize("name,K,shards,bits,cb,Ms", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("x_dtype", ["bf16", "f16"])
def test_forward_equals_transform_then_linear(name, K, shards, bits, cb, Ms, x_dtype):
    lay = wl.small_layer(f"fw_{name}", K, shards, bits, cb, (max(Ms),), seed=1300 + K % 97 + bits)
    t = wl.gen_all(lay)
    w = weight(t)
    for M, expect in Ms.items():
        x = x_dev(t.x[:M], x_dtype)
        fused = _fused(w, M)
        assert fused == expect, f"M={M}: rotation in the GEMM {fused}, expected {expect} ({ex.plan(w, M)})"
        for out in (torch.bfloat16, torch.float16):
            want = bits16(ex.linear(w, ex.input_transform(x, w.suh), out))
            got = bits16(ex.forward(w, x, out))
            torch.cuda.synchronize()
            assert np.array_equal(got, want), f"{name} M={M} x {x_dtype} out {out} fused={fused}"
        banner(f"forward {name} M={M} x {x_dtype}: rotation in the GEMM {fused}, bits equal")


def test_forward_with_bias_and_oracle():
    lay = wl.small_layer("fw_bias", 2048, (512, 256), 5, "mcg", (13,), seed=1390)
    t = wl.gen_all(lay)
    rng = np.random.default_rng(1391)
    bias = (rng.standard_normal(lay.N) * 2).astype(np.float16).view(np.uint16)
    w = ex.Exl3Weight(dev16(t.trellis), dev16(t.suh, torch.float16), dev16(t.svh, torch.float16), lay.bits,
                      lay.codebook, lay.shards, bias=dev16(bias, torch.float16))
    M = 13
    assert _fused(w, M), ex.plan(w, M)
    x = x_dev(t.x[:M])
    got = bits16(ex.forward(w, x, torch.bfloat16))
    want = bits16(ex.linear(w, ex.input_transform(x, w.suh), torch.bfloat16))
    assert np.array_equal(got, want)
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x[:M], "bf16", bias_bits=bias)
    res = olin.check(got, ref, t.svh, lay.K, "bf16")
    banner(f"forward with bias, rotation in the GEMM: {res}")
    assert res.ok, str(res)


def test_forward_rows_alone_and_repeat():
    """A row's bits alone equal its bits in the batch, and a repeated call
    gives the same bits (the rotation in the GEMM, finishing workgroup)."""
    lay = wl.small_layer("fw_rows", 4096, (2048,), 4, "mcg", (16,), seed=1392)
    t = wl.gen_all(lay)
    w = weight(t)
    x = x_dev(t.x[:16])
    assert _fused(w, 16) and _fused(w, 1)
    batch = bits16(ex.forward(w, x, torch.bfloat16))
    again = bits16(ex.forward(w, x, torch.bfloat16))
    assert np.array_equal(batch, again)
    for r in (0, 5, 15):
        alone = bits16(ex.forward(w, x_dev(t.x[r:r + 1]), torch.bfloat16))
        assert np.array_equal(alone[0], batch[r]), f"row {r}"


def test_forward_under_graph_capture():
    lay = wl.small_layer("fw_graph", 4096, (2048,), 4, "mcg", (16,), seed=1393)
    t = wl.gen_all(lay)
    w = weight(t)
    x = x_dev(t.x[:16])
    want = bits16(ex.forward(w, x, torch.bfloat16))
    y = torch.empty((16, w.N), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ex.forward(w, x, torch.bfloat16, out=y)  # sizes this stream's workspace eagerly
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            ex.forward(w, x, torch.bfloat16, out=y)
        for _ in range(3):
            y.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits16(y), want)
            assert np.array_equal(bits16(ex.forward(w, x, torch.bfloat16)), want)


def test_staged_forward_leaves_the_counters_zero():
    """A forward that stages x_rot in the workspace (its plan needs no
    workspace of its own) followed by ones that rotate in the GEMM and
    elect a finishing workgroup through the shared arrival counters."""
    staged = wl.small_layer("fw_staged", 1024, (32768,), 4, "mul1", (16,), seed=1394)
    fused = wl.small_layer("fw_after", 4096, (2048,), 4, "mcg", (16,), seed=1395)
    ts, tf = wl.gen_all(staged), wl.gen_all(fused)
    ws_, wf = weight(ts), weight(tf)
    assert ex.plan(ws_, 16)["workspace"] == 0 and not _fused(ws_, 16) and _fused(wf, 16)
    xs, xf = x_dev(ts.x[:16]), x_dev(tf.x[:16])
    want = bits16(ex.linear(wf, ex.input_transform(xf, wf.suh), torch.bfloat16))
    for _ in range(2):
        ex.forward(ws_, xs, torch.bfloat16)
        for _ in range(2):
            assert np.array_equal(bits16(ex.forward(wf, xf, torch.bfloat16)), want)
    banner("staged forward then fused forwards: bits equal")
