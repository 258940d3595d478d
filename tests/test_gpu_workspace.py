"""GPU: the binding's process-wide workspaces (cuda-exl3 README, "VRAM":
activation and split-k workspaces are process-wide; the arrival counters at
a workspace's start are zero on entry and left zero by every call).

One workspace per (device, stream): calls on two streams that overlap do not
share counters or slabs.  A workspace is never freed once used, so a graph
captured against it stays valid after a larger call grows the stream's
workspace; one allocated under capture zeroes its counters inside the graph
and again before its first eager use."""
import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from gpu_util import banner, bits16, weight, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ex.load()
    torch.cuda.init()


def _layer(seed, K=2048, N=512, bits=4, cb="mcg", M=256):
    lay = wl.small_layer(f"ws{seed}", K, (N,), bits, cb, (M,), seed=seed)
    t = wl.gen_all(lay)
    return t, weight(t)


def test_graph_survives_workspace_growth():
    """Capture at 16 rows (finishing-workgroup slabs), grow the stream's
    workspace eagerly at 256 rows, replay: the graph's bits are the eager
    bits on every replay, with eager calls between replays."""
    t, w = _layer(901)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xr16 = ex.input_transform(x_dev(t.x[:16]), w.suh)
        want16 = bits16(ex.linear(w, xr16, torch.bfloat16))
        assert ex.plan(w, 16)["mode"] == ex.EXL3_MODE_SLABS
        y = torch.empty((16, w.N), dtype=torch.bfloat16, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            ex.linear(w, xr16, torch.bfloat16, out=y)
        before = ex._workspaces[ex.workspace_key(stream=s)].data_ptr()
        xr256 = ex.input_transform(x_dev(t.x[:256]), w.suh)
        big = bits16(ex.linear(w, xr256, torch.bfloat16))
        after = ex._workspaces[ex.workspace_key(stream=s)].data_ptr()
        banner(f"workspace {before:#x} -> {after:#x}")
        for _ in range(3):
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits16(y), want16)
            assert np.array_equal(bits16(ex.linear(w, xr256, torch.bfloat16)), big)
    assert np.array_equal(big[:16], want16)


def test_workspace_first_allocated_under_capture():
    """A stream whose first call is captured: the graph zeroes its counters,
    and eager calls on the stream afterwards (between replays) see zero
    counters too."""
    t, w = _layer(902, M=64)
    xr = ex.input_transform(x_dev(t.x[:64]), w.suh)
    want = bits16(ex.linear(w, xr, torch.bfloat16))
    s = torch.cuda.Stream()
    assert ex.workspace_key(stream=s) not in ex._workspaces
    y = torch.empty((64, w.N), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ex.linear(w, xr, torch.bfloat16, out=y)
    with torch.cuda.stream(s):
        for _ in range(3):
            assert np.array_equal(bits16(ex.linear(w, xr, torch.bfloat16)), want)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits16(y), want)


def test_two_streams_do_not_share_counters():
    """Two layers with finishing-workgroup slabs launched alternately on two
    streams, many calls in flight at once: every output is the serial one."""
    t1, w1 = _layer(903, K=4096, N=1024, M=16)
    t2, w2 = _layer(904, K=2048, N=2048, M=16)
    x1 = ex.input_transform(x_dev(t1.x[:16]), w1.suh)
    x2 = ex.input_transform(x_dev(t2.x[:16]), w2.suh)
    want1 = bits16(ex.linear(w1, x1, torch.bfloat16))
    want2 = bits16(ex.linear(w2, x2, torch.bfloat16))
    assert ex.plan(w1, 16)["launches"] == 1 and ex.plan(w2, 16)["launches"] == 1
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for i in range(40):
        with torch.cuda.stream(sa):
            outs.append((1, ex.linear(w1, x1, torch.bfloat16)))
        with torch.cuda.stream(sb):
            outs.append((2, ex.linear(w2, x2, torch.bfloat16)))
    torch.cuda.synchronize()
    assert ex.workspace_key(stream=sa) != ex.workspace_key(stream=sb)
    for which, y in outs:
        assert np.array_equal(bits16(y), want1 if which == 1 else want2)
