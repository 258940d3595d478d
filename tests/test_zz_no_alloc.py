"""GPU: exl3_linear_noalloc, the entry point for callers that cannot
allocate, through the C ABI: every call's output has exactly the bits of
exl3_linear with its workspace, on two calls in a row with the second one
smaller -- plans whose workspace fits the library's scratch, one whose slabs
need row chunks there, one whose planner schedule (dequantized weights)
does not fit and runs another schedule of the same part tree, and one-part
plans on the 512- and 128-row tiles."""
import ctypes

import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from gpu_util import banner, bits16, weight, x_dev

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ex.load()
    torch.cuda.init()


def _noalloc(w, xr, M, out_dtype=torch.bfloat16):
    y = torch.empty((M, w.N), dtype=out_dtype, device="cuda")
    st = ex.load().exl3_linear_noalloc(ctypes.byref(w.view()), xr.data_ptr(), M, y.data_ptr(),
                                       1 if out_dtype == torch.bfloat16 else 0, ex._stream())
    ex._check(st)
    return y


CASES = [
    # (name, K, shards, bits, cb, first M, second M)
    ("finisher_slabs", 4096, (2048,), 4, "mcg", 16, 1),
    ("row_chunks", 4096, (2048,), 4, "mcg", 3000, 517),
    ("dense_planner", 4096, (4096, 4096), 4, "mul1", 2048, 100),
    ("table", 5120, (12288,), 6, "mul1", 64, 24),
    # one part over all of K (256 column blocks): 512-row tiles, then 128-row
    # tiles two to a CU
    ("wide_tiles", 1024, (32768,), 4, "mul1", 600, 128),
]


@pytest.mark.parametrize("name,K,shards,bits,cb,m1,m2", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_linear(name, K, shards, bits, cb, m1, m2):
    lay = wl.small_layer(f"na_{name}", K, shards, bits, cb, (m1,), seed=950 + len(name))
    t = wl.gen_all(lay)
    w = weight(t)
    plan1 = ex.plan(w, m1)
    banner(f"noalloc {name}: planner at M={m1} {plan1}")
    if name == "dense_planner":
        assert plan1["decoder"] == ex.EXL3_DECODER_DENSE and plan1["workspace"] > SCRATCH
    if name == "wide_tiles":
        assert plan1["bm"] == 512 and plan1["parts"] == 1 and ex.plan(w, m2)["bm"] == 128
    if name == "row_chunks":
        # the planner keeps 8 group slabs of all 3000 rows (196 MB); the
        # scratch takes them in row chunks
        assert plan1["mode"] == ex.EXL3_MODE_SLABS and plan1["workspace"] > SCRATCH
    for M, dt in ((m1, torch.bfloat16), (m2, torch.float16)):
        xr = ex.input_transform(x_dev(t.x[:M]), w.suh)
        want = bits16(ex.linear(w, xr, dt))
        got = bits16(_noalloc(w, xr, M, dt))
        torch.cuda.synchronize()
        assert np.array_equal(got, want), f"M={M}"


def test_noalloc_checks_before_any_work():
    lay = wl.small_layer("na_check", 1024, (256,), 4, "mcg", (4,), seed=990)
    t = wl.gen_all(lay)
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x), w.suh)
    y = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    L = ex.load()
    assert L.exl3_linear_noalloc(ctypes.byref(w.view()), xr.data_ptr(), 4, y.data_ptr(), 7, ex._stream()) == 1
    assert "y_dtype=7" in L.exl3_last_error().decode()
    assert L.exl3_linear_noalloc(ctypes.byref(w.view()), xr.data_ptr(), 0, None, 1, ex._stream()) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0
