"""Golden fixtures (tests/golden/): values worked by hand from the pages'
constants, the numbers the pages print, and small worked examples of the
whole linear written by tests/golden/make_golden.py (which calls only the
oracle).  The CPU tests pin the oracle to them; the GPU test checks the
library against the stored reference and bound without running the oracle."""
import json
import os
import struct
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import format as fmt
from oracle import linear as olin
from oracle import transform as otf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
import make_golden  # noqa: E402

CB_ID = {"3inst": fmt.CB_3INST, "mcg": fmt.CB_MCG, "mul1": fmt.CB_MUL1}


def _worked_codebook():
    rows = []
    for line in open(os.path.join(GOLDEN, "codebook_worked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        cb, state, bits = line.split()[:3]
        rows.append((cb, int(state, 16), int(bits, 16)))
    return rows


@pytest.mark.parametrize("cb,state,bits", _worked_codebook())
def test_codebook_worked_by_hand(cb, state, bits):
    assert int(fmt.codebook(CB_ID[cb], np.array([state]))[0]) == bits


def _f16(b):
    return struct.unpack("<e", struct.pack("<H", b))[0]


def test_page_constants():
    pc = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    # mcg: state 1 hashes to the printed multiplier itself; its pair sum by
    # hand through CPython's fp16 rounding
    mult = int(pc["mcg_multiplier"]["value"], 16)
    u = (mult & 0x8FFF8FFF) ^ 0x30003000
    want = struct.unpack("<H", struct.pack("<e", _f16(u & 0xFFFF) + _f16(u >> 16)))[0]
    assert int(fmt.codebook(fmt.CB_MCG, np.array([1]))[0]) == want
    assert otf.BLOCK == pc["hadamard_block"]["value"]
    assert otf.INPUT_SCALE == 2.0 ** pc["input_scale_log2"]["value"]
    assert otf.OUTPUT_SCALE == 2.0 ** pc["output_scale_log2"]["value"]
    assert sorted(fmt.CODEBOOK_NAMES.values()) == sorted(pc["codebooks"]["value"])
    for cb in fmt.CODEBOOK_NAMES:
        assert fmt.codebook_table(cb).shape == (pc["states_per_codebook"]["value"],)
    # a tile of every width unpacks to 16 x 16 values
    rng = np.random.default_rng(5)
    for b in pc["widths"]["value"]:
        tr = rng.integers(0, 65536, (1, 1, 16 * b), dtype=np.uint16)
        assert fmt.dequantize_bits(tr, b, fmt.CB_MCG).shape == tuple(pc["trellis_tile"]["value"])


def _worked_files():
    return sorted(f for f in os.listdir(GOLDEN) if f.startswith("worked_") and f.endswith(".json"))


def _load(name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    L = g["layer"]
    lay = wl.small_layer(L["name"], L["K"], tuple(L["shards"]), L["bits"], L["codebook"], (L["M"],), seed=L["seed"])
    t = wl.gen_all(lay)
    y = np.array([[float.fromhex(v) for v in row] for row in g["y_ref_hex"]])
    b = np.array([[float.fromhex(v) for v in row] for row in g["bound_bf16_hex"]])
    return g, lay, t, y, b


@pytest.mark.parametrize("name", _worked_files())
def test_worked_example_oracle_regression(name):
    """The seeded inputs and the oracle's x~, y* and bound are unchanged."""
    g, lay, t, y, b = _load(name)
    assert make_golden.input_hash(t) == g["input_sha256"], "the seeded input generator changed"
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x)
    assert np.array_equal(ref.x_rot, np.array(g["x_rot_bits"], dtype=np.uint16))
    assert np.array_equal(ref.y, y)
    assert np.array_equal(olin.bound(ref, t.svh, lay.K, "bf16"), b)


@pytest.mark.gpu
@pytest.mark.parametrize("name", _worked_files())
def test_worked_example_on_gpu(name):
    """The library's output within the stored bound of the stored y*."""
    import torch

    import linear_exl3_input_amd as ex
    from gpu_util import bits16, weight, x_dev
    g, lay, t, y, b = _load(name)
    w = weight(t)
    xr = ex.input_transform(x_dev(t.x), w.suh)
    out = bits16(ex.linear(w, xr, torch.bfloat16))
    err = np.abs(otf.bf16_bits_to_f32(out).astype(np.float64) - y)
    assert np.all(err <= b), f"worst {np.max(err / b):.3f} of the bound"
