"""Writes tests/golden/worked_*.json: small worked examples of the whole
linear, computed by the CPU oracle alone (``oracle/``), from the seeded
synthetic inputs of ``workloads``.

    python tests/golden/make_golden.py

Each file stores the inputs' generation recipe and a hash of them, the rotated
activations x~ (fp16 bits), the fp64 reference output y* (exact float hex) and
the per-element error bound B of the oracle, so a test can check a result
against them without running the oracle.  Nothing here comes from the GPU.
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402
from oracle import linear as olin  # noqa: E402

CASES = [
    # name, K, shards, bits, codebook, M, seed
    ("worked_256x2x128_b3_mcg", 256, (128, 128), 3, "mcg", 3, 701),
    ("worked_384x128_b6_mul1", 384, (128,), 6, "mul1", 2, 702),
    ("worked_128x256_b5_3inst", 128, (256,), 5, "3inst", 5, 703),
]


def input_hash(t) -> str:
    h = hashlib.sha256()
    for a in (t.trellis, t.suh, t.svh, t.x):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:32]


def make(name, K, shards, bits, cb, M, seed):
    lay = wl.small_layer(name, K, shards, bits, cb, (M,), seed=seed)
    t = wl.gen_all(lay)
    ref = olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x)
    b = olin.bound(ref, t.svh, lay.K, "bf16")
    return {
        "layer": {"name": name, "K": K, "shards": list(shards), "bits": bits, "codebook": cb, "M": M, "seed": seed},
        "recipe": "workloads.gen_all(workloads.small_layer(name, K, shards, bits, codebook, (M,), seed=seed))",
        "input_sha256": input_hash(t),
        "x_rot_bits": ref.x_rot.astype(int).tolist(),
        "y_ref_hex": [[float(v).hex() for v in row] for row in ref.y],
        "bound_bf16_hex": [[float(v).hex() for v in row] for row in b],
    }


def main():
    for case in CASES:
        out = make(*case)
        path = os.path.join(HERE, case[0] + ".json")
        with open(path, "w") as f:
            json.dump(out, f, separators=(",", ":"))
            f.write("\n")
        print("wrote", path)


if __name__ == "__main__":
    main()
