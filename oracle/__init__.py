"""CPU oracle for the EXL3 quantized linear  y = had(W_q . had(x*suh)) * svh.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the C-ABI library and its Python binding) never
imports it, and this package never imports the product: the two share no
code, tables, constants or helpers.  The only common dependency is the seeded
input generator in ``workloads``, which holds no arithmetic of the method.

The oracle is plain, slow and written to be checked by eye against the pages:

* ``format``    -- the trellis tile unpack, the three procedural codebooks and
                   the in-tile value order (sources: the cuda-exl3 page,
                   "What is supported" and "Notes on the format"; the
                   TensorFold PR "cuda: EXL3 projections behind qlinear",
                   "What it adds" and "Arithmetic" step 2).
* ``transform`` -- the 128-point Hadamard rotations on both sides, with the
                   rounding order of the TensorFold PR, "Arithmetic" steps 1
                   and 3.
* ``linear``    -- the fp64 reference output and the per-element error bound
                   derived from that rounding order ("Tests (GB10)" reports
                   errors as a fraction of such a bound).

Where the pages leave a convention open (bit order in a tile, the window
anchor, the 3inst and mul1 constants, the fp32 add order of the Hadamard) the
oracle takes one reading, stated in the docstring of the function that uses
it.  Parity status per function is listed in each module's header.
"""
from . import format, transform, linear  # noqa: F401
