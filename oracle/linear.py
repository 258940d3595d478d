"""Reference output and error bound of the EXL3 linear (oracle; test
infrastructure).

  y = had(W_q . had(x*suh)) * svh        (cuda-exl3 page, "One op per layer")

Pages
-----
* The whole quantized linear is one call; fused layers (qkv, gate_up) run all
  shards in one GEMM; trellis, svh and the output are addressed by absolute
  column, and only the activation slice (one suh row per shard) differs
  (cuda-exl3, "One op per layer" and "Notes on the format").
* fp16 inputs to the products, fp32 sums, one rounding at the output; the
  reference is fp64 and the error is reported as a fraction of "a bound
  derived from the kernels' rounding order", with the worst column also
  reported (TensorFold PR "cuda: EXL3 projections behind qlinear",
  "Arithmetic" and "Tests (GB10)").

The reference keeps the one rounding the format itself specifies -- x~ in
fp16, produced in the format's fp32 order (``transform.rotate_input``) -- and
computes everything after it exactly in float64:
    z* = x~ @ W_q                       (numpy float64 matmul)
    y* = H128(z*) * 2**-3 * svh         (float64)

The bound (per element m, n; blk(n) is n's 128-column block):

    B_mn = u_o |y*_mn| + (1 + u_o) * 2**-3 |svh_n|
           * sum_{j in blk(n)} ( g_K A_mj + g_8 (|z*_mj| + g_K A_mj) ) + a_o

    A_mj = sum_k |x~_mk w_kj|,   g_n = n u / (1 - n u).

Derivation: the contraction has K products, each exact in fp32 (fp16 x fp16),
summed in some order, so |z^ - z*| <= g_K A (with u = 2**-23 for this term,
which also covers sums rounded toward zero inside the matrix unit).  The
output butterfly is 7 fp32 adds per element and the svh scale one fp32
multiply (*2**-3 is exact): at most g_8 times the sum of |z^| over the block
(u = 2**-24).  The final rounding adds u_o |y| (u_o = 2**-8 for bf16, 2**-11
for fp16) plus a_o, half the subnormal spacing of the output type.

Parity status: the bound is pinned by tests/test_oracle_linear.py, which
checks that independent float32 evaluations (numpy float32 GEMMs in several
summation orders and K splits) stay inside it and that planted mistakes (a
dropped 2**-3, a flipped svh sign, a transposed tile) fall outside it; the
reference itself is pinned by the dense reconstruction
diag(suh) H W_q H diag(svh) / 128 through a single numpy matmul.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

import numpy as np

from . import format as fmt
from . import transform as tf

U_ACC = 2.0 ** -23
U_F32 = 2.0 ** -24
U_OUT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
A_OUT = {"bf16": 2.0 ** -134, "f16": 2.0 ** -25}
MIN_ROWS_FOR_COLUMNS = 8


def gamma(n: int, u: float) -> float:
    return n * u / (1.0 - n * u)


def shard_of_columns(shards: Sequence[int]) -> np.ndarray:
    """Shard index of every absolute output column."""
    return np.concatenate([np.full(w, s, dtype=np.int64) for s, w in enumerate(shards)])


@dataclass
class Reference:
    x_rot: np.ndarray     # fp16 bits [S, M, K]
    z: np.ndarray         # float64 [M, Nsel]  exact x~ @ W_q
    absdot: np.ndarray    # float64 [M, Nsel]  sum_k |x~ w|
    y: np.ndarray         # float64 [M, Nsel]  exact output
    cols: np.ndarray      # absolute column index of each selected column
    bias: bool = False    # y includes the layer's bias


def reference(trellis: np.ndarray, suh_bits: np.ndarray, svh_bits: np.ndarray,
              shards: Sequence[int], bits: int, cb: int, x_bits: np.ndarray,
              x_dtype: str = "bf16", col_blocks: Sequence[int] | None = None,
              bias_bits: np.ndarray | None = None) -> Reference:
    """fp64 reference for all columns, or for the 128-column blocks listed.

    ``trellis`` [K/16, N/16, 16*bits]; ``suh_bits`` [S, K]; ``svh_bits`` [N];
    ``x_bits`` [M, K].  Shard widths must be multiples of 128.
    """
    shards = list(shards)
    N = int(sum(shards))
    K = trellis.shape[0] * 16
    assert trellis.shape[1] * 16 == N and all(w % 128 == 0 for w in shards)
    x_rot = tf.rotate_input(x_bits, suh_bits, x_dtype)
    xr = tf.f16_from_bits(x_rot).astype(np.float64)  # [S, M, K]
    shard_col = shard_of_columns(shards)
    if col_blocks is None:
        col_blocks = range(N // 128)
    col_blocks = list(col_blocks)
    M = x_bits.shape[0]
    z = np.zeros((M, 128 * len(col_blocks)))
    a = np.zeros_like(z)
    cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in col_blocks])
    for i, b in enumerate(col_blocks):
        w = fmt.dequantize(trellis[:, 8 * b:8 * b + 8, :], bits, cb)  # [K, 128]
        s = shard_col[128 * b]
        z[:, 128 * i:128 * i + 128] = xr[s] @ w
        a[:, 128 * i:128 * i + 128] = np.abs(xr[s]) @ np.abs(w)
    y = tf.output_transform_f64(z, svh_bits[cols], None if bias_bits is None else bias_bits[cols])
    del K
    return Reference(x_rot, z, a, y, cols, bias_bits is not None)


def bound(ref: Reference, svh_bits: np.ndarray, K: int, out_dtype: str) -> np.ndarray:
    """Per-element error bound B_mn for the selected columns (see header)."""
    g_k = gamma(K, U_ACC)
    g_8 = gamma(8, U_F32)
    per = g_k * ref.absdot + g_8 * (np.abs(ref.z) + g_k * ref.absdot)  # [M, Nsel]
    M, nsel = per.shape
    blk = per.reshape(M, nsel // 128, 128).sum(axis=-1)  # [M, nblk]
    blk = np.repeat(blk, 128, axis=1)
    svh = np.abs(tf.f16_from_bits(svh_bits[ref.cols]).astype(np.float64))[None, :]
    u_o = U_OUT[out_dtype]
    scaled = tf.OUTPUT_SCALE * svh * blk
    if ref.bias:
        # the fp32 add of the bias: one more rounding of at most U_F32 of
        # the sum, whose distance from y* is at most the scaled term
        scaled = scaled + U_F32 * (np.abs(ref.y) + scaled)
    return u_o * np.abs(ref.y) + (1.0 + u_o) * scaled + A_OUT[out_dtype]


def output_stage_reference(z_parts: np.ndarray, svh_bits: np.ndarray, out_dtype: str,
                           bias_bits: np.ndarray | None = None):
    """The output stage on given fp32 K-part sums, against its plain
    definition: y* = H128(sum_p z_p) * 2**-3 * svh (+ bias) in float64, and
    the per-element bound of any fp32 evaluation that adds the P parts in
    some order and then runs the output stage of reading R11 (TensorFold PR,
    "Arithmetic" step 3: output transform, svh and 2**-3, one rounding).

    ``z_parts`` [P, M, N] float32.  Derivation as in ``bound`` with the
    K-sum replaced by the sum of P fp32 terms in any order, which errs by
    at most g_{P-1} * A, A = sum_p |z_p| (u = 2**-24, round to nearest):
        B_mn = u_o |y*| + (1 + u_o) 2**-3 |svh_n|
               * sum_{j in blk(n)} ( g_{P-1} A_mj + g_8 (|z*_mj| + g_{P-1} A_mj) ) + a_o
    (plus the bias add's one rounding, as in ``bound``).  Returns (y*, B).
    """
    z = np.asarray(z_parts, dtype=np.float64)
    P, M, N = z.shape
    zs = z.sum(axis=0)
    A = np.abs(z).sum(axis=0)
    y = tf.output_transform_f64(zs, svh_bits, bias_bits)
    g_p = gamma(max(P - 1, 0), U_F32)
    g_8 = gamma(8, U_F32)
    per = g_p * A + g_8 * (np.abs(zs) + g_p * A)
    blk = np.repeat(per.reshape(M, N // 128, 128).sum(axis=-1), 128, axis=1)
    svh = np.abs(tf.f16_from_bits(svh_bits).astype(np.float64))[None, :]
    scaled = tf.OUTPUT_SCALE * svh * blk
    if bias_bits is not None:
        scaled = scaled + U_F32 * (np.abs(y) + scaled)
    u_o = U_OUT[out_dtype]
    return y, u_o * np.abs(y) + (1.0 + u_o) * scaled + A_OUT[out_dtype]


def out_bits_to_f64(y_bits: np.ndarray, out_dtype: str) -> np.ndarray:
    if out_dtype == "bf16":
        return tf.bf16_bits_to_f32(y_bits).astype(np.float64)
    return tf.f16_from_bits(y_bits).astype(np.float64)


@dataclass
class CheckResult:
    ok: bool
    max_ratio: float          # max |y - y*| / B
    worst_col_rel: float      # max_n max_m |y - y*| / max_m |y*|
    matrix_rel: float         # max |y - y*| / max |y*|
    n_values: int

    def __str__(self) -> str:
        return (f"{'PASS' if self.ok else 'FAIL'}: {self.n_values} values, max {self.max_ratio:.4f} of "
                f"bound, worst column {self.worst_col_rel:.3e}, matrix {self.matrix_rel:.3e}")


def check(y_bits: np.ndarray, ref: Reference, svh_bits: np.ndarray, K: int, out_dtype: str,
          worst_col_limit: float = 5e-3) -> CheckResult:
    """Compare output bits (columns ``ref.cols``) against the reference."""
    y = out_bits_to_f64(y_bits, out_dtype)
    assert y.shape == ref.y.shape, (y.shape, ref.y.shape)
    if not np.all(np.isfinite(y)):
        return CheckResult(False, float("inf"), float("inf"), float("inf"), y.size)
    err = np.abs(y - ref.y)
    b = bound(ref, svh_bits, K, out_dtype)
    ratio = float(np.max(err / b)) if err.size else 0.0
    colmax = np.max(np.abs(ref.y), axis=0)
    colerr = np.max(err, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        col_rel = np.where(colmax > 0, colerr / colmax, np.where(colerr > 0, np.inf, 0.0))
    worst = float(np.max(col_rel)) if col_rel.size else 0.0
    gmax = float(np.max(np.abs(ref.y))) if ref.y.size else 0.0
    mrel = float(np.max(err) / gmax) if gmax > 0 else 0.0
    # A column's largest output over a handful of rows can sit arbitrarily
    # close to zero (the one value of a one-row call, say), where any
    # rounding is a large relative error; below MIN_ROWS_FOR_COLUMNS rows the
    # worst column is still reported but the limit applies matrix-wide.
    rel = worst if y.shape[0] >= MIN_ROWS_FOR_COLUMNS else mrel
    return CheckResult(ratio <= 1.0 and rel <= worst_col_limit, ratio, worst, mrel, int(y.size))


def dense_weight(trellis: np.ndarray, suh_bits: np.ndarray, svh_bits: np.ndarray,
                 shards: Sequence[int], bits: int, cb: int) -> np.ndarray:
    """The layer as one dense fp64 matrix, for the single-matmul cross-check.

    W[s] = diag(suh_s) H W_q H diag(svh) * 2**-7 restricted to shard s's
    columns (2**-4 * 2**-3 = 2**-7 = 1/128); returns [S, K, N] with the other
    shards' columns zero.
    """
    wq = fmt.dequantize(trellis, bits, cb)
    K, N = wq.shape
    hk = np.kron(np.eye(K // 128), tf.sylvester())
    hn = np.kron(np.eye(N // 128), tf.sylvester())
    suh = tf.f16_from_bits(suh_bits).astype(np.float64)
    svh = tf.f16_from_bits(svh_bits).astype(np.float64)
    core = hk @ wq @ hn
    shard_col = shard_of_columns(shards)
    out = np.zeros((len(shards), K, N))
    for s in range(len(shards)):
        mask = (shard_col == s).astype(np.float64)
        out[s] = (suh[s][:, None] * core * (svh * mask)[None, :]) / 128.0
    return out
