"""The two 128-point Hadamard rotations of the EXL3 linear (oracle; test
infrastructure).

Pages
-----
* Input side: x*suh, then the 128-point Hadamard transform in a fixed order
  of fp32 adds, times 2**-4 (exact), rounded once to fp16 (TensorFold PR
  "cuda: EXL3 projections behind qlinear", "Arithmetic" step 1).  suh is one
  value per input channel and one row per shard of a fused layer (cuda-exl3
  page, "Notes on the format").
* Output side: the output transform, svh and 2**-3, one rounding to bf16
  (TensorFold PR, "Arithmetic" step 3); the caller's dtype, bf16 or fp16, is
  emitted directly (cuda-exl3, "One op per layer").
* The rotation is block diagonal over 128-element blocks, so splitting the
  input dim at multiples of 128 is exact (cuda-exl3, "Tensor parallel").

Readings taken where the pages are silent
-----------------------------------------
R8  The Hadamard matrix is Sylvester's, natural order:
    H[i][j] = (-1)**popcount(i & j); H @ H = 128 I.
R9  The fp32 add order is the radix-2 butterfly with strides 1, 2, 4, ..., 64
    in ascending order; at each stage the pair (a, b) = (t[e], t[e + s]),
    e with bit s clear, becomes (a + b, a - b).  Both rotations use it.
R10 Rounding is to nearest, ties to even, everywhere; subnormals are kept.
R11 Output order: fp32 butterfly, then *2**-3 (exact), then *svh in fp32,
    then one rounding to the output dtype.  x*suh in fp32 is exact (a bf16
    times an fp16 needs 19 significant bits).

Parity status: pinned by tests/test_oracle_transform.py (H @ H = 128 I,
agreement with scipy.linalg.hadamard, the one-hot closed forms, the float32
replay within one fp16 ulp of the exact fp64 rotation, block diagonality).
The fp32 add order itself (R9) is a reading; the HIP kernels must reproduce
it bit for bit.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 128
STAGES = 7
INPUT_SCALE = 2.0 ** -4
OUTPUT_SCALE = 2.0 ** -3


def sylvester(n: int = BLOCK) -> np.ndarray:
    """Reading R8 written out element by element (float64)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(lambda a: bin(int(a)).count("1"))(i & j)
    return np.where(pc % 2 == 0, 1.0, -1.0)


def butterfly(t: np.ndarray) -> np.ndarray:
    """Reading R9: unnormalised 128-point Hadamard over the last axis.

    Runs in the dtype of ``t`` (float32 for the format's order, float64 for
    the exact reference); every add is one IEEE operation of that dtype.
    """
    t = np.array(t, copy=True)
    assert t.shape[-1] % BLOCK == 0
    lead = t.shape[:-1]
    nblk = t.shape[-1] // BLOCK
    t = t.reshape(lead + (nblk, BLOCK))
    for s in range(STAGES):
        stride = 1 << s
        v = t.reshape(lead + (nblk, BLOCK // (2 * stride), 2, stride))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        t = v.reshape(lead + (nblk, BLOCK))
    return t.reshape(lead + (nblk * BLOCK,))


# ---------------------------------------------------------------------------
# bit helpers (fp16 / bf16 <-> float)
# ---------------------------------------------------------------------------

def f16_from_bits(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bits -> float32 (exact: bf16 is the top half of a float32)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (R10).

    Finite inputs only (the linear produces no inf/NaN on finite inputs).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> fp16 bits, round to nearest, ties to even (numpy's cast)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def x_to_f32(x_bits: np.ndarray, x_dtype: str) -> np.ndarray:
    if x_dtype == "bf16":
        return bf16_bits_to_f32(x_bits)
    if x_dtype == "f16":
        return f16_from_bits(x_bits).astype(np.float32)
    raise ValueError(x_dtype)


# ---------------------------------------------------------------------------
# Input rotation
# ---------------------------------------------------------------------------

def rotate_input(x_bits: np.ndarray, suh_bits: np.ndarray, x_dtype: str = "bf16") -> np.ndarray:
    """x~ = fp16( H128(x*suh) * 2**-4 ), in the format's fp32 order.

    x_bits [M, K] (bf16 or fp16 bits), suh_bits [S, K] fp16 bits.
    Returns fp16 bits [S, M, K]: one rotated copy of x per shard.
    """
    x32 = x_to_f32(x_bits, x_dtype)
    suh32 = f16_from_bits(suh_bits).astype(np.float32)
    out = []
    for s in range(suh32.shape[0]):
        t = x32 * suh32[s][None, :]  # exact in float32 (R11)
        h = butterfly(t.astype(np.float32))
        out.append(f32_to_f16_bits(h * np.float32(INPUT_SCALE)))
    return np.stack(out, axis=0)


def rotate_input_f64(x_bits: np.ndarray, suh_bits: np.ndarray, x_dtype: str = "bf16") -> np.ndarray:
    """The exact rotation H128(x*suh)*2**-4 in float64 (no rounding), [S, M, K]."""
    x64 = x_to_f32(x_bits, x_dtype).astype(np.float64)
    suh64 = f16_from_bits(suh_bits).astype(np.float64)
    return np.stack([butterfly(x64 * suh64[s][None, :]) * INPUT_SCALE
                     for s in range(suh64.shape[0])], axis=0)


# ---------------------------------------------------------------------------
# Output transform
# ---------------------------------------------------------------------------

def output_transform_f32(z32: np.ndarray, svh_bits: np.ndarray, out_dtype: str,
                         bias_bits: np.ndarray | None = None) -> np.ndarray:
    """Reading R11 in float32: butterfly, *2**-3, *svh, one rounding.  The
    format's optional bias (cuda-exl3 README, "VRAM": trellis, suh/svh and
    bias are what is stored) is added in float32 right before that rounding
    (reading R16: one rounding for the whole output stage).

    z32 [M, N] float32 -> output bits [M, N] (bf16 or fp16).
    """
    h = butterfly(np.asarray(z32, dtype=np.float32))
    h = h * np.float32(OUTPUT_SCALE)
    y = h * f16_from_bits(svh_bits).astype(np.float32)[None, :]
    if bias_bits is not None:
        y = y + f16_from_bits(bias_bits).astype(np.float32)[None, :]
    if out_dtype == "bf16":
        return f32_to_bf16_bits(y)
    if out_dtype == "f16":
        return f32_to_f16_bits(y)
    raise ValueError(out_dtype)


def output_transform_f64(z64: np.ndarray, svh_bits: np.ndarray, bias_bits: np.ndarray | None = None) -> np.ndarray:
    """Exact output transform in float64: H128(z) * 2**-3 * svh (+ bias)."""
    h = butterfly(np.asarray(z64, dtype=np.float64))
    y = h * OUTPUT_SCALE * f16_from_bits(svh_bits).astype(np.float64)[None, :]
    if bias_bits is not None:
        y = y + f16_from_bits(bias_bits).astype(np.float64)[None, :]
    return y


def reduce_parts_f32(parts: np.ndarray, groups: int | None = None) -> np.ndarray:
    """Ordered fp32 sum of K-part partials.

    With ``groups`` = G (default P, one part per group): the P/G consecutive
    parts of each group are added in part order, then the G group sums in
    group order, each fold taking its first term as is (no 0 + p0).  With
    G = P this is ((p0 + p1) + p2) + ..., the "last part adds the parts in
    part order" of the TensorFold PR ("Arithmetic"); the grouped tree is the
    library's reading for small layers, fixed by the shape like P itself.

    ``parts`` [P, M, N] float32.
    """
    P = parts.shape[0]
    G = P if groups is None else groups
    if G < 1 or P % G:
        raise ValueError(f"{G} groups do not divide {P} parts")
    q = P // G
    total = None
    for gi in range(G):
        gsum = np.array(parts[gi * q], dtype=np.float32, copy=True)
        for p in range(gi * q + 1, (gi + 1) * q):
            gsum = gsum + parts[p].astype(np.float32)
        total = gsum if total is None else total + gsum
    return total


# ------------------------------------------------- SwiGLU before the rotation
#
# Reading R17: the down projection's input transform may take the gate_up
# layer's output directly (cuda-exl3 README, "MoE throughput": SwiGLU folded
# into the down projection's input transform) and computes exactly what the
# unfused pair would: act = rne_dtype(silu(g) * u) in float32, then the
# ordinary rotation of act.  exp is spelled out so that every step is one
# IEEE float32 operation in a fixed order: Cody-Waite range reduction
# (x = n ln2 + r, ln 2 split into a 12-bit head, so n * head is exact, and a
# tail) and the degree-7 Taylor polynomial of e^r on |r| <= ln2 / 2
# (truncation below 1e-8 relative), scaled by 2^n.

EXP_LOG2E = np.float32(1.4426950408889634)
EXP_LN2_HI = np.float32(2839.0 / 4096.0)
EXP_LN2_LO = np.float32(0.6931471805599453 - 2839.0 / 4096.0)
EXP_CLAMP = np.float32(104.0)  # e^104 overflows float32, e^-104 underflows to 0
EXP_TAYLOR = [np.float32(1.0 / math.factorial(i)) for i in range(8)]


def exp_f32(x: np.ndarray) -> np.ndarray:
    """e^x in float32 by the fixed sequence above (NaN stays NaN)."""
    x = np.asarray(x, dtype=np.float32)
    x = np.where(x < -EXP_CLAMP, -EXP_CLAMP, np.where(x > EXP_CLAMP, EXP_CLAMP, x)).astype(np.float32)
    n = np.rint(x * EXP_LOG2E)
    r = (x - n * EXP_LN2_HI) - n * EXP_LN2_LO
    p = np.full_like(r, EXP_TAYLOR[7])
    for c in EXP_TAYLOR[6::-1]:
        p = p * r + c
    ni = np.where(np.isnan(n), 0, n).astype(np.int32)
    with np.errstate(over="ignore"):
        return np.ldexp(p, ni).astype(np.float32)


def silu_f32(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float32)
    return (g / (np.float32(1.0) + exp_f32(-g))).astype(np.float32)


def swiglu_bits(gate_up_bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """[M, 2K] gate_up output bits (gate = columns 0..K-1, up = K..2K-1) ->
    act [M, K] bits of the same dtype: rne_dtype(silu(g) * u) in float32."""
    a = np.asarray(gate_up_bits, dtype=np.uint16)
    K = a.shape[1] // 2
    to32 = bf16_bits_to_f32 if dtype == "bf16" else (lambda b: f16_from_bits(b).astype(np.float32))
    g, u = to32(a[:, :K]), to32(a[:, K:])
    act = (silu_f32(g) * u).astype(np.float32)
    return f32_to_bf16_bits(act) if dtype == "bf16" else f32_to_f16_bits(act)
