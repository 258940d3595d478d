"""Seeded synthetic inputs for the EXL3 linear, shared by the CPU oracle's
tests, the GPU parity tests, ``smoke()`` and ``bench.py``.

This module holds input generation only: shapes, seeds and random draws.
It contains none of the method's arithmetic (no codebook, unpacking,
rotation, contraction or output transform), so both the oracle and the
HIP path can take their inputs from it without sharing any of the
computation they are checked on.

Every tensor is returned as raw bits in numpy arrays:

* ``trellis``  uint16 ``[K/16, N/16, 16*bits]``  -- any 16-bit pattern is a
  legal word, since every 16-bit state decodes in every codebook
  (cuda-exl3 page, "Loading into a dim vLLM has padded").
* ``suh``      uint16 fp16 bits ``[n_shards, K]``
* ``svh``      uint16 fp16 bits ``[N]``
* ``x``        uint16 bf16 bits ``[M_max, K]``; a smaller M uses the first M
  rows, so a row's value is the same at every batch size.

The workloads mirror the layer shapes the pages measure (Qwen-27B-class
q_proj / down_proj / gate_up at 5-6 bits, a GLM-class lm_head, and the
4-bit expert matrices of the TensorFold PR); the pages measured real
checkpoints, which are not available here, so seeded random tensors of the
same shapes and value ranges stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np

CODEBOOKS = ("3inst", "mcg", "mul1")
CB_ID = {name: i for i, name in enumerate(CODEBOOKS)}

TENSOR_TRELLIS, TENSOR_SUH, TENSOR_SVH, TENSOR_X = 0, 1, 2, 3


@dataclass(frozen=True)
class Layer:
    """One EXL3 linear layer: shape, bit width, codebook and shard widths."""

    name: str
    K: int
    shards: Tuple[int, ...]
    bits: int
    codebook: str
    M_values: Tuple[int, ...]
    seed_base: int

    @property
    def N(self) -> int:
        return int(sum(self.shards))

    @property
    def n_shards(self) -> int:
        return len(self.shards)

    @property
    def cb(self) -> int:
        return CB_ID[self.codebook]

    @property
    def M_max(self) -> int:
        return max(self.M_values)

    def weight_bytes(self) -> int:
        return self.K * self.N * self.bits // 8


def _seed(config: int, subshape: int, tensor: int) -> int:
    return 20260000 + 1000 * config + 100 * subshape + tensor


def _sweep_seed(bits: int, cb: int) -> int:
    return 20265000 + 100 * (10 * bits + cb)


M_SWEEP = (1, 8, 16, 24, 32, 64, 128, 256, 512)

LAYERS: List[Layer] = [
    Layer("small_1024x1024_b4_3inst", 1024, (1024,), 4, "3inst", (1, 16), _seed(1, 0, 0)),
    Layer("expert_4096x2048_b4_mcg", 4096, (2048,), 4, "mcg", (1, 16, 512), _seed(2, 0, 0)),
    Layer("expert_2048x4096_b4_mcg", 2048, (4096,), 4, "mcg", (1, 16, 512), _seed(2, 1, 0)),
    Layer("q_proj_5120x12288_b6_mul1", 5120, (12288,), 6, "mul1", M_SWEEP, _seed(3, 0, 0)),
    Layer("down_proj_17408x5120_b6_mul1", 17408, (5120,), 6, "mul1", M_SWEEP, _seed(3, 1, 0)),
    Layer("gate_up_5120x2x17408_b5_mul1", 5120, (17408, 17408), 5, "mul1", (16, 128, 2048, 4096), _seed(4, 0, 0)),
    Layer("lm_head_4096x154880_b6_mul1", 4096, (154880,), 6, "mul1", (1, 16, 512), _seed(5, 0, 0)),
]


def sweep_layer(bits: int, codebook: str) -> Layer:
    """The bit-width sweep at K=N=4096, M=64, one layer per (bits, codebook)."""
    cb = CB_ID[codebook]
    return Layer(f"sweep_4096x4096_b{bits}_{codebook}", 4096, (4096,), bits, codebook, (64,),
                 _sweep_seed(bits, cb))


SWEEP: List[Layer] = [sweep_layer(b, cb) for b in range(1, 9) for cb in ("3inst", "mcg", "mul1")]


def layer(name: str) -> Layer:
    for lay in LAYERS + SWEEP:
        if lay.name == name:
            return lay
    raise KeyError(name)


def _rng(layer: Layer, tensor: int) -> np.random.Generator:
    return np.random.default_rng(layer.seed_base + tensor)


def round_f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16 (nearest, ties to even), returning bits.

    Used only to draw bf16 activations; the inputs are finite normals.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def gen_trellis(layer: Layer, K: int | None = None, N: int | None = None) -> np.ndarray:
    K = layer.K if K is None else K
    N = layer.N if N is None else N
    rng = _rng(layer, TENSOR_TRELLIS)
    return rng.integers(0, 65536, size=(K // 16, N // 16, 16 * layer.bits), dtype=np.uint16)


def _pm1_fp16_bits(rng: np.random.Generator, shape) -> np.ndarray:
    sign = rng.integers(0, 2, size=shape, dtype=np.uint16)
    return (np.uint16(0x3C00) | (sign << np.uint16(15))).astype(np.uint16)


def _scaled_fp16_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """sign * 2**U(-2, 2) rounded to fp16: scales whose magnitudes differ."""
    sign = np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    mag = np.exp2(rng.uniform(-2.0, 2.0, size=shape))
    return (sign * mag).astype(np.float16).view(np.uint16)


def gen_suh(layer: Layer, magnitudes: bool = False) -> np.ndarray:
    rng = _rng(layer, TENSOR_SUH)
    shape = (layer.n_shards, layer.K)
    return _scaled_fp16_bits(rng, shape) if magnitudes else _pm1_fp16_bits(rng, shape)


def gen_svh(layer: Layer, magnitudes: bool = False) -> np.ndarray:
    rng = _rng(layer, TENSOR_SVH)
    shape = (layer.N,)
    return _scaled_fp16_bits(rng, shape) if magnitudes else _pm1_fp16_bits(rng, shape)


def gen_x(layer: Layer, M: int | None = None) -> np.ndarray:
    """bf16 bits [M, K]; rows are a prefix of the M_max draw."""
    rng = _rng(layer, TENSOR_X)
    full = rng.standard_normal((layer.M_max, layer.K), dtype=np.float32)
    M = layer.M_max if M is None else M
    if M > layer.M_max:
        raise ValueError(f"{layer.name}: M={M} exceeds the drawn {layer.M_max} rows")
    return round_f32_to_bf16_bits(full[:M])


def small_layer(name: str, K: int, shards: Sequence[int], bits: int, codebook: str,
                M_values: Sequence[int] = (1, 7, 16, 33), seed: int = 1) -> Layer:
    """A small layer for parity tests (sizes the oracle finishes quickly)."""
    return Layer(name, K, tuple(shards), bits, codebook, tuple(M_values), 20269000 + 10 * seed)


@dataclass
class Tensors:
    layer: Layer
    trellis: np.ndarray
    suh: np.ndarray
    svh: np.ndarray
    x: np.ndarray = field(repr=False)


def gen_all(layer: Layer, M: int | None = None, magnitudes: bool = False) -> Tensors:
    return Tensors(layer, gen_trellis(layer), gen_suh(layer, magnitudes), gen_svh(layer, magnitudes),
                   gen_x(layer, M))
