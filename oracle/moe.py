"""Oracle for the routed-expert path (test infrastructure only: imported by
the tests, never by the library).

cuda-exl3 README, "What is supported": the (token, expert) pairs are sorted
by expert and each expert's run padded to whole row blocks, so every block
belongs to one expert; "Determinism": each token's top-k routed rows are
summed in a fixed order in fp32 and rounded once.  Pair p = t * topk + j.
"""
from __future__ import annotations

import numpy as np

from . import transform as tf


def rows_max(T: int, topk: int, E: int, block: int) -> int:
    pairs = T * topk
    rows = pairs + min(E, pairs) * (block - 1)
    return (rows + block - 1) // block * block


def align_runs(topk_ids: np.ndarray, E: int, block: int):
    """-> (rows, runs, block_expert): runs[e] = (first row, the pairs of
    expert e in pair order); block_expert [rows / block], -1 after the last
    run.  Pairs whose id is outside 0..E-1 are dropped."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    T, k = np.asarray(topk_ids).shape
    rows = rows_max(T, k, E, block)
    runs, start = {}, 0
    block_expert = np.full(rows // block, -1, dtype=np.int32)
    for e in range(E):
        pairs = np.nonzero(ids == e)[0]
        padded = -(-len(pairs) // block) * block
        runs[e] = (start, pairs)
        block_expert[start // block:(start + padded) // block] = e
        start += padded
    return rows, runs, block_expert


def combine_bits(y_bits: np.ndarray, dtype: str, pair_row: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """out[t] = rne(sum_j fp32(w[t, j] * y[pair_row[t*k + j]])) summed in fp32
    from 0 in j order (dropped pairs, row -1, add nothing)."""
    T, k = weights.shape
    y = tf.bf16_bits_to_f32(y_bits) if dtype == "bf16" else tf.f16_from_bits(y_bits).astype(np.float32)
    acc = np.zeros((T, y.shape[1]), dtype=np.float32)
    w = np.asarray(weights, dtype=np.float32)
    for j in range(k):
        r = np.asarray(pair_row).reshape(T, k)[:, j]
        live = r >= 0
        term = (w[:, j:j + 1] * y[np.where(live, r, 0)]).astype(np.float32)
        acc = np.where(live[:, None], (acc + term).astype(np.float32), acc)
    return tf.f32_to_bf16_bits(acc) if dtype == "bf16" else tf.f32_to_f16_bits(acc)
