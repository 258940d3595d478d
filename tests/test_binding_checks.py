"""The Python binding rejects caller-supplied buffers whose size does not
match what the kernels write or read, before any HIP call: an `out` tensor
smaller than the result would otherwise be written past its end.  CPU only
(the checks run before a device pointer is taken)."""
import os
from types import SimpleNamespace

import pytest
import torch

import linear_exl3_input_amd as ex

pytestmark = pytest.mark.skipif(not os.path.exists(ex.lib_path()), reason="libexl3.so not built")

K, N = 256, 384


def fake_weight(n_shards=1):
    return SimpleNamespace(K=K, N=N, n_shards=n_shards)


def x_rot(M, n_shards=1):
    return torch.zeros(ex.rot_shape(n_shards, M, K), dtype=torch.float16)


@pytest.mark.parametrize("shape", [(3, N), (4, N - 16), (1, N), (4, N, 1), (5, N)])
def test_linear_out_of_the_wrong_shape_is_refused(shape):
    out = torch.empty(shape, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out has shape"):
        ex.linear(fake_weight(), x_rot(4), torch.bfloat16, out=out)


def test_linear_out_of_the_right_shape_passes_the_shape_check():
    # the next check is the device one: this tensor lives on the CPU
    out = torch.empty((4, N), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        ex.linear(fake_weight(), x_rot(4), torch.bfloat16, out=out)


def test_linear_out_of_the_wrong_dtype_is_refused_before_the_device_check():
    out = torch.empty((4, N), dtype=torch.float32)
    with pytest.raises(ValueError):
        ex.linear(fake_weight(), x_rot(4), torch.bfloat16, out=out)


def test_debug_epilogue_out_shape_is_checked():
    z = torch.zeros((2, 2, N, 4), dtype=torch.float32)  # P = 2 slabs of M = 8 rows
    with pytest.raises(ValueError, match="out has shape"):
        ex.debug_epilogue(fake_weight(), z, 8, out=torch.empty((7, N), dtype=torch.bfloat16))


@pytest.mark.parametrize("fn", ["stream", "mfma"])
def test_ruler_outputs_must_hold_every_word(fn):
    short = torch.empty(ex.RULER_WORDS - 1, dtype=torch.int32 if fn == "stream" else torch.float32)
    with pytest.raises(ValueError, match="out has shape"):
        if fn == "stream":
            buf = torch.zeros(1024, dtype=torch.int32)
            # the stream ruler checks its input first: hand it a stand-in
            # that passes as a device tensor
            buf = SimpleNamespace(is_cuda=True, is_contiguous=lambda: True, numel=lambda: 1024,
                                  element_size=lambda: 4, data_ptr=lambda: 0x100000)
            ex.debug_stream_read(buf, out=short)
        else:
            ex.debug_mfma_loop(1, out=short)


def test_decode_rate_out_shape_is_checked():
    with pytest.raises(ValueError, match="out has shape"):
        ex.debug_decode_rate(fake_weight(), out=torch.empty((K // 128, N // 128 + 1), dtype=torch.int32))


def test_moe_linear_needs_one_expert_per_row_block():
    w = SimpleNamespace(K=K, N=N, n_shards=1, E=4)
    block_expert = torch.zeros(3, dtype=torch.int32)  # 64 rows / 16 = 4 blocks expected
    with pytest.raises(ValueError, match="block_expert has 3 entries"):
        ex.moe_linear(w, x_rot(64), block_expert, block=16)


def test_moe_linear_checks_the_rotated_shape():
    w = SimpleNamespace(K=K, N=N, n_shards=2, E=4)
    with pytest.raises(ValueError, match="x_rot shape"):
        ex.moe_linear(w, x_rot(64, n_shards=1), torch.zeros(4, dtype=torch.int32), block=16)


def test_moe_input_transform_checks_the_route_sizes():
    T, topk, E, block = 5, 2, 4, 16
    rows = ex.moe_rows_max(T, topk, E, block)
    w = SimpleNamespace(K=K, N=N, n_shards=1, E=E, stack=(None, None, None, None))
    x = torch.zeros((T, K), dtype=torch.bfloat16)
    route = (torch.zeros(rows - 1, dtype=torch.int32), torch.zeros(rows // block, dtype=torch.int32), None)
    with pytest.raises(ValueError, match="route has"):
        ex.moe_input_transform(x, w, route, topk, block)


def test_moe_combine_checks_pair_row_length():
    y = torch.zeros((32, N), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="pair_row has 9 entries"):
        ex.moe_combine(y, torch.zeros(9, dtype=torch.int32), torch.zeros((5, 2), dtype=torch.float32))
