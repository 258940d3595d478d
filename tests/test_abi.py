"""The C-ABI library on the CPU: it loads, exports what the header declares,
plans from the shape alone, and rejects bad arguments before any HIP call.
No call here reaches a kernel launch (there is no GPU on this machine)."""
import ctypes
import os

import pytest

import linear_exl3_input_amd as ex
import workloads as wl

LIB = ex.lib_path()
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libexl3.so not built")

FAKE = 0x100000  # a 16-byte aligned address that is never dereferenced


def view(K, shards, bits, cb, trellis=FAKE, suh=FAKE, svh=FAKE):
    arr = (ctypes.c_int32 * len(shards))(*shards)
    w = ex._Weight(trellis, suh, svh, K, sum(shards), bits, cb, len(shards), arr)
    w._keep = arr
    return w


def last_error():
    return ex.load().exl3_last_error().decode()


def test_exports_every_header_symbol():
    L = ex.load()
    names = ex.header_symbols()
    assert len(names) >= 12
    for name in names:
        assert hasattr(L, name), name
    assert L.exl3_abi_version() == ex.ABI_VERSION == 6


def test_status_strings():
    L = ex.load()
    assert L.exl3_status_str(0) == b"EXL3_OK"
    assert L.exl3_status_str(3) == b"EXL3_ERR_WORKSPACE"


@pytest.mark.parametrize("K,shards,bits,cb,msg", [
    (100, (128,), 4, 1, "K=100 must be a positive multiple of 128"),
    (256, (100, 156), 4, 1, "shard 0 width 100"),
    (256, (128, 128), 9, 1, "bits=9"),
    (256, (128,), 0, 1, "bits=0"),
    (256, (128,), 4, 3, "codebook=3"),
])
def test_bad_weight_rejected(K, shards, bits, cb, msg):
    L = ex.load()
    w = view(K, shards, bits, cb)
    st = L.exl3_linear(ctypes.byref(w), FAKE, 4, FAKE, 1, None, 0, None)
    assert st == 1
    assert msg in last_error()


def test_shard_sum_mismatch_rejected():
    L = ex.load()
    w = view(256, (128, 256), 4, 1)
    w.N = 256  # shards sum to 384
    st = L.exl3_linear(ctypes.byref(w), FAKE, 4, FAKE, 1, None, 0, None)
    assert st == 1 and "sum to 384 but N=256 (off by 128)" in last_error()


def test_pointer_checks():
    L = ex.load()
    w = view(256, (128,), 4, 1, trellis=0)
    assert L.exl3_linear(ctypes.byref(w), FAKE, 4, FAKE, 1, None, 0, None) == 1
    assert "trellis is NULL" in last_error()
    w = view(256, (128,), 4, 1, trellis=FAKE + 4)
    assert L.exl3_linear(ctypes.byref(w), FAKE, 4, FAKE, 1, None, 0, None) == 1
    assert "not 16-byte aligned" in last_error()
    w = view(256, (128,), 4, 1)
    assert L.exl3_linear(ctypes.byref(w), FAKE + 2, 4, FAKE, 1, None, 0, None) == 1
    assert "x_rot" in last_error()
    assert L.exl3_linear(ctypes.byref(w), FAKE, 4, FAKE, 7, None, 0, None) == 1
    assert "y_dtype=7" in last_error()
    assert L.exl3_linear(ctypes.byref(w), FAKE, -1, FAKE, 1, None, 0, None) == 1


def test_workspace_too_small_rejected():
    L = ex.load()
    w = view(4096, (2048,), 4, 1)  # P > 1, slab mode at 16 rows
    need = L.exl3_workspace_bytes(ctypes.byref(w), 16)
    assert need > 0
    st = L.exl3_linear(ctypes.byref(w), FAKE, 16, FAKE, 1, FAKE, need - 16, None)
    assert st == 3 and "short by 16" in last_error()


def test_zero_rows_needs_nothing():
    L = ex.load()
    w = view(256, (128,), 4, 1)
    assert L.exl3_linear(ctypes.byref(w), None, 0, None, 1, None, 0, None) == 0
    assert L.exl3_input_transform(None, 1, 0, 256, FAKE, 1, None, None) == 0


def test_input_transform_checks():
    L = ex.load()
    assert L.exl3_input_transform(FAKE, 1, 4, 200, FAKE, 1, FAKE, None) == 1
    assert L.exl3_input_transform(FAKE, 1, 4, 256, FAKE, 0, FAKE, None) == 1
    assert L.exl3_input_transform(FAKE, 1, 4, 256, FAKE, 17, FAKE, None) == 1
    assert L.exl3_input_transform(FAKE, 2, 4, 256, FAKE, 1, FAKE, None) == 1
    assert L.exl3_input_transform(FAKE, 1, 4, 256, None, 1, FAKE, None) == 1


def _plan(w, M):
    p = ex._Plan()
    assert ex.load().exl3_plan_query(ctypes.byref(w), M, ctypes.byref(p)) == 0
    return p


def F(parts=-1, mode=-1, bm=-1, decoder=-1, groups=-1, unit=-1, wg_cols=-1):
    """A forced plan (fields <= 0 keep the automatic choice)."""
    return ex._Plan(parts, groups, mode, bm, decoder, unit, 0, wg_cols, 0)


CB = ex.COUNTER_BYTES


def test_parts_depend_on_shape_only():
    for lay in wl.LAYERS:
        w = view(lay.K, lay.shards, lay.bits, lay.cb)
        trees = {(_plan(w, M).parts, _plan(w, M).groups) for M in (1, 16, 64, 65, 512, 4096)}
        assert len(trees) == 1, (lay.name, trees)
        P, G = trees.pop()
        assert (lay.K // 128) % P == 0 and P % G == 0


def test_small_layers_split_groups_into_parts():
    """Fewer than 512 (column block, group) pairs: each group of 4 (or 2)
    blocks splits into parts of one block; larger layers keep one part per
    group."""
    expert = view(4096, (2048,), 4, 1)  # 16 blocks x 8 groups = 128 pairs
    p = _plan(expert, 1)
    assert (p.parts, p.groups, p.unit, p.mode, p.launches) == (32, 8, 4, ex.EXL3_MODE_SLABS, 1)
    assert p.workspace == CB + 8 * 4 * 2048 * 4
    p = _plan(expert, 512)  # group slabs, separate output kernel
    assert (p.parts, p.groups, p.unit, p.bm, p.launches) == (32, 8, 4, 256, 2)
    assert p.workspace == CB + 8 * 512 * 2048 * 4
    assert _plan(view(2048, (4096,), 4, 1), 16).parts == 16
    assert _plan(view(1024, (1024,), 4, 0), 1).parts == 8 and _plan(view(1024, (1024,), 4, 0), 1).groups == 4
    q = _plan(view(5120, (12288,), 6, 2), 32)  # 96 blocks x 5 groups: one part per group
    assert (q.parts, q.groups) == (5, 5)
    d = _plan(view(17408, (5120,), 6, 2), 32)  # 40 blocks x 17 groups
    assert (d.parts, d.groups) == (17, 17)


def test_row_chunks_keep_slabs_bounded():
    """Several parts per group at a batch whose group slabs exceed 192 MiB:
    slab mode in row chunks (one chunk's slabs in the workspace)."""
    w = view(4096, (4096,), 4, 1)  # 32 blocks x 4 groups of 4 parts
    p = _plan(w, 4096)
    assert p.mode == ex.EXL3_MODE_SLABS and p.groups == 4 and p.parts == 16
    assert p.workspace <= CB + 192 * 2 ** 20 and p.launches > 2
    L = ex.load()
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 4096, ctypes.byref(F(mode=ex.EXL3_MODE_FUSED))) == 0
    assert "fused folds one level" in last_error()


def test_plan_modes_and_workspace():
    w = view(17408, (5120,), 6, 2)
    small, big = _plan(w, 16), _plan(w, 4096)
    assert small.parts == big.parts > 1
    assert small.mode == ex.EXL3_MODE_SLABS and small.workspace == CB + small.parts * 16 * 5120 * 4
    # 4096 rows of a 89M-weight layer: dequantize once into K*N fp16, dense GEMM
    assert big.mode == ex.EXL3_MODE_FUSED and big.decoder == ex.EXL3_DECODER_DENSE
    # dequantization, then 17 parts folded in registers by the 256 x 128 kernel
    assert big.workspace == CB + 17408 * 5120 * 2 and big.launches == 2
    assert small.bm == 16 and _plan(w, 24).bm == 32 and big.bm == 256
    assert _plan(w, 2047).decoder == ex.EXL3_DECODER_ALU and _plan(w, 2048).decoder == ex.EXL3_DECODER_DENSE
    assert _plan(view(4096, (2048,), 4, 1), 4096).decoder == ex.EXL3_DECODER_ALU  # 8.4M weights
    mid = _plan(w, 512)  # 17 parts x 512 x 5120 x 4 B = 178 MB of partials: slabs of 512 rows
    assert mid.mode == ex.EXL3_MODE_SLABS and mid.bm == 512
    head = view(4096, (154880,), 6, 2)
    assert _plan(head, 1).parts == 1 and _plan(head, 1).workspace == 0


def test_forced_512_row_tile_needs_one_part_per_workgroup():
    L = ex.load()
    w = view(4096, (2048,), 4, 1)
    fused_multi = F(4, ex.EXL3_MODE_FUSED, 512, 0)
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 600, ctypes.byref(fused_multi)) == 0
    assert "bm=512" in last_error()
    slabs = F(4, ex.EXL3_MODE_SLABS, 512, 0)
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 600, ctypes.byref(slabs)) == CB + 4 * 600 * 2048 * 4
    grouped = F(4, ex.EXL3_MODE_SLABS, 512, 0, groups=2)  # units of 2 parts: two accumulator sets
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 600, ctypes.byref(grouped)) == 0
    assert "units of 2 parts" in last_error()
    single = F(1, ex.EXL3_MODE_AUTO, 512, 0)
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 600, ctypes.byref(single)) == 0
    assert L.exl3_linear_ex(ctypes.byref(w), FAKE, 600, FAKE, 1, FAKE, 1 << 30, None,
                            ctypes.byref(fused_multi)) == 2  # EXL3_ERR_UNSUPPORTED, before any launch


def test_part_sums_hook_checks_its_buffer():
    L = ex.load()
    w = view(1024, (256,), 4, 1)
    f = F(4)
    need = 4 * 4 * 256 * 4  # 4 parts x 4 rows x 256 columns x fp32
    assert L.exl3_debug_parts(ctypes.byref(w), FAKE, 3, FAKE, need - 16, None, ctypes.byref(f)) == 3
    assert "short by 16" in last_error()


def test_table_decoder_choice_and_limits():
    """M <= 64 on layers of 2^25 weights or more: the table decoder (reported
    with bm 16, 32 or 64); forcing it above 64 rows, or an unknown decoder,
    is refused before any launch."""
    L = ex.load()
    head = view(4096, (154880,), 6, 2)
    for M in (1, 8, 16):
        p = _plan(head, M)
        assert p.decoder == ex.EXL3_DECODER_TABLE and p.bm == 16, M
    for M in (17, 24, 32):
        p = _plan(head, M)
        assert p.decoder == ex.EXL3_DECODER_TABLE and p.bm == 32, M
    for M in (33, 64):
        p = _plan(head, M)
        assert p.decoder == ex.EXL3_DECODER_TABLE and p.bm == 64, M
    assert _plan(head, 65).decoder == ex.EXL3_DECODER_ALU
    qp = view(5120, (12288,), 6, 2)  # 62.9M weights: the ALU tiles up to 16 rows, the table above
    assert _plan(qp, 1).decoder == _plan(qp, 16).decoder == ex.EXL3_DECODER_ALU
    assert _plan(qp, 17).decoder == _plan(qp, 64).decoder == ex.EXL3_DECODER_TABLE
    assert _plan(view(17408, (5120,), 6, 2), 1).decoder == ex.EXL3_DECODER_TABLE  # 89M weights
    assert _plan(view(4096, (2048,), 4, 1), 1).decoder == ex.EXL3_DECODER_ALU     # 8.4M weights
    small = view(1024, (1024,), 4, 0)
    slabs = F(4, ex.EXL3_MODE_SLABS, -1, ex.EXL3_DECODER_TABLE)
    assert L.exl3_workspace_bytes_ex(ctypes.byref(small), 16, ctypes.byref(slabs)) == CB + 4 * 16 * 1024 * 4
    too_tall = F(decoder=ex.EXL3_DECODER_TABLE)
    assert L.exl3_linear_ex(ctypes.byref(small), FAKE, 65, FAKE, 1, FAKE, 1 << 30, None,
                            ctypes.byref(too_tall)) == 2  # EXL3_ERR_UNSUPPORTED
    assert "at most 64 rows" in last_error()
    unknown = F(decoder=7)
    assert L.exl3_linear_ex(ctypes.byref(small), FAKE, 4, FAKE, 1, FAKE, 1 << 30, None,
                            ctypes.byref(unknown)) == 1  # EXL3_ERR_INVALID_ARG
    assert "decoder=7" in last_error()


def test_forced_groups_checked():
    L = ex.load()
    w = view(1024, (256,), 4, 1)  # 8 blocks of 128 in K
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 4, ctypes.byref(F(4, groups=3))) == 0
    assert "groups=3 do not divide parts=4" in last_error()
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 4, ctypes.byref(F(groups=2))) == 0
    assert "needs forced parts" in last_error()
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 4, ctypes.byref(F(6, groups=3))) == 0
    assert "equal parts" in last_error()  # 6 parts of 8 blocks, grouped: unequal
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 4, ctypes.byref(F(4, groups=2))) == CB + 2 * 4 * 256 * 4
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 4, ctypes.byref(F(4, groups=2, unit=1))) == CB + 4 * 4 * 256 * 4
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 4, ctypes.byref(F(4, groups=2, unit=3))) == 0
    assert "unit=3" in last_error()


def test_epilogue_hook_checks_groups():
    L = ex.load()
    w = view(256, (256,), 4, 1)
    assert L.exl3_debug_epilogue(FAKE, 6, 4, 3, ctypes.byref(w), FAKE, 1, None) == 1
    assert "groups=4" in last_error()


def test_dense_decoder_plan_and_limits():
    """Forced decoder=2: K*N fp16 of B fragments after the counters and the
    slabs (256-byte aligned); the part-sums hook refuses it (it has no
    workspace to decode into)."""
    L = ex.load()
    w = view(1024, (384,), 4, 1)
    fused = F(1, ex.EXL3_MODE_FUSED, -1, ex.EXL3_DECODER_DENSE)
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 300, ctypes.byref(fused)) == CB + 1024 * 384 * 2
    slabs = F(4, ex.EXL3_MODE_SLABS, -1, ex.EXL3_DECODER_DENSE)
    slab_b = 4 * 20 * 384 * 4  # 4 parts x 17 rows padded to 20 x 384 columns x fp32
    assert L.exl3_workspace_bytes_ex(ctypes.byref(w), 17, ctypes.byref(slabs)) == \
        ((CB + slab_b + 255) // 256) * 256 + 1024 * 384 * 2
    assert L.exl3_debug_parts(ctypes.byref(w), FAKE, 17, FAKE, 1 << 30, None, ctypes.byref(slabs)) == 2
    assert "decoder=dense" in last_error()


def test_ruler_hooks_check_arguments():
    L = ex.load()
    assert L.exl3_debug_stream_read(FAKE, 24, FAKE, None) == 1  # not a multiple of 16
    assert "bytes=24" in last_error()
    assert L.exl3_debug_stream_read(FAKE + 8, 32, FAKE, None) == 1
    assert "not 16-byte aligned" in last_error()
    assert L.exl3_debug_mfma_loop(0, 0x3C00, FAKE, None) == 1
    assert "iters=0" in last_error()
    assert L.exl3_debug_decode_rate(ctypes.byref(view(1024, (256,), 4, 1)), None, None) == 1
    assert "out is NULL" in last_error()


def test_tuned_schedules_table():
    """exl3_tune_set records a schedule for (shape, M bucket); unforced plan
    queries and workspace sizes follow it inside the bucket and only there;
    a schedule with another tree is refused; exl3_tune_clear forgets."""
    L = ex.load()
    L.exl3_tune_clear()
    w = view(5120, (12288,), 6, 2)
    base = _plan(w, 100)
    assert base.bm == 128
    f = F(base.parts, ex.EXL3_MODE_SLABS, 64, ex.EXL3_DECODER_ALU, base.groups)
    assert L.exl3_tune_set(ctypes.byref(w), 100, ctypes.byref(f)) == 0
    for M in (65, 100, 128):  # bucket 128
        p = _plan(w, M)
        assert p.bm == 64 and p.parts == base.parts and p.decoder == ex.EXL3_DECODER_ALU, M
        assert L.exl3_workspace_bytes(ctypes.byref(w), M) == p.workspace
    assert _plan(w, 129).bm == 256 and _plan(w, 64).decoder == ex.EXL3_DECODER_TABLE  # other buckets
    other = view(5120, (12288, 128), 6, 2)  # another shard map is another shape
    assert _plan(other, 100).bm == 128
    bad = F(base.parts * 2, -1, 64, ex.EXL3_DECODER_ALU)
    assert L.exl3_tune_set(ctypes.byref(w), 100, ctypes.byref(bad)) == 1
    assert "keeps the shape's tree" in last_error()
    L.exl3_tune_clear()
    assert _plan(w, 100).bm == 128


def test_tune_checks_arguments_and_sizes():
    L = ex.load()
    w = view(5120, (12288,), 6, 2)
    p = ex._Plan()
    assert L.exl3_tune(ctypes.byref(w), 1, FAKE, 16, FAKE, 1, FAKE, 1 << 30, 0, None, ctypes.byref(p)) == 1
    assert "reps=0" in last_error()
    assert L.exl3_tune(ctypes.byref(w), 1, None, 16, FAKE, 1, FAKE, 1 << 30, 3, None, ctypes.byref(p)) == 1
    assert L.exl3_tune(ctypes.byref(w), 1, FAKE, 0, FAKE, 1, FAKE, 1 << 30, 3, None, ctypes.byref(p)) == 1
    w2 = view(5120, (12160, 128), 6, 2)  # kept alive: the copy's shard map points into it
    pair = (ex._Weight * 2)(w, w2)
    assert L.exl3_tune(pair, 2, FAKE, 16, FAKE, 1, FAKE, 1 << 30, 3, None, ctypes.byref(p)) == 1
    assert "copy 1 has another shape" in last_error()
    # the candidates at 512 rows include the dense decoder's K*N fp16
    assert L.exl3_tune_workspace_bytes(ctypes.byref(w), 512) >= CB + 5120 * 12288 * 2
    assert L.exl3_tune_workspace_bytes(ctypes.byref(w), 16) >= L.exl3_workspace_bytes(ctypes.byref(w), 16)


def test_bias_and_swiglu_transform_checks():
    L = ex.load()
    w = view(1024, (256,), 4, 1)
    w.bias = FAKE + 2  # misaligned
    assert L.exl3_workspace_bytes(ctypes.byref(w), 4) == 0
    assert "bias" in last_error() and "not 16-byte aligned" in last_error()
    w.bias = FAKE
    assert L.exl3_workspace_bytes(ctypes.byref(w), 4) > 0
    assert L.exl3_input_transform_swiglu(FAKE, 1, 4, 100, FAKE, 1, FAKE, None) == 1
    assert "K=100" in last_error()
    assert L.exl3_input_transform_swiglu(None, 1, 4, 128, FAKE, 1, FAKE, None) == 1
    assert "gate_up is NULL" in last_error()
    assert L.exl3_input_transform_swiglu(FAKE, 1, 0, 128, FAKE, 1, FAKE, None) == 0  # no rows: nothing to do


def test_moe_entry_points_check_arguments():
    L = ex.load()
    assert L.exl3_moe_rows_max(3, 2, 3, 16) == 64 and L.exl3_moe_rows_max(0, 2, 3, 16) == 0
    assert L.exl3_moe_rows_max(1000, 8, 256, 16) == ((8000 + 256 * 15 + 15) // 16) * 16
    assert L.exl3_moe_align(FAKE, 4, 2, 8, 24, FAKE, FAKE, FAKE, None) == 1
    assert "block=24" in last_error()
    assert L.exl3_moe_align(FAKE, 4, 2, 5000, 16, FAKE, FAKE, FAKE, None) == 1
    w = view(1024, (256,), 4, 1)
    assert L.exl3_moe_linear(ctypes.byref(w), 4, FAKE, 40, FAKE, 16, FAKE, 1, FAKE, 1 << 30, None) == 1
    assert "multiple of block=16" in last_error()
    assert L.exl3_moe_workspace_bytes(ctypes.byref(w), 64, 16) > 0
    assert L.exl3_moe_input_transform(FAKE, 1, 0, 3, 1024, FAKE, 1, 3, FAKE, FAKE, 2, 16, 48, FAKE, None) == 1
    assert "rows=48" in last_error()  # 3 tokens x 2 of 3 experts in blocks of 16: 64 routed rows
    assert L.exl3_moe_combine(FAKE, 1, FAKE, FAKE, 2, 2, 7, FAKE, None) == 1


def test_finisher_needs_slabs_under_two_gib():
    """The finishing workgroup addresses slabs with 32-bit offsets: a forced
    plan whose slabs reach 2 GiB sums them in the second kernel (64-bit
    addresses) instead; the same plan with small slabs keeps one launch."""
    L = ex.load()
    w = view(16384, (154880,), 4, 1)
    f = F(128, ex.EXL3_MODE_SLABS, 64, 0, unit=1)
    p = ex._Plan()
    assert L.exl3_plan_query_ex(ctypes.byref(w), 64, ctypes.byref(f), ctypes.byref(p)) == 0
    assert p.workspace >= 2 ** 31 and p.launches == 2
    small = view(16384, (1024,), 4, 1)
    assert L.exl3_plan_query_ex(ctypes.byref(small), 64, ctypes.byref(f), ctypes.byref(p)) == 0
    assert p.workspace < 2 ** 31 and p.launches == 1
    # the unforced query is the automatic plan
    q = ex._Plan()
    assert L.exl3_plan_query_ex(ctypes.byref(w), 64, None, ctypes.byref(q)) == 0
    assert (q.parts, q.mode, q.bm) == (_plan(w, 64).parts, _plan(w, 64).mode, _plan(w, 64).bm)


def test_wide_layers_keep_k_whole():
    """From 256 column blocks a layer is one K part at every M (gate_up's
    34816 columns, the lm_head's 154880); below, the split rule holds."""
    for K, shards, bits in ((5120, (17408, 17408), 5), (4096, (154880,), 6), (5120, (32768,), 4)):
        w = view(K, shards, bits, 2)
        for M in (1, 16, 128, 2048):
            assert (_plan(w, M).parts, _plan(w, M).groups) == (1, 1), (K, shards, M)
    assert _plan(view(5120, (32640,), 4, 2), 1).parts > 1  # 255 blocks


def test_forward_workspace_keeps_the_counters():
    """Where exl3_forward stages x_rot in the workspace, x_rot lies after the
    plan's workspace and after the arrival counters, also for a plan that
    needs no workspace of its own (one part over all of K): the counters stay
    zero for the next call that shares the workspace."""
    L = ex.load()
    for K, shards, bits, cb, M in ((1024, (32768,), 4, 0, 16), (1024, (32768,), 4, 0, 300),
                                   (4096, (2048,), 4, 1, 512), (2048, (640,), 3, 0, 64)):
        w = view(K, shards, bits, cb)
        need = L.exl3_forward_workspace_bytes(ctypes.byref(w), M)
        p = _plan(w, M)
        x_rot = len(shards) * M * K * 2
        if need == p.workspace:  # the rotation runs in the GEMM
            continue
        assert need >= max(p.workspace, CB) + x_rot, (K, shards, M, need, p.workspace)
    w = view(1024, (32768,), 4, 0)
    assert _plan(w, 16).workspace == 0  # the case that needs the rule
    assert L.exl3_forward_workspace_bytes(ctypes.byref(w), 16) == CB + 16 * 1024 * 2


def test_forward_rotates_in_the_gemm_only_when_short():
    """exl3_forward rotates inside the small-tile GEMM while a tile's rows
    times the stages of a quad stay within 16, else stages x_rot."""
    L = ex.load()
    sweep = view(4096, (4096,), 4, 1)  # two stages a quad on 16-row tiles
    expert = view(4096, (2048,), 4, 1)  # one stage a quad
    for w, M, fused in ((sweep, 1, True), (sweep, 8, True), (sweep, 9, False), (sweep, 64, False),
                        (expert, 16, True), (expert, 17, False)):
        need = L.exl3_forward_workspace_bytes(ctypes.byref(w), M)
        assert (need == _plan(w, M).workspace) == fused, (M, need, _plan(w, M).workspace)


def test_dense_gemm_splits_the_last_round():
    """The dense GEMM runs its 256 x 256 tiles over whole rounds of the CUs
    (256 without a GPU) and, when the last round's tiles fit one round as
    twice as many 256 x 128 tiles, those columns in a second launch."""
    gu = view(5120, (17408, 17408), 5, 2)  # 136 column tiles
    for M, launches in ((2048, 3), (4096, 3), (2304, 2), (2560, 3)):
        # 2048: 1088 tiles, 64 past 4 rounds -> 8 column tiles as 128 narrow;
        # 4096: 2176, 128 past 8 -> 256 narrow; 2304 (9 row tiles): 200 past
        # 4 rounds need 23 column tiles = 414 narrow workgroups > 256: no
        # split; 2560 (10 row tiles): 1360, 80 past 5 -> 8 tiles, 160 narrow
        p = _plan(gu, M)
        assert p.decoder == ex.EXL3_DECODER_DENSE and p.launches == launches, (M, p.launches)
    q = view(5120, (12288,), 6, 2)  # 48 column tiles x 16 row tiles = 768: 3 whole rounds
    assert _plan(q, 4096).launches == 2


def test_forward_argument_checks():
    """exl3_forward validates every argument before any HIP call: dtypes, M,
    the x and y pointers, suh, and a workspace short of
    exl3_forward_workspace_bytes (staged and rotated-in-GEMM plans)."""
    L = ex.load()
    w = view(4096, (2048,), 4, 1)
    need = L.exl3_forward_workspace_bytes(ctypes.byref(w), 16)
    assert need > 0
    assert L.exl3_forward(ctypes.byref(w), FAKE, 7, 16, FAKE, 1, FAKE, need, None) == 1
    assert "x_dtype=7" in last_error()
    assert L.exl3_forward(ctypes.byref(w), FAKE, 1, 16, FAKE, 3, FAKE, need, None) == 1
    assert "y_dtype=3" in last_error()
    assert L.exl3_forward(ctypes.byref(w), FAKE, 1, -1, FAKE, 1, FAKE, need, None) == 1
    assert L.exl3_forward(ctypes.byref(w), None, 1, 16, FAKE, 1, FAKE, need, None) == 1
    assert "x" in last_error()
    assert L.exl3_forward(ctypes.byref(w), FAKE + 2, 1, 16, FAKE, 1, FAKE, need, None) == 1
    assert L.exl3_forward(ctypes.byref(w), FAKE, 1, 16, None, 1, FAKE, need, None) == 1
    assert "y" in last_error()
    assert L.exl3_forward(ctypes.byref(w), FAKE, 1, 16, FAKE, 1, FAKE, need - 16, None) == 3
    assert "short by 16" in last_error()
    assert L.exl3_forward(ctypes.byref(w), FAKE, 1, 16, FAKE, 1, FAKE + 8, need, None) == 1
    assert "aligned" in last_error()
    nosuh = view(4096, (2048,), 4, 1, suh=0)
    assert L.exl3_forward(ctypes.byref(nosuh), FAKE, 1, 16, FAKE, 1, FAKE, need, None) == 1
    assert "suh" in last_error()
    staged = view(1024, (32768,), 4, 0)  # no workspace of its own: x_rot after the counters
    n2 = L.exl3_forward_workspace_bytes(ctypes.byref(staged), 16)
    assert L.exl3_forward(ctypes.byref(staged), FAKE, 1, 16, FAKE, 1, FAKE, n2 - 2, None) == 3
    assert L.exl3_forward(ctypes.byref(w), None, 1, 0, None, 1, None, 0, None) == 0  # zero rows: nothing


def test_dense_gemm_hook_checks():
    """exl3_debug_dense_gemm validates which, y_dtype, M, its pointers and
    the fragment bytes, and refuses plans that are not one part fused."""
    L = ex.load()
    gu = view(5120, (17408, 17408), 5, 2)
    nbytes = 5120 * 34816 * 2
    bulk = ctypes.c_int32(-1)
    assert L.exl3_debug_dense_gemm(ctypes.byref(gu), FAKE, nbytes, FAKE, 2048, FAKE, 1, 0, ctypes.byref(bulk),
                                   None) == 1
    assert "which=0" in last_error()
    assert L.exl3_debug_dense_gemm(ctypes.byref(gu), FAKE, nbytes, FAKE, 2048, FAKE, 5, 3, None, None) == 1
    assert "y_dtype=5" in last_error()
    assert L.exl3_debug_dense_gemm(ctypes.byref(gu), FAKE, nbytes, FAKE, 0, FAKE, 1, 3, None, None) == 1
    assert L.exl3_debug_dense_gemm(ctypes.byref(gu), None, nbytes, FAKE, 2048, FAKE, 1, 3, None, None) == 1
    assert "frags" in last_error()
    assert L.exl3_debug_dense_gemm(ctypes.byref(gu), FAKE, nbytes - 2, FAKE, 2048, FAKE, 1, 3, None, None) == 3
    assert "short by 2" in last_error()
    down = view(17408, (5120,), 6, 2)  # 17 parts folded in registers: not one part a workgroup
    assert L.exl3_debug_dense_gemm(ctypes.byref(down), FAKE, 17408 * 5120 * 2, FAKE, 4096, FAKE, 1, 3, None,
                                   None) == 2
    assert "one-part fused" in last_error()
    assert bulk.value == -1  # nothing written on a refused call
