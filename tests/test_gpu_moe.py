"""GPU: routed experts as one grouped GEMM (cuda-exl3 README, "What is
supported" and "Determinism").  Synthetic routing; the alignment against the
oracle's, every routed row bit-identical to the plain linear of its token on
its expert's weight alone, the combine bit-exact against the oracle's, and the
whole path within the oracle's bound."""
import ctypes

import numpy as np
import pytest
import torch

import linear_exl3_input_amd as ex
import workloads as wl
from oracle import linear as olin
from oracle import moe as omoe
from oracle import transform as otf
from gpu_util import banner, bits16, dev16, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ex.load()
    torch.cuda.init()


def _experts(E, K, shards, bits, cb, seed, bias=False):
    lay = wl.small_layer("moe_expert", K, shards, bits, cb, (1,), seed=seed)
    rng = np.random.default_rng(seed)
    N = sum(shards)
    tr = rng.integers(0, 65536, (E, K // 16, N // 16, 16 * bits), dtype=np.uint16)
    suh = (np.where(rng.integers(0, 2, (E, len(shards), K)) == 1, -1.0, 1.0)
           * np.exp2(rng.uniform(-1, 1, (E, len(shards), K)))).astype(np.float16).view(np.uint16)
    svh = (np.where(rng.integers(0, 2, (E, N)) == 1, -1.0, 1.0)).astype(np.float16).view(np.uint16)
    b = (rng.standard_normal((E, N))).astype(np.float16).view(np.uint16) if bias else None
    w = ex.MoeWeight(dev16(tr), dev16(suh, torch.float16), dev16(svh, torch.float16), bits, cb, shards,
                     dev16(b, torch.float16) if bias else None)
    return lay, w, (tr, suh, svh, b)


def _routing(T, k, E, seed, drop=False):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    if drop:
        ids[0, 0] = -1
        ids[-1, -1] = E + 3
    wts = rng.dirichlet(np.ones(k), T).astype(np.float32)
    return ids, wts


@pytest.mark.parametrize("T,k,E,block", [(37, 4, 8, 16), (5, 8, 64, 16), (200, 2, 6, 32), (64, 1, 3, 64)])
def test_align_matches_the_oracle(T, k, E, block):
    ids, _ = _routing(T, k, E, 700 + T, drop=True)
    row_pair, block_expert, pair_row = (t.cpu().numpy() for t in ex.moe_align(torch.from_numpy(ids).cuda(), E, block))
    rows, runs, be = omoe.align_runs(ids, E, block)
    assert len(row_pair) == rows and np.array_equal(block_expert, be)
    seen = np.full(rows, False)
    for e, (start, pairs) in runs.items():
        run = row_pair[start:start + len(pairs)]
        assert sorted(run.tolist()) == sorted(pairs.tolist()), f"expert {e}"
        seen[start:start + len(pairs)] = True
    assert np.all(row_pair[~seen] == -1)
    live = pair_row >= 0
    assert np.array_equal(row_pair[pair_row[live]], np.nonzero(live)[0])
    flat = ids.reshape(-1)
    assert np.all(pair_row[(flat < 0) | (flat >= E)] == -1)


TABLE, ALU, AUTO = ex.EXL3_DECODER_TABLE, ex.EXL3_DECODER_ALU, ex.EXL3_DECODER_AUTO


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("T,k,E,block,bias,decoder", [(21, 2, 4, 16, False, AUTO), (9, 3, 5, 32, True, AUTO),
                                                      (40, 2, 3, 64, False, AUTO), (21, 2, 4, 16, False, TABLE),
                                                      (33, 3, 6, 16, True, TABLE), (12, 2, 5, 16, True, ALU)])
def test_routed_rows_equal_the_plain_linear(T, k, E, block, bias, decoder, swiglu):
    """Each live routed row has the bits of exl3_linear of its token alone on
    its expert's weight (batch and grouping invariance), on either decoder of
    the grouped GEMM: the table decoder folds the shape's tree (8 parts in 4
    groups here) in two levels inside one fused unit, the ALU tiles through
    the finishing workgroup."""
    lay, w, _ = _experts(E, 1024, (256, 256), 4, "mcg", 710 + T, bias)
    ids, wts = _routing(T, k, E, 711 + T)
    rng = np.random.default_rng(712)
    width = 2 * w.K if swiglu else w.K
    x = x_dev(otf.f32_to_bf16_bits(rng.standard_normal((T, width)).astype(np.float32)))
    route = ex.moe_align(torch.from_numpy(ids).cuda(), E, block)
    xr = ex.moe_input_transform(x, w, route, k, block, swiglu)
    y = bits16(ex.moe_linear(w, xr, route[1], block, decoder=decoder))
    pair_row = route[2].cpu().numpy()
    for p in range(T * k):
        t, e = divmod(p, k)[0], ids.reshape(-1)[p]
        we = w.expert(int(e))
        xt = x[t:t + 1]
        xr1 = ex.input_transform_swiglu(xt, we.suh) if swiglu else ex.input_transform(xt, we.suh)
        want = bits16(ex.linear(we, xr1, torch.bfloat16))
        assert np.array_equal(y[pair_row[p]], want[0]), f"pair {p} (token {t}, expert {e})"
    banner(f"moe rows T={T} k={k} E={E} block={block} decoder={decoder} swiglu={swiglu}: {T * k} routed rows "
           "bit-identical")


def test_combine_bit_exact():
    """Generated routed rows and weights (not from the GPU path): the
    combine against the oracle's fp32 ordered sum."""
    rng = np.random.default_rng(720)
    T, k, E, block, N = 30, 4, 8, 16, 384
    ids, wts = _routing(T, k, E, 721, drop=True)
    rows, runs, _ = omoe.align_runs(ids, E, block)
    pair_row = np.full(T * k, -1, dtype=np.int32)
    for e, (start, pairs) in runs.items():
        pair_row[pairs] = start + np.arange(len(pairs))
    yb = otf.f32_to_bf16_bits((rng.standard_normal((rows, N)) * 3).astype(np.float32))
    got = bits16(ex.moe_combine(x_dev(yb), torch.from_numpy(pair_row).cuda(), torch.from_numpy(wts).cuda()))
    assert np.array_equal(got, omoe.combine_bits(yb, "bf16", pair_row, wts))


@pytest.mark.parametrize("K,shards,bits,cb,E,T,k,decoder", [(1024, (256,), 5, "mul1", 6, 23, 2, AUTO),
                                                          (4096, (2048,), 4, "mcg", 8, 48, 2, AUTO),
                                                          (1024, (256, 128), 6, "3inst", 5, 30, 3, TABLE)])
def test_moe_forward_within_the_oracle_bound(K, shards, bits, cb, E, T, k, decoder):
    """out[t] against sum_j w_j * y*_j in float64 (y*_j the oracle's exact
    layer output of token t on expert j): within sum_j |w_j| (B_j + u_bf16
    |y*_j|) plus the combine's own roundings."""
    lay, w, (tr, suh, svh, _) = _experts(E, K, shards, bits, cb, 730 + K)
    ids, wts = _routing(T, k, E, 731)
    rng = np.random.default_rng(732)
    xb = otf.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    out = bits16(ex.moe_forward(x_dev(xb), w, torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda(),
                                decoder=decoder))
    got = olin.out_bits_to_f64(out, "bf16")
    N = sum(shards)
    want = np.zeros((T, N))
    lim = np.zeros((T, N))
    for e in range(E):
        toks = np.nonzero((ids == e).any(axis=1))[0]
        if toks.size == 0:
            continue
        ref = olin.reference(tr[e], suh[e], svh[e], shards, bits, {"3inst": 0, "mcg": 1, "mul1": 2}[cb], xb[toks])
        b = olin.bound(ref, svh[e], K, "bf16")
        for i, t in enumerate(toks):
            wj = float(wts[t][list(ids[t]).index(e)])
            want[t] += wj * ref.y[i]
            lim[t] += abs(wj) * (b[i] + 2.0 ** -8 * np.abs(ref.y[i]))
    lim += 2.0 ** -8 * np.abs(want) + k * 2.0 ** -23 * np.abs(want) + 2.0 ** -30
    err = np.abs(got - want)
    banner(f"moe forward K={K} E={E} T={T} k={k}: max err/limit {np.max(err / lim):.3f}")
    assert np.all(err <= lim)


@pytest.mark.parametrize("decoder", [AUTO, TABLE])
def test_out_of_range_block_experts_are_skipped(decoder):
    """A caller-built routing whose block_expert holds an expert index past
    the stack (or below -1) is treated as a padding block: the routed
    rotation writes zeros for its rows and the grouped GEMM leaves its output
    rows untouched, while the valid blocks keep their bits."""
    E, block, T, k = 3, 16, 20, 2
    lay, w, _ = _experts(E, 512, (256,), 4, "mcg", 760)
    ids, _ = _routing(T, k, E, 761)
    rng = np.random.default_rng(762)
    x = x_dev(otf.f32_to_bf16_bits(rng.standard_normal((T, w.K)).astype(np.float32)))
    row_pair, block_expert, pair_row = ex.moe_align(torch.from_numpy(ids).cuda(), E, block)
    good = block_expert.clone()
    xr_good = ex.moe_input_transform(x, w, (row_pair, good, pair_row), k, block)
    y_good = bits16(ex.moe_linear(w, xr_good, good, block))
    be = block_expert.cpu().numpy()
    live = np.nonzero(be >= 0)[0]
    assert live.size >= 3
    bad_blocks = live[:2]
    hacked = be.copy()
    hacked[bad_blocks[0]] = E
    hacked[bad_blocks[1]] = E + 1000
    hacked_dev = torch.from_numpy(hacked).cuda()
    xr = ex.moe_input_transform(x, w, (row_pair, hacked_dev, pair_row), k, block)
    xr_n = bits16(xr).reshape(w.n_shards, w.K // 32, -1, 32)
    for b in bad_blocks:
        assert np.all(xr_n[:, :, block * b:block * (b + 1)] == 0), f"block {b} not rotated as zeros"
    rows = xr.shape[2]
    y = torch.full((rows, w.N), 7.0, dtype=torch.bfloat16, device="cuda")
    L = ex.load()
    need = L.exl3_moe_workspace_bytes(ctypes.byref(w.first.view()), rows, block)
    ws, wsn = ex._workspace(need, torch.device("cuda"))
    ex._check(L.exl3_moe_linear_ex(ctypes.byref(w.first.view()), w.E, xr.data_ptr(), rows, hacked_dev.data_ptr(),
                                   block, y.data_ptr(), 1, ws, wsn, ex._stream(), decoder))
    yb = bits16(y)
    seven = bits16(torch.full((1,), 7.0, dtype=torch.bfloat16))[0]
    for b in range(len(be)):
        r = slice(block * b, block * (b + 1))
        if b in bad_blocks:
            assert np.all(yb[r] == seven), f"block {b} written"
        elif be[b] >= 0:
            assert np.array_equal(yb[r], y_good[r]), f"block {b}"


@pytest.mark.parametrize("K,N", [(4096, 2048), (2048, 4096)])
def test_grouped_table_equals_alu_on_the_expert_pair(K, N):
    """The expert pair's shapes (4-bit mcg, 32 parts in 8 groups and 16 in
    4), 64 experts, 16 tokens routed to 8 each: the grouped table decoder
    (which the automatic choice takes here) gives every live routed row the
    bits of the grouped ALU tiles."""
    E, T, k, block = 64, 16, 8, 16
    lay, w, _ = _experts(E, K, (N,), 4, "mcg", 780 + K)
    ids, _ = _routing(T, k, E, 781)
    rng = np.random.default_rng(782)
    x = x_dev(otf.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32)))
    route = ex.moe_align(torch.from_numpy(ids).cuda(), E, block)
    xr = ex.moe_input_transform(x, w, route, k, block)
    y_alu = bits16(ex.moe_linear(w, xr, route[1], block, decoder=ALU))
    y_tab = bits16(ex.moe_linear(w, xr, route[1], block, decoder=TABLE))
    y_auto = bits16(ex.moe_linear(w, xr, route[1], block))
    live = route[2].cpu().numpy()
    live = live[live >= 0]
    assert np.array_equal(y_tab[live], y_alu[live])
    assert np.array_equal(y_auto[live], y_alu[live])
    banner(f"grouped table == ALU: {K}x{N}, {live.size} routed rows over {int((route[1] >= 0).sum())} blocks")


def test_grouped_table_refusals():
    """The table decoder of the grouped GEMM takes 16-row blocks only, and
    an unknown decoder is refused before any launch."""
    E, block = 2, 32
    lay, w, _ = _experts(E, 512, (256,), 4, "mcg", 790)
    rows = 64
    xr = torch.zeros(ex.rot_shape(1, rows, 512), dtype=torch.float16, device="cuda")
    be = torch.zeros(rows // block, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="16-row blocks"):
        ex.moe_linear(w, xr, be, block, decoder=TABLE)
    with pytest.raises(RuntimeError, match="decoder=7"):
        ex.moe_linear(w, xr, be, block, decoder=7)
