#!/usr/bin/env python3
"""Benchmark of the EXL3 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path -- the input rotation and the
trellis GEMM with its output transform, one exl3_forward call each -- over
every (shape, M) of the workload, each on its own copy of the weights drawn
from a pool larger than the GPU's caches (so every step reads its trellis
from HBM, as a real model step does).  The default workload, ``all_configs``, is every configuration
of the metric in one step (57 calls): the 1024 x 1024 4-bit 3inst layer at
1 and 16 rows; the 4-bit mcg expert pair (4096 x 2048, 2048 x 4096) at 1,
16 and 512; the Qwen-27B-shaped 6-bit mul1 q_proj (5120 x 12288) and
down_proj (17408 x 5120) at 1 .. 512 rows; the fused 5-bit mul1 gate_up
(5120 x 2 x 17408) at 16 .. 4096 rows; the 6-bit mul1 lm_head (4096 x
154880) at 1, 16 and 512; and the bit-width sweep (4096 x 4096, 1-8 bits,
every codebook) at 64 rows.

The timed region replays a HIP graph per step (the small calls are
launch-bound), bracketed by synchronizations; ``value`` is the aggregate
fraction of speed of light, 100 * sum(SoL) / measured time, with
SoL = max(K*N*bits/8 / 8 TB/s, 2*M*K*N / 2.5 PFLOP/s) per call.

Afterwards every call class is timed alone with HIP events on its launch
stream (the queue is pre-filled by a spin kernel so no host gap falls
between an event pair); those per-launch durations give the per-shape GB/s,
TFLOP/s and %SoL and the roofline of the dominant kernel.  The CPU oracle is
timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_BPS = 8.0e12
MFMA_F16_FLOPS = 2.5e15

M_SWEEP = (1, 8, 16, 24, 32, 64, 128, 256, 512)
SWEEP_LAYERS = [f"sweep_4096x4096_b{b}_{cb}" for b in range(1, 9) for cb in ("3inst", "mcg", "mul1")]
# Each workload is a list of (layer, row counts); a step runs every (layer, M).
WORKLOADS = {
    # every configuration of the metric in one step: the 1024 x 1024 3inst
    # layer, the 4-bit mcg expert pair, the Qwen-27B-shaped q_proj and
    # down_proj over the continuous-batching sweep, the fused gate_up pair up
    # to 4096 rows, the lm_head, and the bit-width sweep at 64 rows
    "all_configs": ([("small_1024x1024_b4_3inst", (1, 16)),
                     ("expert_4096x2048_b4_mcg", (1, 16, 512)), ("expert_2048x4096_b4_mcg", (1, 16, 512)),
                     ("q_proj_5120x12288_b6_mul1", M_SWEEP), ("down_proj_17408x5120_b6_mul1", M_SWEEP),
                     ("gate_up_5120x2x17408_b5_mul1", (16, 128, 2048, 4096)),
                     ("lm_head_4096x154880_b6_mul1", (1, 16, 512))]
                    + [(n, (64,)) for n in SWEEP_LAYERS]),
    "expert_4096x2048+2048x4096_b4_mcg": [("expert_4096x2048_b4_mcg", (1, 16, 512)),
                                          ("expert_2048x4096_b4_mcg", (1, 16, 512))],
    "small_1024x1024_b4_3inst": [("small_1024x1024_b4_3inst", (1, 16))],
    "qwen27b_q_down_b6_mul1": [("q_proj_5120x12288_b6_mul1", M_SWEEP), ("down_proj_17408x5120_b6_mul1", M_SWEEP)],
    "gate_up_5120x2x17408_b5_mul1": [("gate_up_5120x2x17408_b5_mul1", (16, 128, 2048, 4096))],
    "lm_head_4096x154880_b6_mul1": [("lm_head_4096x154880_b6_mul1", (1, 16, 512))],
    # bit-width sweep: K = N = 4096 at 64 rows, 1..8 bits, every codebook
    "sweep_4096x4096_b1-8_all_cb": [(n, (64,)) for n in SWEEP_LAYERS],
}
DEFAULT_WORKLOAD = "all_configs"
# Routed experts (grouped GEMM): the expert pair's shapes, 64 experts each,
# top-8 synthetic routing, T tokens per call.
MOE_WORKLOADS = {"moe_e64_top8_4096x2048+2048x4096_b4_mcg":
                 (["expert_4096x2048_b4_mcg", "expert_2048x4096_b4_mcg"], 64, 8, (1, 4, 16, 64))}

# Sources each kernel family is built from (its file and what it includes):
# a stored counter figure is used only while these files are unchanged.
KERNEL_SOURCES = {
    "dense": ["gemm_dense.hip", "exl3_gemm_dense.hpp", "exl3_gemm.hpp", "exl3_device.hpp", "exl3_launch.hpp"],
    "tile": ["exl3_gemm.hpp", "exl3_gemm_wide.hpp", "exl3_device.hpp", "exl3_launch.hpp"],
    "table": ["exl3_gemm_lut.hpp", "exl3_gemm.hpp", "exl3_device.hpp", "exl3_launch.hpp"],
    "misc": ["exl3_misc.hip", "exl3_gemm.hpp", "exl3_device.hpp", "exl3_launch.hpp"],
}


def sol_seconds(M, K, N, bits):
    return max(K * N * bits / 8 / HBM_BPS, 2.0 * M * K * N / MFMA_F16_FLOPS)


def kernel_key(lay, plan) -> str:
    """The GEMM template instance a call launches (what rocprof's per-kernel
    statistics group by): tile family and rows, width, codebook, part fold
    in registers, quads of waves (the host's rule, mirrored)."""
    bm, unit = plan["bm"], plan["unit"]
    cb = {"3inst": 0, "mcg": 1, "mul1": 2}[lay.codebook]
    if plan.get("decoder") == 1:
        return f"exl3::gemm_table_kernel<{lay.bits}, {cb}u, 2>"
    if plan.get("decoder") == 2:
        return "exl3::gemm_dense_kernel<true>" if unit > 1 else "exl3::gemm_dense_wide_kernel"
    quads = unit if (bm <= 64 and unit in (2, 4) and (lay.K // 128) % plan["parts"] == 0) else 1
    multi = unit > 1 and quads == 1
    if bm <= 64:
        qw = plan["wg_cols"] // 32
        name = f"exl3::gemm_kernel<{lay.bits}, {cb}u, {bm // 16}, {str(multi).lower()}, {quads}, {qw}, false>"
    elif bm == 128 and not multi:
        name = f"exl3::gemm_wide_kernel<{lay.bits}, {cb}u, 64, false, 1>"
    elif bm == 128:
        name = f"exl3::gemm_big_kernel<{lay.bits}, {cb}u, 8, true>"
    elif bm == 512:
        name = f"exl3::gemm_wide4_kernel<{lay.bits}, {cb}u>"
    else:
        name = f"exl3::gemm_wide_kernel<{lay.bits}, {cb}u, {bm // 2}, {str(multi).lower()}, 1>"
    return name


def kernel_family(key: str) -> str:
    if "dense" in key:
        return "dense"
    if "table" in key:
        return "table"
    if "gemm" in key:
        return "tile"
    return "misc"


def kernel_hash(family: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "linear_exl3_input_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_info():
    """The host CPU's model name and the cores this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, avail


def cpu_baseline(calls_spec, budget_s=24.0):
    """The oracle, as it stands, on a bounded sample of the same step: every
    (layer, M) call, each on as many 128-column blocks as its share of the
    time budget allows, scaled up to the full call."""
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import linear as olin

    calls = [(wl.layer(n), M) for n, Ms in calls_spec for M in Ms]
    share = budget_s / len(calls)
    total = 0.0
    parts = []
    for lay, M in calls:
        t = wl.gen_all(lay, M=M)
        nblk = lay.N // 128
        blocks, spent, per_block = 1, 0.0, None
        while True:
            s0 = time.perf_counter()
            olin.reference(t.trellis, t.suh, t.svh, lay.shards, lay.bits, lay.cb, t.x,
                           col_blocks=list(range(blocks)))
            dt = time.perf_counter() - s0
            spent += dt
            per_block = dt / blocks
            if spent > share / 2 or blocks >= nblk:
                break
            blocks = min(nblk, max(2 * blocks, int(share / 2 / max(per_block, 1e-4))))
        full = per_block * nblk
        total += full
        parts.append(f"{lay.name} M={M}: {blocks}/{nblk} blocks -> {full:.2f} s")
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    model, avail = cpu_info()
    sol = sum(sol_seconds(M, l.K, l.N, l.bits) for l, M in calls)
    return {
        "value": 100.0 * sol / total,
        "unit": "% of SoL (aggregate over the step)",
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": model,
        "cores_available": int(avail),
        "sample": ("fp64 oracle (decode, rotation, GEMM, output transform) per call on a prefix of its "
                   "128-column blocks, scaled to the whole call, BLAS on the stated threads; " + "; ".join(parts)
                   + f"; step total {total:.2f} s"),
        "seconds_per_step": total,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS) + sorted(MOE_WORKLOADS))
    ap.add_argument("--pool-mb", type=int, default=640, help="weight pool size (defeats the 256 MB cache)")
    ap.add_argument("--timing-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--only", default=None, metavar="LAYER:M",
                    help="counter runs: launch only this call class (its forward call), --steps times")
    ap.add_argument("--tune", action="store_true",
                    help="time every schedule of each call's part tree on the weight pool first (same bits) and "
                         "run the fastest")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="counter runs: copy MB of device memory --steps times (a kernel of known bytes)")
    ap.add_argument("--mfma-calibration", type=int, default=0, metavar="ITERS",
                    help="counter runs: the matrix-core ruler (ITERS rounds, a kernel of known MFMA count) --steps "
                         "times")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this EXL3 linear runs on one GPU only "
              "(the multi-GPU sharding is a design note, not built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import linear_exl3_input_amd as ex
    import workloads as wl

    ex.load()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in MOE_WORKLOADS:
        return moe_main(args, ex, wl, torch, np, dev)
    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration} MiB x {args.steps}")
        return
    if args.mfma_calibration:
        out = torch.empty(ex.RULER_WORDS, dtype=torch.float32, device=dev)
        for _ in range(args.steps):
            ex.debug_mfma_loop(args.mfma_calibration, out=out)
        torch.cuda.synchronize()
        log(f"mfma ruler x {args.steps}: {ex.mfma_loop_flops(args.mfma_calibration) / 16384:.0f} MFMAs each")
        return
    spec = list(WORKLOADS[args.workload])
    if args.only:
        oname, oM = args.only.split(":")
        spec = [(oname, (int(oM),))]
    layers = [wl.layer(n) for n, _ in spec]
    Ms_of = [tuple(Ms) for _, Ms in spec]
    calls = [(li, M) for li in range(len(layers)) for M in Ms_of[li]]

    def d16(a, dt=torch.int16):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)

    # ---- inputs resident in HBM: per layer a pool of weight copies at least
    # --pool-mb large (so calls cycling through it stream the trellis from
    # HBM, not from the 256 MB cache), and at least one copy per call of
    # the layer in a step (so no call of a step finds the previous call's
    # weights in cache)
    per_layer = []
    pool_bytes = 0
    for li, lay in enumerate(layers):
        Ms = Ms_of[li]
        M_max = max(Ms)
        t = wl.gen_all(lay, M=M_max)
        tr = d16(t.trellis)
        copies = min(2048, max(len(Ms), int(math.ceil(args.pool_mb * 2 ** 20 / lay.weight_bytes()))))
        pool = [tr] + [tr.clone() for _ in range(copies - 1)]
        pool_bytes += copies * lay.weight_bytes()
        suh, svh = d16(t.suh, torch.float16), d16(t.svh, torch.float16)
        ws = [ex.Exl3Weight(p_, suh, svh, lay.bits, lay.codebook, lay.shards) for p_ in pool]
        x = d16(t.x, torch.bfloat16)
        xr = {M: torch.empty(ex.rot_shape(lay.n_shards, M, lay.K), dtype=torch.float16, device=dev) for M in Ms}
        y = {M: torch.empty((M, lay.N), dtype=torch.bfloat16, device=dev) for M in Ms}
        per_layer.append((lay, ws, x, xr, y))
        del t
    log(f"workload {args.workload}: {len(layers)} layers, {len(calls)} calls per step, weight pools "
        f"{pool_bytes / 2 ** 30:.1f} GiB")
    tuned = {}
    if args.tune:
        ex.tune_clear()
        for li, M in calls:
            lay, ws, x, xr, y = per_layer[li]
            ex.input_transform(x[:M], ws[0].suh, out=xr[M])
            tuned[f"{lay.name} M={M}"] = ex.tune(ws, xr[M], reps=max(3, min(20, len(ws))))
            log(f"tuned {lay.name} M={M}: {tuned[f'{lay.name} M={M}']}")
    # workspace for the largest need (forward's, which holds x_rot where the
    # rotation does not run in the GEMM), allocated before capture
    need = max(max(ex.workspace_bytes(per_layer[li][1][0], M), ex.forward_workspace_bytes(per_layer[li][1][0], M))
               for li, M in calls)
    stream = torch.cuda.Stream()
    if need:
        ex.reserve_workspace(need, dev, stream)

    def call(li, M, copy):
        # the whole layer in one call: the rotation inside the small-tile
        # GEMM where it fits, else the transform into the workspace first
        lay, ws, x, xr, y = per_layer[li]
        ex.forward(ws[copy % len(ws)], x[:M], torch.bfloat16, out=y[M])

    def step(g):
        # graph g: call j of a layer takes copy g * (calls of the layer) + j
        for li in range(len(per_layer)):
            n = len(Ms_of[li])
            for j, M in enumerate(Ms_of[li]):
                call(li, M, g * n + j)

    if args.only:
        with torch.cuda.stream(stream):
            for i in range(args.warmup + args.steps):
                step(i)
        torch.cuda.synchronize()
        log(f"ran {args.only} x {args.warmup + args.steps}")
        return

    # ---- HIP graphs of the step, each on its own weight copies
    n_graphs = 2
    graphs = []
    with torch.cuda.stream(stream):
        step(0)
    torch.cuda.synchronize()
    for g_ in range(n_graphs):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=stream):
            step(g_)
        graphs.append(gr)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        graphs[i % n_graphs].replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % n_graphs].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    sol_step = sum(sol_seconds(M, layers[li].K, layers[li].N, layers[li].bits) for li, M in calls)
    value = 100.0 * sol_step / (ms_per_step / 1e3)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step, SoL {sol_step * 1e3:.4f} ms -> {value:.2f}% SoL")

    # ---- per-launch timing with HIP events on the launch stream: R launches
    # back to back between one event pair, queued behind a spin kernel so the
    # GPU never waits on the host inside the pair (an event pair per launch
    # costs several microseconds on this stack, more than the small kernels).
    spin = getattr(torch.cuda, "_sleep", None)

    def time_calls(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        if spin is not None:
            spin(int(1e7))
        e0.record(stream)
        for r in range(reps):
            fn(r)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # microseconds per call

    def time_batches(fn, reps, batches=5):
        """The pages' protocol: batches of `reps` calls after the warm-up, each
        timed by one event pair; returns (median, min) of the per-call means."""
        ts = sorted(time_calls(fn, reps) for _ in range(batches))
        return ts[len(ts) // 2], ts[0]

    per_shape = []
    with torch.cuda.stream(stream):
        for li, M in calls:
            lay, ws, x, xr, y = per_layer[li]
            copies = len(ws)
            pick = lambda r: ws[(r * 7 + 3) % copies]
            t_in = time_calls(lambda r: ex.input_transform(x[:M], pick(r).suh, out=xr[M]), args.timing_reps)
            t_lin, t_lin_min = time_batches(lambda r: ex.linear(pick(r), xr[M], torch.bfloat16, out=y[M]),
                                            args.timing_reps)
            # warm: the same weight copy every call (L2/MALL-resident when it fits)
            t_warm = time_calls(lambda r: ex.linear(ws[0], xr[M], torch.bfloat16, out=y[M]), args.timing_reps)
            t_fw = time_calls(lambda r: ex.forward(pick(r), x[:M], torch.bfloat16, out=y[M]), args.timing_reps)
            pl = ex.plan(ws[0], M)
            byts = lay.weight_bytes()
            flops = 2.0 * M * lay.K * lay.N
            sol = sol_seconds(M, lay.K, lay.N, lay.bits)
            per_shape.append({
                "layer": lay.name, "M": M, "K": lay.K, "N": lay.N, "bits": lay.bits, "codebook": lay.codebook,
                "plan": pl, "transform_us": round(t_in, 3), "linear_us": round(t_lin, 3),
                "linear_us_min": round(t_lin_min, 3), "linear_us_warm": round(t_warm, 3),
                "forward_us": round(t_fw, 3), "rotation_in_gemm": ex.forward_workspace_bytes(ws[0], M) == pl["workspace"],
                "kernels_per_linear": pl["launches"],
                "GBps": round(byts / (t_lin * 1e-6) / 1e9, 1),
                "TFLOPS": round(flops / (t_lin * 1e-6) / 1e12, 2),
                "pct_sol": round(100.0 * sol / (t_lin * 1e-6), 2),
                "pct_sol_with_transform": round(100.0 * sol / ((t_lin + t_in) * 1e-6), 2),
                "pct_sol_forward": round(100.0 * sol / (t_fw * 1e-6), 2),
                "bound": "mfma" if flops / MFMA_F16_FLOPS > byts / HBM_BPS else "hbm",
            })
            log(f"{lay.name} M={M}: plan {pl}, transform {t_in:.2f} us, linear {t_lin:.2f} us, forward {t_fw:.2f} us "
                f"({per_shape[-1]['GBps']} GB/s, {per_shape[-1]['TFLOPS']} TFLOP/s, "
                f"{per_shape[-1]['pct_sol']}% SoL)")

    # ---- rulers measured in this run: a streaming read of 2 GiB, a pure fp16
    # matrix-core loop, and per layer the decode path alone (the tile
    # kernels' trellis staging and decode without products or stores), so
    # the figures can be read against what this GPU delivers to simple
    # kernels as well as against the data-sheet peaks.
    with torch.cuda.stream(stream):
        big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        rw = torch.empty(ex.RULER_WORDS, dtype=torch.int32, device=dev)
        t_rd = time_calls(lambda r: ex.debug_stream_read(big, out=rw), 5)
        hbm_ruler = big.numel() / (t_rd * 1e-6)
        del big
        iters = 2000
        rf = torch.empty(ex.RULER_WORDS, dtype=torch.float32, device=dev)
        t_mf = time_calls(lambda r: ex.debug_mfma_loop(iters, out=rf), 5)
        mfma_ruler = ex.mfma_loop_flops(iters) / (t_mf * 1e-6)
        # the same loop on operands that change every product (real data's
        # power draw: the clock drops)
        t_mt = time_calls(lambda r: ex.debug_mfma_loop(iters, one=0, out=rf), 5)
        mfma_toggle = ex.mfma_loop_flops(iters) / (t_mt * 1e-6)
        decode = {}
        for li, (lay, ws, x, xr, y) in enumerate(per_layer):
            ro = torch.empty((lay.K // 128, lay.N // 128), dtype=torch.int32, device=dev)
            t_dr = time_calls(lambda r: ex.debug_decode_rate(ws[(r * 7 + 3) % len(ws)], out=ro), args.timing_reps)
            decode[lay.name] = {"us": round(t_dr, 3),
                                "weights_per_s": float(f"{lay.K * lay.N / (t_dr * 1e-6):.4g}"),
                                "trellis_GBps": round(lay.weight_bytes() / (t_dr * 1e-6) / 1e9, 1)}
    rulers = {"hbm_read_GBps": round(hbm_ruler / 1e9, 1), "mfma_f16_TFLOPS": round(mfma_ruler / 1e12, 1),
              "mfma_f16_toggling_TFLOPS": round(mfma_toggle / 1e12, 1),
              "decode": decode, "spec": {"hbm_GBps": HBM_BPS / 1e9, "mfma_f16_TFLOPS": MFMA_F16_FLOPS / 1e12},
              "how": "stream read: 2 GiB, 262144 threads, 16-byte loads; mfma: 4096 waves x 16 independent "
                     "v_mfma_f32_16x16x32_f16 chains x 2000, constant operands (toggling: two sets of hashed "
                     "operands alternating); decode: trellis staging + decode per 128x128 block, "
                     "weight copies cycled"}
    att_step = 0.0
    for s_ in per_shape:
        att = max(s_["K"] * s_["N"] * s_["bits"] / 8 / hbm_ruler, 2.0 * s_["M"] * s_["K"] * s_["N"] / mfma_ruler)
        s_["pct_attainable"] = round(100.0 * att / (s_["linear_us"] * 1e-6), 2)
        att_step += att
    rulers["step_pct_of_attainable"] = round(100.0 * att_step / (ms_per_step / 1e3), 3)
    log(f"rulers: stream read {rulers['hbm_read_GBps']} GB/s, mfma {rulers['mfma_f16_TFLOPS']} TFLOP/s "
        f"({rulers['mfma_f16_toggling_TFLOPS']} on toggling operands); "
        f"step at {rulers['step_pct_of_attainable']}% of the rulers' bound")

    # ---- roofline of the dominant kernel: the kernel template instance with
    # the most time per step.  Each call's kernels are timed alone: a
    # two-launch slab call is the GEMM stage (through the part-sums hook,
    # with the call's own plan and unit) plus the ordered part sum + output
    # transform (through its hook); a dense-decoder call is the dequantization
    # (through its hook) plus the GEMM over the fragments (the call minus the
    # dequantization); a one-launch call (fused, or slabs summed by the
    # tile's last workgroup) is its GEMM kernel.  So each kernel's average
    # launch duration is the one rocprof reports for it.
    frag_buf = {}
    with torch.cuda.stream(stream):
        for s_ in per_shape:
            li = [l.name for l in layers].index(s_["layer"])
            lay_, ws_, xr_ = per_layer[li][0], per_layer[li][1], per_layer[li][3]
            pl_ = s_["plan"]
            gk = kernel_key(lay_, pl_)
            kern = {gk: s_["linear_us"]}
            if pl_["decoder"] == ex.EXL3_DECODER_DENSE:
                if lay_.name not in frag_buf:
                    frag_buf[lay_.name] = torch.empty((lay_.K // 32, lay_.N // 128, 8, 64, 8), dtype=torch.int16,
                                                      device=dev)
                fb = frag_buf[lay_.name]
                t_dq = time_calls(lambda r: ex.debug_dequant(ws_[(r * 7 + 3) % len(ws_)], out=fb), args.timing_reps)
                dk = f"exl3::dequant_kernel<{lay_.bits}, {lay_.cb}u>"
                kern = {gk: round(s_["linear_us"] - t_dq, 3), dk: round(t_dq, 3)}
                if gk == "exl3::gemm_dense_wide_kernel":
                    # its two launches apart, over the fragments just decoded:
                    # 256 x 256 tiles on the first `bulk` column blocks, then
                    # 256 x 128 tiles on the rest
                    M_, nblk = s_["M"], lay_.N // 128
                    yo = torch.empty((M_, lay_.N), dtype=torch.bfloat16, device=dev)
                    gemm = lambda which: ex.debug_dense_gemm(ws_[0], fb, xr_[M_], which=which, out=yo)
                    _, bulk = gemm(1)
                    kern = {gk: round(time_calls(lambda r: gemm(1), args.timing_reps), 3), dk: round(t_dq, 3)}
                    s_["kernel_cols"] = {gk: 128 * bulk}
                    if bulk < nblk:
                        tk = "exl3::gemm_dense_kernel<false>"
                        kern[tk] = round(time_calls(lambda r: gemm(2), args.timing_reps), 3)
                        s_["kernel_cols"][tk] = 128 * (nblk - bulk)
                    del yo
            elif pl_["mode"] == ex.EXL3_MODE_SLABS and pl_["launches"] == 2:
                n_sl = pl_["parts"] // pl_["unit"]
                zp = torch.zeros((n_sl, (s_["M"] + 3) // 4, lay_.N, 4), dtype=torch.float32, device=dev)
                yo = torch.empty((s_["M"], lay_.N), dtype=torch.bfloat16, device=dev)
                t_epi = time_calls(lambda r: ex.debug_epilogue(ws_[0], zp, s_["M"], out=yo), args.timing_reps)
                t_gemm = time_calls(lambda r: ex.debug_parts(ws_[(r * 7 + 3) % len(ws_)], xr_[s_["M"]],
                                                             parts=pl_["parts"], groups=pl_["groups"],
                                                             unit=pl_["unit"], bm=pl_["bm"],
                                                             decoder=pl_["decoder"], out=zp), args.timing_reps)
                kern = {gk: round(t_gemm, 3), "exl3::epilogue_kernel": round(t_epi, 3)}
                del zp
            s_["kernels_us"] = kern
            s_["kernel"] = gk
            s_["gemm_us"] = kern[gk]
    del frag_buf
    groups = {}
    for s_ in per_shape:
        for k_, us in s_["kernels_us"].items():
            groups.setdefault(k_, []).append((s_, us))
    dom_key = max(groups, key=lambda k: sum(us for _, us in groups[k]))
    dom = groups[dom_key]
    secs = sum(us for _, us in dom) * 1e-6
    if dom_key.startswith("exl3::dequant_kernel"):
        work = sum(g["K"] * g["N"] * (g["bits"] / 8 + 2) for g, _ in dom)
        roof = {"bound": "hbm", "achieved": round(work / secs / 1e9, 1), "peak": 8000.0, "unit": "GB/s"}
        wpl = "K*N*bits/8 trellis bytes read + K*N*2 fragment bytes written"
    elif dom_key == "exl3::epilogue_kernel":
        work = sum((g["plan"]["parts"] // g["plan"]["unit"]) * g["M"] * g["N"] * 4 + g["M"] * g["N"] * 2
                   for g, _ in dom)
        roof = {"bound": "hbm", "achieved": round(work / secs / 1e9, 1), "peak": 8000.0, "unit": "GB/s"}
        wpl = "fp32 slabs read + bf16 output written"
    elif max(dom, key=lambda d: d[1])[0]["bound"] == "mfma":
        # a call whose GEMM runs in two launches (the dense decoder's) counts
        # each launch's own columns
        work = sum(2.0 * g["M"] * g["K"] * g.get("kernel_cols", {}).get(dom_key, g["N"]) for g, _ in dom)
        roof = {"bound": "mfma", "achieved": round(work / secs / 1e12, 2), "peak": 2500.0, "unit": "TFLOP/s"}
        wpl = "2*M*K*N flops (N: the columns this kernel covers)"
    else:
        work = sum(g["K"] * g["N"] * g["bits"] / 8 for g, _ in dom)
        roof = {"bound": "hbm", "achieved": round(work / secs / 1e9, 1), "peak": 8000.0, "unit": "GB/s"}
        wpl = "K*N*bits/8 trellis bytes"
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = dom_key
    roof["launches"] = [f"{g['layer']} M={g['M']}" for g, _ in dom]
    roof["avg_launch_us"] = round(secs * 1e6 / len(dom), 3)
    roof["work_per_launch"] = wpl
    roof["time_share_of_step"] = round(secs / (ms_per_step / 1e3), 4)
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            tj = json.load(open(tfile))
            ent = tj.get("entries", {}).get(dom_key)
            if ent and ent.get("source_hash") == kernel_hash(kernel_family(dom_key)):
                n = len(dom)
                # Bytes the kernel must move at least once: its weight operand (fp16 fragments for the
                # dense GEMM, the trellis otherwise), the rotated activations and the bf16/fp16 output.
                cols = lambda g: g.get("kernel_cols", {}).get(dom_key, g["N"])
                wbytes = (lambda g: g["K"] * cols(g) * 2) if "dense" in dom_key else \
                         (lambda g: g["K"] * g["N"] * g["bits"] / 8)
                alg = sum(wbytes(g) + g["M"] * g["K"] * 2 + g["M"] * cols(g) * 2 for g, _ in dom) / n
                roof["traffic"] = {"hbm_bytes_per_launch": ent["fetch_bytes"] + ent["write_bytes"],
                                   "fetch_bytes_per_launch": ent["fetch_bytes"],
                                   "write_bytes_per_launch": ent["write_bytes"],
                                   "algorithmic_bytes_per_launch": round(alg),
                                   "scale": ent.get("scale"), "measured_on": ent.get("measured_on")}
        except Exception as e:  # a malformed file only loses the traffic field
            log(f"traffic file unreadable: {e}")
    roof["ruler_peak"] = rulers["mfma_f16_TFLOPS"] if roof["unit"] == "TFLOP/s" else rulers["hbm_read_GBps"]
    roof["ruler_frac"] = round(roof["achieved"] / roof["ruler_peak"], 4)
    if roof["unit"] == "TFLOP/s":
        roof["ruler_peak_toggling"] = rulers["mfma_f16_toggling_TFLOPS"]
        roof["ruler_frac_toggling"] = round(roof["achieved"] / roof["ruler_peak_toggling"], 4)
    log(f"roofline: {dom_key} over {roof['launches']}: {roof['achieved']} {roof['unit']} = "
        f"{100 * roof['frac']:.1f}% of peak, {roof['avg_launch_us']} us per launch")

    line = {
        "metric": "EXL3 linear achieved GB/s + TFLOPS and %SoL vs max(HBM,MFMA) per (M,K,N,bits)",
        "value": round(value, 3),
        "unit": "% of SoL (aggregate over the step)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded uniform trellis, +-1 suh/svh, N(0,1) bf16 x)",
        "config": {"workload": args.workload, "layers": [
            {"name": l.name, "K": l.K, "N": l.N, "shards": list(l.shards), "bits": l.bits, "codebook": l.codebook,
             "M": list(Ms_of[i]), "weight_copies": len(per_layer[i][1])} for i, l in enumerate(layers)],
            "calls_per_step": len(calls), "sol_ms_per_step": round(sol_step * 1e3, 5),
            "schedules": "tuned on the weight pool (same bits)" if args.tune else "planner",
            "parallelism": "single GPU"},
        "roofline": roof,
        "rulers": rulers,
        "per_shape": per_shape,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        line["cpu_baseline"] = cpu_baseline(spec)
    out = json.dumps(line)
    print(out, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(out + "\n")


def moe_main(args, ex, wl, torch, np, dev):
    """Routed experts: per layer and token count T, one call = alignment,
    routed input rotation, grouped GEMM and ordered combine.  Routings are
    drawn per call from a pool of 32 (so the experts touched change and
    stream from HBM); SoL = max(trellis bytes of the distinct experts the
    call touches / HBM, 2 * T * topk * K * N / MFMA peak)."""
    names, E, k, Ts = MOE_WORKLOADS[args.workload]
    layers = [wl.layer(n) for n in names]
    rng = np.random.default_rng(20269000)
    per = []
    stream = torch.cuda.Stream()
    spin = getattr(torch.cuda, "_sleep", None)

    def time_calls(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for r in range(2):  # warm-up: first launches load the kernels
            fn(r)
        torch.cuda.synchronize()
        if spin is not None:
            spin(int(1e7))
        e0.record(stream)
        for r in range(reps):
            fn(r)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def d(a, dt=torch.int16):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)

    sol_step, rows_out = 0.0, []
    with torch.cuda.stream(stream):
        for lay in layers:
            tr = rng.integers(0, 65536, (E, lay.K // 16, lay.N // 16, 16 * lay.bits), dtype=np.uint16)
            suh = np.where(rng.integers(0, 2, (E, 1, lay.K)) == 1, 0xBC00, 0x3C00).astype(np.uint16)
            svh = np.where(rng.integers(0, 2, (E, lay.N)) == 1, 0xBC00, 0x3C00).astype(np.uint16)
            w = ex.MoeWeight(d(tr), d(suh, torch.float16), d(svh, torch.float16), lay.bits, lay.codebook)
            del tr
            for T in Ts:
                pool = [np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
                        for _ in range(32)]
                ids = [torch.from_numpy(a).to(dev) for a in pool]
                wts = [torch.from_numpy(rng.dirichlet(np.ones(k), T).astype(np.float32)).to(dev) for _ in pool]
                x = d(wl.round_f32_to_bf16_bits(rng.standard_normal((T, lay.K)).astype(np.float32)), torch.bfloat16)
                t_call = time_calls(lambda r: ex.moe_forward(x, w, ids[r % 32], wts[r % 32]), args.timing_reps)
                routes = [ex.moe_align(i, E) for i in ids]
                xrs = [ex.moe_input_transform(x, w, rt, k) for rt in routes]
                t_gemm = time_calls(lambda r: ex.moe_linear(w, xrs[r % 32], routes[r % 32][1]), args.timing_reps)
                # each decoder of the grouped GEMM forced, for the automatic choice's record
                t_dec = {name: time_calls(lambda r: ex.moe_linear(w, xrs[r % 32], routes[r % 32][1], decoder=dc),
                                          args.timing_reps)
                         for name, dc in (("alu", ex.EXL3_DECODER_ALU), ("table", ex.EXL3_DECODER_TABLE))}
                touched = float(np.mean([len(np.unique(a)) for a in pool]))
                byts = touched * lay.weight_bytes()
                flops = 2.0 * T * k * lay.K * lay.N
                sol = max(byts / HBM_BPS, flops / MFMA_F16_FLOPS)
                sol_step += sol
                per.append({"layer": lay.name, "experts": E, "topk": k, "T": T, "experts_touched": touched,
                            "call_us": round(t_call, 3), "grouped_gemm_us": round(t_gemm, 3),
                            "grouped_gemm_us_by_decoder": {k_: round(v_, 3) for k_, v_ in t_dec.items()},
                            "GBps": round(byts / (t_gemm * 1e-6) / 1e9, 1),
                            "TFLOPS": round(flops / (t_gemm * 1e-6) / 1e12, 2),
                            "pct_sol_call": round(100 * sol / (t_call * 1e-6), 2),
                            "pct_sol_gemm": round(100 * sol / (t_gemm * 1e-6), 2)})
                log(f"moe {lay.name} E={E} top{k} T={T}: {touched:.1f} experts touched, call {t_call:.2f} us, "
                    f"grouped GEMM {t_gemm:.2f} us ({per[-1]['GBps']} GB/s, {per[-1]['pct_sol_gemm']}% SoL; "
                    f"ALU {t_dec['alu']:.2f} us, table {t_dec['table']:.2f} us)")
            del w
    step_us = sum(p_["call_us"] for p_ in per)
    gemm = sum(p_["grouped_gemm_us"] for p_ in per)
    byts = sum(p_["experts_touched"] * wl.layer(p_["layer"]).weight_bytes() for p_ in per)
    line = {
        "metric": "EXL3 linear achieved GB/s + TFLOPS and %SoL vs max(HBM,MFMA) per (M,K,N,bits)",
        "value": round(100.0 * sol_step / (step_us * 1e-6), 3),
        "unit": "% of SoL (aggregate over the routed calls)",
        "n_gpus": 1, "steps": args.timing_reps, "warmup": 2, "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded uniform trellis, +-1 suh/svh, N(0,1) bf16 x, uniform top-k routing)",
        "config": {"workload": args.workload, "experts": E, "topk": k, "T": list(Ts),
                   "layers": [{"K": l.K, "N": l.N, "bits": l.bits, "codebook": l.codebook} for l in layers],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(byts / (gemm * 1e-6) / 1e9, 1), "peak": HBM_BPS / 1e9,
                     "unit": "GB/s", "frac": round(byts / (gemm * 1e-6) / HBM_BPS, 4), "traffic": None,
                     "kernel": "grouped GEMM (exl3::gemm_table_kernel<..., true> from 256 units, else "
                               "exl3::gemm_kernel<..., true>)",
                     "work_per_launch": "trellis bytes of the experts the call touches"},
        "per_shape": per,
    }
    print(json.dumps(line), flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(json.dumps(line) + "\n")


if __name__ == "__main__":
    main()
