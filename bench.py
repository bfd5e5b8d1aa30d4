#!/usr/bin/env python3
"""Benchmark of the ball-tree + ball-attention hot path on one MI355X.

One step = one ball-attention pass (ball_attn) over one synthetic point cloud
of the measured shape, gathering q/k/v through a tree permutation and
scattering the result back to original order.  The GPU tree builder is
limited to 1,024 points in this version, so the permutation is a seeded random
one: the synthetic clouds are in random original order, so a tree order is a
random gather pattern too, and the kernel's work does not depend on which
permutation it is.  Inputs are resident in HBM before the timed region
starts.  The q/k/v/out tensors rotate over several copies
(default 4, 540 MB in all) so that no step finds its inputs in the 256 MB
Infinity Cache left behind by the previous one.

Prints ONE JSON line.  Besides the required fields it carries:
  roofline      for the ball-attention kernel: algorithmic bytes per launch
                (q, k, v read once, out written once, perm read once) over the
                mean launch time measured with HIP events on the launching
                stream, against the 8 TB/s HBM peak; `traffic` is the HBM
                byte count of the kernel per launch from rocprofv3 FETCH_SIZE +
                WRITE_SIZE counters (profiles/), or null if the kernel source
                changed since they were taken;
  cpu_baseline  the CPU oracle (NumPy fp64 ball attention) timed on this
                host on whole steps of the same workload;
  rows          the other rows of the path timed in the same run on their
                own workloads: permute gather/scatter of 512-byte rows at the
                rotated-pair size, the BSA step (also with group compression),
                and tree build + fp32 ball attention at 1,024 points (the
                largest tree the GPU builder takes in this version).

Other workloads (--workload bsa | cosmo | rotpair) print their own line and
are not the default measurement.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ball-attn points/sec + TFLOP/s (% roofline) at N=65,536, ball 128, H=8 d=32"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def _src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "ball_tree_sparse_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, src_names):
    """Per-launch HBM bytes from the committed counter summary, if current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("src_hash") != _src_hash(src_names):
        return None
    return t.get("bytes_per_launch")


def _cpu_baseline(w, budget_s):
    """The oracle on whole steps of the workload until the budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as A
    n = w.coords.shape[0]
    p = np.random.default_rng(1234).permutation(n)
    steps, t0 = 0, time.perf_counter()
    while True:
        A.ball_attn(w.q, w.k, w.v, p, w.ball)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": steps * n / el, "unit": "points/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} whole steps (fp64 ball attention over all balls) of the "
                      f"{n}-point workload in {el:.1f} s, through {threads}-thread BLAS on "
                      f"{len(os.sched_getaffinity(0))} host cores"}


def bench_ball(args, dev, torch, ops, synth):
    w = synth.make(args.workload)
    N, H, d, ball, leaf = w.coords.shape[0], w.H, w.d, w.ball, w.leaf
    g = torch.Generator().manual_seed(1234)
    perm = torch.randperm(N, generator=g).to(torch.int32).to(dev)
    sets = []
    for _ in range(args.sets):
        q, k, v = (t.to(dev).clone() for t in (w.q, w.k, w.v))
        sets.append((q, k, v, torch.empty_like(q)))

    def step(i):
        q, k, v, out = sets[i % len(sets)]
        ops.ball_attn(q, k, v, perm, ball, out=out)

    for i in range(len(sets)):                 # load the kernel, touch every set
        step(i)
    torch.cuda.synchronize()
    if args.copy_probe:
        # a plain device copy of known size, for scaling HBM byte counters
        src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
    if args.eager:
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"eager_launches": args.steps}), flush=True)
        return None
    # warmup: back-to-back launches until the clocks have settled
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: back-to-back launches on the current stream, HIP events
    # recorded on that stream around them
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nsteps = args.steps
    t0 = time.perf_counter()
    e0.record()
    for i in range(nsteps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    attn_us = e0.elapsed_time(e1) * 1e3 / nsteps
    # the same launches replayed from a HIP graph (one launch per input set),
    # for comparison: replays add a gap between kernels
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(len(sets)):
            step(i)
    reps = max(1, nsteps // len(sets))
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(reps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_us = g0.elapsed_time(g1) * 1e3 / (reps * len(sets))
    # single launches, each between its own pair of events with the device
    # idle before it: median and minimum of 60 (no back-to-back overlap)
    single = []
    for i in range(60):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        step(i)
        a1.record()
        torch.cuda.synchronize()
        single.append(a0.elapsed_time(a1) * 1e3)
    single.sort()

    esize = 2 if w.dtype == "bf16" else 4
    attn_bytes = 4 * N * H * d * esize + 4 * N
    attn_flops = 4 * N * ball * d * H
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    traffic = _traffic(f"ball_attn/{args.workload}", ["ball_attn.hip", "common.h"])
    ms = el / nsteps * 1e3
    line = {
        "metric": METRIC, "value": N / (ms * 1e-3), "unit": "points/s", "n_gpus": 1,
        "steps": nsteps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{args.workload}: ball attention over a tree permutation, "
                               f"N={N}, ball {ball}, H={H}, d={d}, {w.dtype}",
                   "N": N, "ball": ball, "leaf": leaf, "H": H, "d": d,
                   "input_sets_rotated": len(sets),
                   "timing": "back-to-back launches on one stream; HIP events on that "
                             "stream around the timed launches"},
        "roofline": {"kernel": "ball_attn_mfma" if w.dtype == "bf16" else "ball_attn_valu",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": attn_bytes},
        "ball_attn": {"us": attn_us, "us_graph_replay": graph_us,
                      "us_single_median": single[len(single) // 2], "us_single_min": single[0],
                      "points_per_s": N / (attn_us * 1e-6),
                      "tflops": attn_flops / (attn_us * 1e-6) / 1e12,
                      "mfma_frac": attn_flops / (attn_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS},
    }
    if not args.no_side_rows:
        line["rows"] = side_rows(dev, torch, ops, synth)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(w, args.cpu_seconds)
    return line


def _event_us(torch, fn, reps, warm=3):
    """Mean time per call of fn() over reps back-to-back calls (HIP events
    on the current stream, the stream the library launches on)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def side_rows(dev, torch, ops, synth):
    """The other rows of the path, timed in the same run on their own
    workloads: permute (gather and scatter of 512-byte rows at the rotated-
    pair size), coarsen / refine, the BSA steps, padded ball attention of an
    uneven N, the backward of ball attention, and tree build + fp32 ball
    attention at the size the GPU tree builder takes (1,024 points)."""
    rows = {}
    # permute: N = 262,144 rows of H*d bf16 = 512 bytes; three source and
    # destination pairs (805 MB) rotate so that no call finds its rows in the
    # 256 MB Infinity Cache
    n, row = 262144, 8 * 32
    gen = torch.Generator(device=dev).manual_seed(4)
    srcs = [torch.randint(-32768, 32767, (n, row), dtype=torch.int16, device=dev, generator=gen)
            for _ in range(3)]
    dsts = [torch.empty_like(srcs[0]) for _ in range(3)]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(4)).to(torch.int32).to(dev)
    nbytes = 2 * n * row * 2 + 4 * n
    for name, mode in (("gather", ops.BT_GATHER), ("scatter", ops.BT_SCATTER)):
        it = [0]

        def call():
            i = it[0] % 3
            it[0] += 1
            ops.bt_permute(srcs[i], perm, mode, dst=dsts[i])
        us = _event_us(torch, call, 60, warm=6)
        rows["a5_permute_" + name] = {"workload": "N=262144 rows of 512 B (rotated-pair size)",
                                      "us": us, "GBps": nbytes / us / 1e3,
                                      "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS}
    del srcs, dsts
    # coarsen / refine by 8 (Erwin's U-Net levels) at the sphere size: three
    # input sets rotate so that every call reads HBM
    n, H, d, s = 65536, 8, 32, 8
    xs = [torch.randint(-32768, 32767, (n, H, d), dtype=torch.int16, device=dev,
                        generator=gen).view(torch.bfloat16) for _ in range(3)]
    xs = [x.masked_fill(~torch.isfinite(x), 0) for x in xs]
    pc = torch.randperm(n, generator=torch.Generator().manual_seed(5)).to(torch.int32).to(dev)
    cs = [torch.empty((n // s, H, d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    fs = [torch.empty_like(xs[0]) for _ in range(3)]
    row = H * d * 2
    for name, fn, nbytes in (
            ("coarsen", lambda i: ops.bt_coarsen(xs[i % 3], pc, s, out=cs[i % 3]),
             n * row + n // s * row + 4 * n),
            ("refine", lambda i: ops.bt_refine(cs[i % 3], pc, s, out=fs[i % 3]),
             n // s * row + n * row + 4 * n)):
        it = [0]

        def call(fn=fn):
            fn(it[0])
            it[0] += 1
        us = _event_us(torch, call, 60, warm=6)
        rows["f2_" + name] = {"workload": "N=65536, H=8, d=32 bf16, s=8, perm",
                              "us": us, "GBps": nbytes / us / 1e3,
                              "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS}
    del xs, cs, fs
    # BSA step
    w = synth.make("bsa")
    x = w.extra
    N, H, d = w.coords.shape[0], w.H, w.d
    p = torch.randperm(N, generator=torch.Generator().manual_seed(1234)).to(torch.int32).to(dev)
    bws = torch.empty(ops.bsa_workspace_size(N, H, d, w.ball, x["block"], x["group"], x["topk"]),
                      dtype=torch.uint8, device=dev)
    Wg = torch.from_numpy(w.gate_w).to(dev)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    out = torch.empty_like(q)
    us = _event_us(torch, lambda: ops.bsa_attn(q, k, v, p, w.ball, x["block"], x["group"],
                                               x["topk"], x["mask_own_ball"], gate_w=Wg,
                                               out=out, workspace=bws), 100, warm=20)
    flops = 4 * N * H * d * (w.ball + N // x["block"] + x["topk"] * x["block"])
    rows["a7_a11_bsa"] = {"workload": "N=65536 deformed sphere, ball 128, block 64, group 64, "
                                      "top-16, H=8, d=32 bf16",
                          "us_per_step": us, "points_per_s": N / (us * 1e-6),
                          "tflops": flops / (us * 1e-6) / 1e12,
                          "mfma_frac": flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}
    # the same with group (query) compression
    bws2 = torch.empty(ops.bsa_workspace_size(N, H, d, w.ball, x["block"], x["group"], x["topk"],
                                              query_compression=True),
                       dtype=torch.uint8, device=dev)
    us2 = _event_us(torch, lambda: ops.bsa_attn(q, k, v, p, w.ball, x["block"], x["group"],
                                                x["topk"], x["mask_own_ball"], gate_w=Wg,
                                                out=out, workspace=bws2, query_compression=True),
                    100, warm=20)
    flops2 = 4 * H * d * (N * w.ball + (N // x["block"]) ** 2 +
                          (N // x["group"]) * x["topk"] * x["block"])
    rows["f1_bsa_group_compression"] = {
        "workload": "as a7_a11_bsa, queries pooled before compression and selection",
        "us_per_step": us2, "points_per_s": N / (us2 * 1e-6),
        "tflops": flops2 / (us2 * 1e-6) / 1e12, "speedup_vs_bsa": us / us2}
    # backward of BSA (no group compression) at the same size
    bdo = q.clone()
    bgr = [torch.empty_like(q) for _ in range(3)]
    bws3 = torch.empty(ops.bsa_attn_bwd_workspace_size(N, H, d, w.ball, x["block"], x["group"],
                                                       x["topk"]),
                       dtype=torch.uint8, device=dev)
    us4 = _event_us(torch, lambda: ops.bsa_attn_bwd(q, k, v, p, bdo, w.ball, x["block"],
                                                    x["group"], x["topk"], x["mask_own_ball"],
                                                    gate_w=Wg, grads=bgr, workspace=bws3),
                    30, warm=5)
    rows["f4_bsa_bwd"] = {"workload": "as a7_a11_bsa: dq, dk, dv and the gate gradients",
                          "us": us4, "tflops": 2.5 * flops / (us4 * 1e-6) / 1e12,
                          "mfma_frac": 2.5 * flops / (us4 * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
                          "vs_forward": us4 / us}
    del q, k, v, out, bws, bws2, bws3, bdo, bgr
    # uneven N: 65,000 sphere points in 65,536 slots (535 unused slots spread
    # over the balls), masked ball attention; three input sets rotate
    n3, slots = 65000, 65536
    w = synth.make("sphere", n=n3)
    g3 = torch.Generator().manual_seed(11)
    pp = torch.full((slots,), -1, dtype=torch.int32)
    pp[torch.randperm(slots, generator=g3)[:n3]] = torch.randperm(n3, generator=g3).to(torch.int32)
    pp = pp.to(dev)
    sets = [tuple(t.to(dev).clone() for t in (w.q, w.k, w.v)) for _ in range(3)]
    o3 = [torch.empty_like(sets[0][0]) for _ in range(3)]
    it = [0]

    def call3():
        i = it[0] % 3
        it[0] += 1
        ops.ball_attn_padded(*sets[i], pp, w.ball, out=o3[i])
    us3 = _event_us(torch, call3, 300, warm=100)
    nb3 = 4 * n3 * w.H * w.d * 2 + 4 * slots
    rows["f3_ball_attn_padded"] = {"workload": "N=65,000 in 65,536 slots, ball 128, H=8, d=32 bf16",
                                   "us": us3, "GBps": nb3 / us3 / 1e3,
                                   "hbm_frac": nb3 / us3 / 1e3 / HBM_PEAK_GBS}
    del sets, o3
    # backward of ball attention at the sphere size
    w = synth.make("sphere")
    gq, gk, gv = (t.to(dev) for t in (w.q, w.k, w.v))
    gdo = gq.clone()
    pb = torch.randperm(w.coords.shape[0], generator=torch.Generator().manual_seed(7)) \
        .to(torch.int32).to(dev)
    grads = [torch.empty_like(gq) for _ in range(3)]
    us_b = _event_us(torch, lambda: ops.ball_attn_bwd(gq, gk, gv, gdo, pb, w.ball, *grads), 300,
                     warm=100)
    nb = w.coords.shape[0]
    bflops = 4 * nb * w.ball * w.d * w.H * 2.5        # S, dP, dV, dQ, dK (2.5x the forward)
    bbytes = 7 * nb * w.H * w.d * 2 + 4 * nb     # q, k, v, dO gathered; dq, dk, dv scattered
    rows["f4_ball_attn_bwd"] = {"workload": "N=65536, ball 128, H=8, d=32 bf16",
                                "us": us_b, "tflops": bflops / (us_b * 1e-6) / 1e12,
                                "GBps": bbytes / us_b / 1e3,
                                "hbm_frac": bbytes / us_b / 1e3 / HBM_PEAK_GBS,
                                "mfma_frac": bflops / (us_b * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}
    del gq, gk, gv, gdo, grads
    # tree build + fp32 ball attention at 1,024 points
    w = synth.make("tiny")
    c = torch.from_numpy(w.coords).to(dev)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    tws = torch.empty(max(256, ops.bt_build_workspace_size(c.shape[0], w.leaf)), dtype=torch.uint8,
                      device=dev)
    pt = torch.empty(c.shape[0], dtype=torch.int32, device=dev)
    ot = torch.empty_like(q)
    us_b = _event_us(torch, lambda: ops.bt_build(c, w.leaf, perm=pt, workspace=tws), 200)
    us_a = _event_us(torch, lambda: ops.ball_attn(q, k, v, pt, w.ball, out=ot), 200)
    rows["a1_a4_a6_tiny"] = {"workload": "N=1024 uniform cube, leaf = ball 32, H=4, d=16 fp32",
                             "build_us": us_b, "ball_attn_us": us_a,
                             "bound": "latency (one workgroup; 16 KB of records)"}
    # padded tree of an uneven N: 972 points (the Elasticity cloud size), leaf 32
    c9 = c[:972].contiguous()
    tws9 = torch.empty(max(256, ops.lib().bt_build_padded_workspace_size(972, 32)),
                       dtype=torch.uint8, device=dev)
    pt9 = torch.empty(ops.bt_padded_size(972, 32), dtype=torch.int32, device=dev)
    us_p = _event_us(torch, lambda: ops.bt_build_padded(c9, 32, perm=pt9, workspace=tws9), 200)
    rows["f3_tree_padded"] = {"workload": "N=972 uniform cube in 1,024 slots, leaf 32",
                              "build_us": us_p, "bound": "latency (one workgroup)"}
    return rows


def bench_bsa(args, dev, torch, ops, synth):
    w = synth.make("bsa")
    x = w.extra
    N, H, d = w.coords.shape[0], w.H, w.d
    g = torch.Generator().manual_seed(1234)
    perm = torch.randperm(N, generator=g).to(torch.int32).to(dev)
    bws = torch.empty(ops.bsa_workspace_size(N, H, d, w.ball, x["block"], x["group"], x["topk"]),
                      dtype=torch.uint8, device=dev)
    Wg = torch.from_numpy(w.gate_w).to(dev)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    out = torch.empty_like(q)

    def step():
        ops.bsa_attn(q, k, v, perm, w.ball, x["block"], x["group"], x["topk"],
                     x["mask_own_ball"], gate_w=Wg, out=out, workspace=bws)

    warm, steps = min(args.warmup, 300), min(args.steps, 500)   # ~0.65 ms per step
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms = el / steps * 1e3
    flops = 4 * N * H * d * (w.ball + N // x["block"] + x["topk"] * x["block"])
    return {"metric": "bsa points/sec", "value": N / (ms * 1e-3), "unit": "points/s",
            "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "bsa: BSA over a tree permutation (ball 128, block 64, "
                                   "group 64, top-16), N=65536, H=8, d=32"},
            "attention_tflops": flops / (ms * 1e-3) / 1e12}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=8000)
    ap.add_argument("--workload", default="sphere",
                    choices=["sphere", "cosmo", "rotpair", "tiny", "bsa"])
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side-rows", action="store_true",
                    help="skip the permute, BSA and tiny tree measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--eager", action="store_true",
                    help="only launch the kernels (for counter collection)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of known size (counter scaling)")
    ap.add_argument("--copy-probe-mb", type=int, default=128)
    ap.add_argument("--rows-only", action="store_true",
                    help="time only the other rows (permute, coarsen/refine, BSA, padded "
                         "attention, backward, small trees); for kernel traces and counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from ball_tree_sparse_amd import ops, synth
    ops.lib()                                  # fail loudly if the library is missing
    dev = torch.device("cuda:0")
    if args.rows_only:
        if args.copy_probe:
            src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            for _ in range(4):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        print(json.dumps({"rows": side_rows(dev, torch, ops, synth)}), flush=True)
        return
    if args.workload == "bsa":
        line = bench_bsa(args, dev, torch, ops, synth)
    else:
        line = bench_ball(args, dev, torch, ops, synth)
    if line is not None:
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
