#!/usr/bin/env python3
"""Benchmark of the ball-tree + ball-attention hot path on one MI355X.

One step = one ball-attention pass (ball_attn) over one synthetic point cloud
of the measured shape, gathering q/k/v through a permutation into ball order
and scattering the result back to original order.  The permutation is the
cloud's ball tree, built on the GPU (bt_build) before the timed region.
Inputs are resident in HBM before the timed region starts.  The q/k/v/out tensors rotate
over several copies (default 4, 540 MB in all) so that no step finds its
inputs in the 256 MB Infinity Cache left behind by the previous one.

Timing: before the W warmup steps the kernel runs back to back for about
0.3 s so that the clocks settle (reported as config.settle_launches); then
the K timed steps run back to back between two HIP events recorded on the
launching stream.  `value`, `ms_per_step` and `roofline.achieved` all come
from that one event interval.

Prints ONE JSON line.  Besides the required fields it carries:
  roofline      for the ball-attention kernel: algorithmic bytes per launch
                (q, k, v read once, out written once, perm read once) over the
                mean launch time, against the 8 TB/s HBM peak (source in
                peak_source, and gpu_rocminfo gives the clock and compute units
                that rocminfo reports); `traffic` is the HBM byte count of the kernel
                per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE counters
                (profiles/), or null if the kernel source changed since they
                were taken; `measured_copy_GBps` is a timed 128 MiB
                device-to-device copy in the same run, a secondary reference;
  cpu_baseline  the CPU oracle (NumPy fp64 ball attention) timed on this
                host on whole steps of the same workload, with the CPU model
                and the BLAS thread count;
  rows          the other rows of the path timed in the same run on their
                own workloads: permute gather/scatter of 512-byte rows at the
                rotated-pair size, coarsen/refine, the BSA step (also with
                group compression) with the count of top-k rows whose
                selection differs from the oracle's (near ties), padded
                attention, the backward passes, and tree build + fp32 ball
                attention at 1,024 points, and trees of 8,192 points and of
                the pages' 3,586- and 5,000-point clouds (padded).

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
PEAK_SOURCE = ("AMD Instinct MI355X public specification: HBM3E 8.0 TB/s; dense bf16 "
               "MFMA 2.5 PFLOP/s (without sparsity); 256 CUs at 2.4 GHz")


def _rocminfo_gpu():
    """The GPU agent's clock and compute units as rocminfo prints them (a
    child process, run before this process touches the GPU), or None."""
    import subprocess
    try:
        r = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60)
    except (OSError, subprocess.SubprocessError):
        return None
    agent, found = {}, None
    for line in r.stdout.splitlines():
        t = line.strip()
        if t.startswith("Name:") and "gfx" in t:
            agent = {"name": t.split(":", 1)[1].strip()}
        elif agent and t.startswith("Max Clock Freq. (MHz):"):
            agent["max_clock_mhz"] = int(t.split(":", 1)[1].split()[0])
        elif agent and t.startswith("Compute Unit:"):
            agent["compute_units"] = int(t.split(":", 1)[1].split()[0])
        if "max_clock_mhz" in agent and "compute_units" in agent:
            found = agent
            break
    return found


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


def _cpu_baseline(w, budget_s, sel_check=None):
    """The oracle on whole steps of the workload until the budget is spent.
    With sel_check (the BSA row's inputs and the GPU's selections), the
    oracle's top-k selection is computed too and the rows whose selected set
    differs from the GPU's are counted (near ties of fp32 scores)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as A
    from oracle import tree as T
    n = w.coords.shape[0]
    p = T.build(w.coords, w.leaf)              # the oracle's tree, outside the timed steps
    steps, t0 = 0, time.perf_counter()
    while True:
        A.ball_attn(w.q, w.k, w.v, p, w.ball)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    out = {"value": steps * n / el, "unit": "points/s", "cores": threads, "kind": "oracle",
           "cpu_model": _cpu_model(), "host_cores_visible": len(os.sched_getaffinity(0)),
           "sample": f"{steps} whole steps (fp64 ball attention over all balls of the "
                     f"oracle's tree) of the {n}-point workload in {el:.1f} s, through "
                     f"{threads}-thread BLAS"}
    if sel_check is not None:
        out["bsa_topk_rows_differing"] = _sel_differences(**sel_check)
    return out


def _sel_differences(wb, perm, sel_gpu, tau_rel=1e-4):
    """Rows (head, group) whose GPU top-k set differs from the oracle's, and
    how many of those differ only by near ties (every differing block's
    fp64 score within tau_rel * max|s| of the oracle's k-th score)."""
    import numpy as np

    from oracle import bsa as B
    x = wb.extra
    qt = np.asarray(wb.q.float().numpy(), np.float64)[perm]
    kt = np.asarray(wb.k.float().numpy(), np.float64)[perm]
    kc = B.pool_blocks(kt, x["block"])
    sel, s = B.select(qt, kc, wb.ball, x["block"], x["group"], x["topk"], x["mask_own_ball"])
    diff = near = 0
    H, G, K = sel.shape
    for h in range(H):
        for g in range(G):
            a, b = set(sel[h, g].tolist()), set(sel_gpu[h, g].tolist())
            if a == b:
                continue
            diff += 1
            sc = s[g, h]
            kth = sc[sel[h, g][-1]]
            tau = tau_rel * np.max(np.abs(sc[np.isfinite(sc)]))
            near += all(abs(sc[j] - kth) <= tau for j in a ^ b)
    return {"rows": H * G, "differing": diff, "differing_by_near_ties": near,
            "tau": f"{tau_rel} * max|s| of the row"}


def bench_ball(args, dev, torch, ops, synth):
    w = synth.make(args.workload)
    N, H, d, ball, leaf = w.coords.shape[0], w.H, w.d, w.ball, w.leaf
    # the step's permutation: the GPU tree of the cloud, built before the
    # timed region
    perm = ops.bt_build(torch.from_numpy(w.coords).to(dev), leaf)
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
    # a plain device-to-device copy of known size: a measured bandwidth
    # reference, and the scale for HBM byte counters
    src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    copy_us = _event_us(torch, lambda: dst.copy_(src), 20, warm=4)
    copy_gbs = 2 * src.numel() / copy_us / 1e3
    del src, dst
    if args.eager:
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        print(json.dumps({"eager_launches": args.steps}), flush=True)
        return None
    # clock settle: back-to-back launches for about 0.3 s, then the warmup
    settle, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.settle_seconds:
        for i in range(50):
            step(i)
        settle += 50
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: exactly `steps` back-to-back launches on the current
    # stream (the one the library launches on), HIP events on that stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nsteps = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(nsteps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    host_el = time.perf_counter() - t0
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
    ms = attn_us * 1e-3
    line = {
        "metric": METRIC, "value": N / (ms * 1e-3), "unit": "points/s", "n_gpus": 1,
        "steps": nsteps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{args.workload}: ball attention over the cloud's ball tree "
                               f"(built on the GPU before the timed region; gather through "
                               f"it, scatter back), N={N}, ball {ball}, leaf {leaf}, H={H}, "
                               f"d={d}, {w.dtype}",
                   "N": N, "ball": ball, "leaf": leaf, "H": H, "d": d,
                   "input_sets_rotated": len(sets), "settle_launches": settle,
                   "timing": "exactly `steps` back-to-back launches on one stream between "
                             "two HIP events on that stream; value, ms_per_step and "
                             "roofline.achieved all come from that interval",
                   "host_wall_ms_per_step": host_el / nsteps * 1e3},
        "roofline": {"kernel": "ball_attn_mfma" if w.dtype == "bf16" else "ball_attn_valu",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": attn_bytes,
                     "peak_source": PEAK_SOURCE,
                     "measured_copy_GBps": copy_gbs,
                     "frac_of_measured_copy": achieved / copy_gbs},
        "ball_attn": {"us": attn_us, "us_graph_replay": graph_us,
                      "us_single_median": single[len(single) // 2], "us_single_min": single[0],
                      "points_per_s": N / (attn_us * 1e-6),
                      "tflops": attn_flops / (attn_us * 1e-6) / 1e12,
                      "mfma_frac": attn_flops / (attn_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS},
    }
    sel_check = {}
    if not args.no_side_rows:
        line["rows"] = side_rows(dev, torch, ops, synth, sel_check)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(w, args.cpu_seconds, sel_check or None)
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


def side_rows(dev, torch, ops, synth, sel_check=None):
    """The other rows of the path, timed in the same run on their own
    workloads: permute (gather and scatter of 512-byte rows at the rotated-
    pair size), coarsen / refine, the BSA steps, padded ball attention of an
    uneven N, the backward of ball attention, tree build + fp32 ball
    attention at 1,024 points, and the largest trees the GPU builder takes
    (8,192 points or padded slots, built by one workgroup in LDS)."""
    import numpy as np
    rows = {}
    # permute: N = 262,144 rows of H*d bf16 = 512 bytes; three source and
    # destination pairs (805 MB) rotate so that no call finds its rows in the
    # 256 MB Infinity Cache
    n, row = 262144, 8 * 32
    gen = torch.Generator(device=dev).manual_seed(4)
    srcs = [torch.randint(-32768, 32767, (n, row), dtype=torch.int16, device=dev, generator=gen)
            for _ in range(3)]
    dsts = [torch.empty_like(srcs[0]) for _ in range(3)]
    wr = synth.make("rotpair", features=False)               # the rotated tree B
    perm = ops.bt_rotate_build(torch.from_numpy(wr.coords).to(dev), wr.leaf, wr.R)
    nbytes = 2 * n * row * 2 + 4 * n
    for name, mode in (("gather", ops.BT_GATHER), ("scatter", ops.BT_SCATTER)):
        it = [0]

        def call():
            i = it[0] % 3
            it[0] += 1
            ops.bt_permute(srcs[i], perm, mode, dst=dsts[i])
        us = _event_us(torch, call, 60, warm=6)
        rows["a5_permute_" + name] = {"workload": "N=262144 rows of 512 B through the rotated "
                                                  "tree of the rotated-pair cloud",
                                      "us": us, "GBps": nbytes / us / 1e3,
                                      "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS}
    del srcs, dsts
    # coarsen / refine by 8 (Erwin's U-Net levels) at the sphere size: three
    # input sets rotate so that every call reads HBM
    n, H, d, s = 65536, 8, 32, 8
    xs = [torch.randint(-32768, 32767, (n, H, d), dtype=torch.int16, device=dev,
                        generator=gen).view(torch.bfloat16) for _ in range(3)]
    xs = [x.masked_fill(~torch.isfinite(x), 0) for x in xs]
    pc = ops.bt_build(torch.from_numpy(synth.make("sphere", features=False).coords).to(dev), 128)
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
        rows["f2_" + name] = {"workload": "N=65536, H=8, d=32 bf16, s=8, through the sphere's "
                                          "GPU tree (leaf 128)",
                              "us": us, "GBps": nbytes / us / 1e3,
                              "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS}
    del xs, cs, fs
    # BSA step
    w = synth.make("bsa")
    x = w.extra
    N, H, d = w.coords.shape[0], w.H, w.d
    p = ops.bt_build(torch.from_numpy(w.coords).to(dev), w.leaf)     # leaf 64: blocks are nodes
    bws = torch.empty(ops.bsa_workspace_size(N, H, d, w.ball, x["block"], x["group"], x["topk"]),
                      dtype=torch.uint8, device=dev)
    Wg = torch.from_numpy(w.gate_w).to(dev)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    out = torch.empty_like(q)
    # 200 warm-up steps (about 55 ms): the GPU idles while the workload is
    # generated on the host, and 20 steps do not bring its clocks back up
    us = _event_us(torch, lambda: ops.bsa_attn(q, k, v, p, w.ball, x["block"], x["group"],
                                               x["topk"], x["mask_own_ball"], gate_w=Wg,
                                               out=out, workspace=bws), 300, warm=200)
    flops = 4 * N * H * d * (w.ball + N // x["block"] + x["topk"] * x["block"])
    if sel_check is not None:
        _, sel = ops.bsa_attn(q, k, v, p, w.ball, x["block"], x["group"], x["topk"],
                              x["mask_own_ball"], gate_w=Wg, out=out, workspace=bws,
                              return_sel=True)
        sel_check.update(wb=w, perm=p.cpu().numpy(), sel_gpu=sel.cpu().numpy())
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
                    300, warm=100)
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
    # uneven N: 65,000 sphere points in the 65,536 slots of their padded GPU
    # tree (leaf 128; the 536 unused slots end up spread over the leaves),
    # masked ball attention; three input sets rotate
    n3, slots = 65000, 65536
    w = synth.make("sphere", n=n3)
    c3 = torch.from_numpy(w.coords).to(dev)
    us_pt = _event_us(torch, lambda: ops.bt_build_padded(c3, w.leaf), 20, warm=3)
    pp = ops.bt_build_padded(c3, w.leaf)
    assert pp.numel() == slots
    sets = [tuple(t.to(dev).clone() for t in (w.q, w.k, w.v)) for _ in range(3)]
    o3 = [torch.empty_like(sets[0][0]) for _ in range(3)]
    it = [0]

    def call3():
        i = it[0] % 3
        it[0] += 1
        ops.ball_attn_padded(*sets[i], pp, w.ball, out=o3[i])
    us3 = _event_us(torch, call3, 300, warm=100)
    nb3 = 4 * n3 * w.H * w.d * 2 + 4 * slots
    rows["f3_ball_attn_padded"] = {"workload": "N=65,000 in the 65,536 slots of the padded GPU "
                                                "tree, ball 128, H=8, d=32 bf16",
                                   "padded_tree_build_us": us_pt,
                                   "us": us3, "GBps": nb3 / us3 / 1e3,
                                   "hbm_frac": nb3 / us3 / 1e3 / HBM_PEAK_GBS}
    del sets, o3
    # backward of ball attention at the sphere size
    w = synth.make("sphere")
    gq, gk, gv = (t.to(dev) for t in (w.q, w.k, w.v))
    gdo = gq.clone()
    pb = ops.bt_build(torch.from_numpy(w.coords).to(dev), w.leaf)
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
    # the largest trees one workgroup builds in LDS: 8,192 sphere points
    # (leaf 64), the rotated tree of the rotated-pair recipe at 8,192 points
    # (leaf 128), and the pages' uneven clouds as padded trees
    w8 = synth.make("sphere", n=8192, features=False)
    c8 = torch.from_numpy(w8.coords).to(dev)
    wr = synth.make("rotpair", n=8192, features=False)
    cr = torch.from_numpy(wr.coords).to(dev)
    ws8 = torch.empty(256, dtype=torch.uint8, device=dev)
    p8 = torch.empty(8192, dtype=torch.int32, device=dev)
    us_8 = _event_us(torch, lambda: ops.bt_build(c8, 64, perm=p8, workspace=ws8), 100)
    us_r = _event_us(torch, lambda: ops.bt_rotate_build(cr, wr.leaf, wr.R, perm=p8, workspace=ws8),
                     100)
    rows["a1_a4_tree_lds_8192"] = {
        "workload": "N=8192: deformed sphere, leaf 64; rotated-pair recipe rotated, leaf 128",
        "build_us": us_8, "rotate_build_us": us_r, "points_per_s": 8192 / (us_8 * 1e-6),
        "bound": "latency (one 16-wave workgroup, all points in LDS; 12 B/point read, "
                 "4 B/point written)"}
    padded = {}
    for name, n_, leaf_ in (("shapenet_car_3586", 3586, 32), ("cosmology_5000", 5000, 64)):
        cp = torch.from_numpy(synth.deformed_sphere(np.random.default_rng(n_), n_)).to(dev)
        pp = torch.empty(ops.bt_padded_size(n_, leaf_), dtype=torch.int32, device=dev)
        padded[name] = {"slots": pp.numel(), "leaf": leaf_,
                        "build_us": _event_us(torch, lambda: ops.bt_build_padded(
                            cp, leaf_, perm=pp, workspace=ws8), 100)}
    rows["f3_tree_padded_pages_sizes"] = {"workload": "deformed-sphere clouds of the pages' "
                                          "uneven point counts", **padded,
                                          "bound": "latency (one workgroup)"}
    # tree builds at the configured sizes (nodes above 8,192 points split by
    # one workgroup each, streamed through the workspace; then one workgroup
    # per node in LDS).  Algorithmic bytes: the coordinates read once
    # (12 B/point), a 16-byte record read and written per point and level,
    # the permutation written (4 B/point).
    builds = {}
    for name, wl, leaf_, rot in (("sphere_leaf128", "sphere", 128, False),
                                 ("sphere_leaf64", "sphere", 64, False),
                                 ("rotpair", "rotpair", 128, False),
                                 ("rotpair_rotated", "rotpair", 128, True),
                                 ("cosmology", "cosmo", 256, False)):
        wt = synth.make(wl, features=False)
        n_ = wt.coords.shape[0]
        ct = torch.from_numpy(wt.coords).to(dev)
        wst = torch.empty(ops.bt_build_workspace_size(n_, leaf_), dtype=torch.uint8, device=dev)
        ptt = torch.empty(n_, dtype=torch.int32, device=dev)
        fn = (lambda: ops.bt_rotate_build(ct, leaf_, wt.R, perm=ptt, workspace=wst)) if rot else \
             (lambda: ops.bt_build(ct, leaf_, perm=ptt, workspace=wst))
        us_t = _event_us(torch, fn, 20, warm=3)
        levels = int(round(np.log2(n_ // leaf_)))
        alg = n_ * (12 + 32 * levels + 4)
        builds[name] = {"N": n_, "leaf": leaf_, "levels": levels, "build_us": us_t,
                        "points_per_s": n_ / (us_t * 1e-6), "algorithmic_bytes": alg,
                        "GBps": alg / us_t / 1e3, "hbm_frac": alg / us_t / 1e3 / HBM_PEAK_GBS,
                        # HBM bytes per build from FETCH_SIZE / WRITE_SIZE counters of
                        # its kernels (profiles/), null once tree.hip has changed
                        "traffic": _traffic(f"tree/{name}", ["tree.hip", "common.h"])}
        del ct, wst, ptt
    rows["a1_a4_tree_build"] = {"workload": "GPU ball trees of the sphere (65,536), rotated-pair "
                                            "(262,144) and cosmology (1,048,576) clouds",
                                **builds,
                                "bound": "latency of one workgroup per node at the top levels"}
    return rows


def bench_bsa(args, dev, torch, ops, synth):
    w = synth.make("bsa")
    x = w.extra
    N, H, d = w.coords.shape[0], w.H, w.d
    perm = ops.bt_build(torch.from_numpy(w.coords).to(dev), w.leaf)  # leaf 64: blocks are nodes
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
    ms = e0.elapsed_time(e1) / steps          # HIP events on the launching stream
    flops = 4 * N * H * d * (w.ball + N // x["block"] + x["topk"] * x["block"])
    return {"metric": "bsa points/sec", "value": N / (ms * 1e-3), "unit": "points/s",
            "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "bsa: BSA over the cloud's GPU ball tree (leaf 64, ball "
                                   "128, block 64, group 64, top-16), N=65536, H=8, d=32",
                       "timing": "back-to-back steps between two HIP events on the launching "
                                 "stream", "host_wall_ms_per_step": el / steps * 1e3},
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
                    help="with --rows-only: also run a plain device copy of known size "
                         "(counter scaling; the default line always times one)")
    ap.add_argument("--copy-probe-mb", type=int, default=128)
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="back-to-back launches before the warmup, for the clocks")
    ap.add_argument("--rows-only", action="store_true",
                    help="time only the other rows (permute, coarsen/refine, BSA, padded "
                         "attention, backward, small trees); for kernel traces and counters")
    args = ap.parse_args()
    # the CPU oracle's BLAS uses the host's cores (set before NumPy loads)
    ncores = str(len(os.sched_getaffinity(0)))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
        os.environ.setdefault(var, ncores)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    gpu_info = None if args.rows_only else _rocminfo_gpu()
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
        line["gpu_rocminfo"] = gpu_info        # the clock and CU count the peaks assume
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
