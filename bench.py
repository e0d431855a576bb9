"""Benchmark: paged-attention decode (split-KV partial + merge) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload long_context_fp16]

Prints ONE JSON line.  A step is one decode step of the whole batch: the
partial kernel over every chunk of every request plus the merge.  Inputs (Q,
K/V pools, page table, plan arrays, workspace) are resident in HBM before
timing; the plan is built outside the timed region, as the pages' microbench
does (PR #984, commit adding the three-way microbench).

The timed region is K back-to-back decode steps, bracketed by device
synchronization and HIP events on the launch stream, after --settle-ms of
untimed steps and W warmup steps (a GPU coming out of idle runs the first few
milliseconds of work about 5% slower).  Consecutive steps read
different copies of the K/V pools (3 by default, each larger than the 256 MB
last-level cache), so every step streams its KV bytes from HBM.  `value` =
algorithmic KV bytes / (region time / K).  The partial kernel alone is timed
the same way for the roofline entry; an isolated step after a 1 GiB cache
flush, bracketed by its own event pair, and back-to-back steps that all read
one pool copy ("warm") are reported for reference.

The GPU result is checked against the f64 oracle on the same inputs before
anything is reported (`parity`); the oracle's own time on the host cores is
`cpu_baseline`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV GB/s and % of HBM peak, paged decode B=4 ctx=32k GQA fp16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak, AMD published
LLC_BYTES = 256 << 20           # MI355X Infinity Cache: a read ceiling needs larger buffers
COUNTERS_FILE = os.path.join(ROOT, "profiles", "partial_long_context_fp16_counters.md")
PARTIAL_SRC = os.path.join(ROOT, "paged_attention_decode_amd", "csrc", "pd_partial.hip")


def kernel_sha() -> str:
    with open(PARTIAL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic():
    """HBM bytes per partial launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    vals = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sha") != kernel_sha():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--settle-ms", type=float, default=50.0,
                   help="untimed steps run for this long before the warmup steps of each "
                        "timed region (the GPU takes a few ms to leave its idle state)")
    p.add_argument("--workload", default="long_context_fp16",
                   choices=["long_context_fp16", "batched_fp16", "tiny_fp32", "cascade_fp16",
                            "token_sparse_fp16", "block_sparse_fp16", "mla_paged_fp16",
                            "dsa_sparse_fp16"])
    p.add_argument("--target-wgs", type=int, default=0, help="plan target (0: device default)")
    p.add_argument("--fixed-pages-per-chunk", type=int, default=0)
    p.add_argument("--mode", default="two-launch", choices=["fused", "two-launch"],
                   help="fused: one launch, the last chunk of each request merges; "
                        "two-launch: partial kernel then merge kernel")
    p.add_argument("--pool-copies", type=int, default=3,
                   help="independent K/V pool copies used in turn by consecutive steps")
    p.add_argument("--cascade-members", type=int, default=4,
                   help="cascade workload: requests sharing the prefix")
    p.add_argument("--cascade-prefix", type=int, default=8192,
                   help="cascade workload: shared prefix tokens")
    p.add_argument("--cascade-separate", action="store_true",
                   help="cascade workload: launch the shared and the per-request level "
                        "separately instead of as one grid")
    p.add_argument("--cascade-hpw", type=int, default=0,
                   help="cascade workload: KV heads per workgroup of the one-grid launch "
                        "(0: automatic)")
    p.add_argument("--cascade-l0-pages", type=int, default=0,
                   help="cascade workload: pages per chunk of the shared level (0: plan)")
    p.add_argument("--cascade-l1-pages", type=int, default=0,
                   help="cascade workload: pages per chunk of the per-request level (0: plan)")
    p.add_argument("--group-size", type=int, default=4,
                   help="long_context_fp16: query heads per KV head (8 KV heads; the metric "
                        "config is 4)")
    p.add_argument("--page-size", type=int, default=16,
                   help="long_context_fp16: tokens per page (the metric config is 16)")
    p.add_argument("--head-dim", type=int, default=128, choices=[64, 128],
                   help="long_context_fp16: head dim (the metric config is 128)")
    p.add_argument("--kernel-choice", type=int, default=0, choices=[0, 1, 2],
                   help="0 default kernels, 1 token kernel only, 2 no MFMA kernel")
    p.add_argument("--sweep-chunks", action="store_true",
                   help="also time the step at every power-of-two pages-per-chunk up to the "
                        "longest request (plus that length and the default plan's choice)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="wall-time budget of the oracle's single-thread run")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the streaming-read ceiling measurement")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (for counter calibration)")
    p.add_argument("--trace-graph", action="store_true",
                   help="time the step only: --steps eager steps, then --steps steps replayed "
                        "from HIP graphs of 30, in that order (for a kernel trace that "
                        "tells the two apart by dispatch order); flat workloads")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: measures one GPU only (the decode path has no "
              "cross-GPU exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_attention_decode_amd import binding as B
    from paged_attention_decode_amd import decode as PD
    from paged_attention_decode_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.load()
    B.paged_decode_set_kernel_choice(args.kernel_choice)
    dev = torch.device("cuda:0")
    if args.trace_graph and args.workload in ("block_sparse_fp16", "mla_paged_fp16",
                                              "dsa_sparse_fp16", "cascade_fp16"):
        print("bench.py: --trace-graph times the flat decode workloads", file=sys.stderr)
        sys.exit(2)
    if args.workload == "block_sparse_fp16":
        return block_sparse(args, torch, B, PD, workloads, dev)
    if args.workload in ("mla_paged_fp16", "dsa_sparse_fp16"):
        return mla(args, torch, B, PD, workloads, dev)
    t0 = time.time()
    if args.workload == "cascade_fp16":
        w = workloads.cascade_fp16(members=args.cascade_members, prefix_tokens=args.cascade_prefix)
    elif args.workload == "token_sparse_fp16":
        # the selection read through a page_size-1 table, one request per KV head
        w = workloads.folded_sparse(workloads.token_sparse_fp16())
    elif args.workload == "long_context_fp16":
        w = workloads.long_context_fp16(num_qo_heads=8 * args.group_size,
                                        page_size=args.page_size, head_dim=args.head_dim)
    else:
        w = getattr(workloads, args.workload)()
    pool_pages = w.k_pool.shape[0]
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            pool_pages)
    flat_runner = None
    if args.workload == "cascade_fp16":
        # detection over the page table picks the members and the shared span
        runner = PD.CascadeDecode(csr, page_size=w.page_size, num_pool_pages=pool_pages,
                                  num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                  head_dim=w.head_dim, target_wgs=args.target_wgs,
                                  pair_launch=not args.cascade_separate,
                                  heads_per_workgroup=args.cascade_hpw,
                                  fixed_pages_level0=args.cascade_l0_pages,
                                  fixed_pages_level1=args.cascade_l1_pages, device=dev)
        plan = runner.plan_summary()
        partial_only = None
        row_bytes = w.num_kv_heads * w.head_dim * 2 * 2
        span_tokens = runner.shared_pages * w.page_size if runner.active else 0
        reads = (len(runner.subgroups) if runner.active else 0) * span_tokens + \
            int(w.visible_tokens.sum()) - runner.member_req.size * span_tokens
        kv_bytes = reads * row_bytes
        # the flat decode of the same batch, timed the same way beside it
        flat_runner = PD.PagedDecode(csr, page_size=w.page_size, num_pool_pages=pool_pages,
                                     num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                     head_dim=w.head_dim, target_wgs=args.target_wgs, device=dev)
    else:
        runner = PD.PagedDecode(csr, page_size=w.page_size, num_pool_pages=pool_pages,
                                num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                head_dim=w.head_dim, target_wgs=args.target_wgs,
                                fixed_pages_per_chunk=args.fixed_pages_per_chunk,
                                fused=args.mode == "fused",
                                dtype=torch.float32 if w.dtype == "fp32" else torch.float16,
                                device=dev)
        plan = runner.plan_summary()
        plan["mode"] = args.mode
        partial_only = runner
        kv_bytes = w.kv_bytes()
    q = torch.from_numpy(w.q).to(dev)
    # independent copies of the K/V pools, used in turn by consecutive steps,
    # so that no step finds the previous step's KV in the 256 MB last-level
    # cache (each copy is larger than that cache)
    kv = [(torch.from_numpy(w.k_pool).to(dev), torch.from_numpy(w.v_pool).to(dev))]
    for _ in range(args.pool_copies - 1):
        kv.append((kv[0][0].clone(), kv[0][1].clone()))
    k, v = kv[0]
    flush = torch.empty(1 << 29, dtype=torch.float16, device=dev).normal_()   # 1 GiB
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step(i=0):
        kk, vv = kv[i % len(kv)]
        return runner.run(q, kk, vv, w.sm_scale)

    # parity gate before timing (the pages' bench refuses to time arms that disagree)
    out, lse = step()
    torch.cuda.synchronize()
    got_v = out.cpu().numpy().astype(np.float64)
    got_l = lse.cpu().numpy().astype(np.float64)

    import oracle
    ocsr = oracle.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                        w.page_size)
    cores = len(os.sched_getaffinity(0))
    tc = time.time()
    ref_v, ref_l = oracle.attention(w.q, w.k_pool, w.v_pool, ocsr, w.page_size, w.sm_scale,
                                    nthreads=cores)
    first_oracle_s = time.time() - tc
    tv, tl = (1e-5, 1e-5) if w.dtype == workloads.FP32 else (2e-3, 1e-3)
    dv = float(np.max(np.abs(got_v - ref_v)))
    fin = np.isfinite(ref_l)
    dl = float(np.max(np.abs(got_l[fin] - ref_l[fin]))) if fin.any() else 0.0
    parity_ok = dv <= tv and dl <= tl and np.array_equal(np.isneginf(got_l), ~fin)
    if not parity_ok:
        print(json.dumps({"error": "parity failed", "max_abs_v": dv, "max_abs_lse": dl}))
        sys.exit(1)

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    def run_steps(n, fn):
        """n back-to-back calls of fn(i), timed as one region (events on the
        launch stream and the wall clock, synchronized on both sides)."""
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        w0 = time.time()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n, (time.time() - w0) / n

    graph_steps = lambda n, fn: PD.graph_time(fn, n)   # noqa: E731

    def settle(fn):
        """Run fn back to back for --settle-ms of wall time (untimed): the
        first few ms of work after an idle period run measurably slower."""
        t_end = time.time() + args.settle_ms * 1e-3
        i = 0
        while time.time() < t_end:
            for _ in range(20):
                fn(i)
                i += 1
            torch.cuda.synchronize()

    if args.trace_graph:
        settle(step)
        run_steps(args.warmup, step)
        step_s, _ = run_steps(args.steps, step)
        g_step = graph_steps(args.steps, step)
        print(json.dumps({"workload": w.name, "plan": plan, "eager_step_us": round(step_s * 1e6, 2),
                          "graph_step_us": round(g_step * 1e6, 2),
                          "dispatch_order": "settle + %d warmup + %d timed eager steps; then "
                                            "3 eager steps, untimed replays of a 30-step graph "
                                            "for 50 ms, and %d timed replays" % (
                                                args.warmup, args.steps, max(1, args.steps // 30))}))
        return

    # settle and warmup, then the timed steps (the metric)
    settle(step)
    run_steps(args.warmup, step)
    step_s, wall_step_s = run_steps(args.steps, step)

    # the dominant kernel alone, back to back over the same pool copies
    part_s = None
    if partial_only is not None:
        if partial_only.fused:
            part_s = step_s
        else:
            kk = lambda i: kv[i % len(kv)]   # noqa: E731
            settle(lambda i: partial_only.partial(q, *kk(i), w.sm_scale))
            run_steps(args.warmup, lambda i: partial_only.partial(q, *kk(i), w.sm_scale))
            part_s, _ = run_steps(args.steps, lambda i: partial_only.partial(q, *kk(i), w.sm_scale))

    # the same step and partial replayed from HIP graphs (no host launch cost);
    # the graph's last replay must still agree with the oracle
    graph = None
    if partial_only is not None:
        g_step = graph_steps(args.steps, step)
        gv = runner.out.cpu().numpy().astype(np.float64)
        gl = runner.lse.cpu().numpy().astype(np.float64)
        g_ok = bool(np.max(np.abs(gv - ref_v)) <= tv and
                    np.array_equal(np.isneginf(gl), ~fin) and
                    (not fin.any() or np.max(np.abs(gl[fin] - ref_l[fin])) <= tl))
        graph = {"step_us": round(g_step * 1e6, 2), "parity_ok": g_ok}
        if not partial_only.fused:
            g_part = graph_steps(args.steps,
                                 lambda i: partial_only.partial(q, *kv[i % len(kv)], w.sm_scale))
            graph["partial_us"] = round(g_part * 1e6, 2)

    sweep = None
    if args.sweep_chunks and partial_only is not None:
        sweep = chunk_sweep(args, torch, PD, w, csr, q, kv, ref_v, ref_l, (tv, tl), run_steps,
                            settle, graph_steps, plan["pages_per_chunk"], dev)

    flat_s = None
    if flat_runner is not None:
        fstep = lambda i: flat_runner.run(q, *kv[i % len(kv)], w.sm_scale)   # noqa: E731
        settle(fstep)
        run_steps(args.warmup, fstep)
        flat_s, _ = run_steps(args.steps, fstep)
        # both arms replayed from HIP graphs (no host launch cost); the
        # cascade's last replay must still agree with the oracle
        g_casc = graph_steps(args.steps, step)
        gv = runner.out.cpu().numpy().astype(np.float64)
        g_casc_ok = bool(np.max(np.abs(gv - ref_v)) <= tv)
        g_flat = graph_steps(args.steps, fstep)

    # reference: one isolated step after a cache flush, bracketed by its own
    # events (includes the fixed cost of an event pair around a launch)
    iso = []
    for i in range(args.steps):
        flush.max()
        e0, e1 = ev(), ev()
        e0.record(stream)
        step(i)
        e1.record(stream)
        iso.append((e0, e1))
    torch.cuda.synchronize()
    iso_s = np.array([a.elapsed_time(b) * 1e-3 for a, b in iso])

    # reference: "warm" steps, back to back on one pool copy (whatever of it
    # the last-level cache keeps between steps is found there)
    warm = lambda i: runner.run(q, kv[0][0], kv[0][1], w.sm_scale)   # noqa: E731
    settle(warm)
    run_steps(args.warmup, warm)
    warm_s, _ = run_steps(args.steps, warm)

    value = kv_bytes / step_s / 1e9
    total_tokens = int(w.visible_tokens.sum())
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, random page ids from a 2x pool)",
        "config": {
            "workload": w.name, "batch": w.batch, "num_qo_heads": w.num_qo_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
            "visible_tokens": [int(x) for x in w.visible_tokens],
            "kv_bytes_per_step": int(kv_bytes), "accumulate": "fp32",
            "timing": "%d back-to-back decode steps (partial + merge) after %.0f ms of "
                      "untimed settle steps and %d warmup steps; step i reads K/V pool "
                      "copy i mod %d (%d x %.0f MB); events on the launch stream"
                      % (args.steps, args.settle_ms, args.warmup, len(kv), len(kv),
                         2 * w.k_pool.nbytes / 1e6),
            "plan": plan,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_tokens_per_s": round(total_tokens / step_s, 1),
        "step_us": round(step_s * 1e6, 2),
        "wall_step_us": round(wall_step_s * 1e6, 2),
        "isolated_flushed_step_us": {"mean": round(float(iso_s.mean()) * 1e6, 2),
                                     "p10": round(float(np.percentile(iso_s, 10)) * 1e6, 2),
                                     "p50": round(float(np.median(iso_s)) * 1e6, 2),
                                     "p90": round(float(np.percentile(iso_s, 90)) * 1e6, 2),
                                     "kv_gbs": round(kv_bytes / float(iso_s.mean()) / 1e9, 2)},
        "warm_step_us": round(warm_s * 1e6, 2),
        "setup_s": round(setup_s, 1),
        "parity": {"max_abs_v": dv, "max_abs_lse2": dl, "tol_v": tv, "tol_lse2": tl,
                   "ok": bool(parity_ok)},
    }
    if flat_s is not None:
        flat_bytes = w.kv_bytes()
        res["cascade_vs_flat"] = {
            "cascade_step_us": round(step_s * 1e6, 2), "flat_step_us": round(flat_s * 1e6, 2),
            "speedup": round(flat_s / step_s, 3), "cascade_kv_bytes": int(kv_bytes),
            "flat_kv_bytes": int(flat_bytes),
            "flat_kv_gbs": round(flat_bytes / flat_s / 1e9, 2),
            "graph_cascade_step_us": round(g_casc * 1e6, 2),
            "graph_flat_step_us": round(g_flat * 1e6, 2),
            "graph_speedup": round(g_flat / g_casc, 3), "graph_parity_ok": g_casc_ok,
            "flat_plan": flat_runner.plan_summary()}
    if sweep is not None:
        res["chunk_sweep"] = sweep
    if graph is not None:
        res["graph"] = graph
    if part_s is not None:
        achieved = kv_bytes / part_s / 1e9
        res["partial_us"] = round(part_s * 1e6, 2)
        res["merge_and_gap_us"] = round((step_s - part_s) * 1e6, 2)
        # the committed counter summary covers the default long-context run only
        default_run = (args.workload == "long_context_fp16" and args.group_size == 4 and
                       args.page_size == 16 and args.head_dim == 128 and
                       args.kernel_choice == 0)
        kind = B.paged_decode_kernel_kind(B.PD_DTYPE_FP16 if w.dtype == workloads.FP16 else
                                          B.PD_DTYPE_FP32, w.head_dim,
                                          w.num_qo_heads // w.num_kv_heads, w.page_size,
                                          w.k_pool.shape[2] * w.head_dim)
        res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": counter_traffic() if default_run else None,
                           "kernel_kind": {0: "token", 1: "page", 2: "mfma", 3: "mfma-any-page"}[kind],
                           "kernel": "paged_decode_partial", "kernel_sha": kernel_sha(),
                           "bytes_per_launch": int(kv_bytes)}
    else:
        # cascade: two partial launches (shared prefix, suffixes) and one merge
        # per step, so the figure covers the whole step
        achieved = kv_bytes / step_s / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": None, "scope": "step",
                           "kernel": "cascade step (prefix and suffix partial launches, merge)",
                           "kernel_sha": kernel_sha(), "bytes_per_launch": int(kv_bytes)}

    if partial_only is not None and not args.no_ceiling and \
            kv[0][0].numel() * kv[0][0].element_size() > LLC_BYTES:
        # the HBM read rate this GPU reaches with a plain streaming-read kernel,
        # over the same pool copies the decode reads, back to back
        res["roofline"]["measured_ceiling_gbs"], res["roofline"]["ceiling_probe"] = \
            read_ceiling(torch, B, kv, settle, run_steps, args)
        res["roofline"]["frac_of_measured_ceiling"] = round(
            res["roofline"]["achieved"] / res["roofline"]["measured_ceiling_gbs"], 4)

    if not args.no_cpu_baseline:
        # the oracle as it stands: the median of 3 runs on all host cores over
        # the whole step (the first run is the parity check's), then one run
        # on one thread over the whole step, or over its first requests if
        # that would take longer than --cpu-seconds
        ts = [first_oracle_s]
        for _ in range(2):
            tc = time.time()
            oracle.attention(w.q, w.k_pool, w.v_pool, ocsr, w.page_size, w.sm_scale,
                             nthreads=cores)
            ts.append(time.time() - tc)
        med = float(np.median(ts))
        rows = w.batch
        per_req = w.visible_tokens.astype(np.float64)
        est_1t = med * cores                      # single-thread estimate of the whole step
        while rows > 1 and est_1t * per_req[:rows].sum() / per_req.sum() > args.cpu_seconds:
            rows -= 1
        sub = oracle_subset(w, ocsr, rows)
        tc = time.time()
        oracle.attention(sub["q"], w.k_pool, w.v_pool, sub["csr"], w.page_size, w.sm_scale,
                         nthreads=1)
        t1 = time.time() - tc
        sub_bytes = kv_bytes * per_req[:rows].sum() / per_req.sum()
        res["cpu_baseline"] = {"value": round(kv_bytes / med / 1e9, 4), "unit": "GB/s",
                               "cores": cores, "kind": "oracle",
                               "sample": "the whole %s step (%d visible tokens, all heads), "
                                         "f64 oracle, median of %d runs: %.3f s wall"
                                         % (w.name, total_tokens, len(ts), med),
                               "runs_s": [round(t, 3) for t in ts],
                               "single_thread": {
                                   "value": round(sub_bytes / t1 / 1e9, 5), "unit": "GB/s",
                                   "cores": 1, "seconds": round(t1, 2),
                                   "sample": "requests 0..%d of the step (%d visible tokens)"
                                             % (rows - 1, int(per_req[:rows].sum()))},
                               "cpu_model": cpu_model()}

    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = int(src.numel() * 2)

    print(json.dumps(res), flush=True)




def chunk_sweep(args, torch, PD, w, csr, q, kv, ref_v, ref_l, tols, run_steps, settle,
                graph_steps, default_c, dev):
    """Step and partial time at each candidate pages-per-chunk (plans with the
    chunk size pinned); every candidate is checked against the oracle first."""
    rows = []
    for c in PD.chunk_candidates(csr["indptr"], default_c):
        r = PD.PagedDecode(csr, page_size=w.page_size, num_pool_pages=w.k_pool.shape[0],
                           num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                           head_dim=w.head_dim, fixed_pages_per_chunk=c,
                           dtype=torch.float32 if w.dtype == "fp32" else torch.float16,
                           device=dev)
        out, lse = r.run(q, *kv[0], w.sm_scale)
        torch.cuda.synchronize()
        gv = out.cpu().numpy().astype(np.float64)
        gl = lse.cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_l)
        ok = (float(np.max(np.abs(gv - ref_v))) <= tols[0] and
              (not fin.any() or float(np.max(np.abs(gl[fin] - ref_l[fin]))) <= tols[1]))
        if not ok:
            print(json.dumps({"error": "parity failed in the chunk sweep", "c": c}))
            sys.exit(1)
        fn = lambda i: r.run(q, *kv[i % len(kv)], w.sm_scale)   # noqa: E731
        settle(fn)
        run_steps(args.warmup, fn)
        st, _ = run_steps(args.steps, fn)
        pf = lambda i: r.partial(q, *kv[i % len(kv)], w.sm_scale)   # noqa: E731
        run_steps(args.warmup, pf)
        pt, _ = run_steps(args.steps, pf)
        gs = graph_steps(args.steps, fn)
        gp = graph_steps(args.steps, pf)
        rows.append({"pages_per_chunk": c, "num_chunks": r.info.num_chunks,
                     "units": r.info.num_wgs, "step_us": round(st * 1e6, 2),
                     "partial_us": round(pt * 1e6, 2), "graph_step_us": round(gs * 1e6, 2),
                     "graph_partial_us": round(gp * 1e6, 2), "default": c == default_c})
    return rows


def mla(args, torch, B, PD, workloads, dev):
    """Paged-MLA / DSA decode (second key stream): the step (partial + merge)
    and the partial alone, eager and replayed from a HIP graph, with the HBM
    and the matrix-core roofline of the partial kernel."""
    import oracle
    t0 = time.time()
    w = getattr(workloads, args.workload)()
    csr = B.paged_csr_build(w.block_tables, w.logical_start, w.written_len, w.page_size,
                            w.k_pool.shape[0])
    dec = PD.MlaDecode(csr, page_size=w.page_size, num_pool_pages=w.k_pool.shape[0],
                       num_qo_heads=w.num_qo_heads, dim=w.dim, extra_dim=w.extra_dim,
                       target_wgs=args.target_wgs,
                       fixed_pages_per_chunk=args.fixed_pages_per_chunk, device=dev)
    q, qx = torch.from_numpy(w.q).to(dev), torch.from_numpy(w.q_extra).to(dev)
    # pool copies used in turn, so the steps stream from HBM when the pools
    # exceed the last-level cache
    kv = [(torch.from_numpy(w.k_pool).to(dev), torch.from_numpy(w.k_extra_pool).to(dev))]
    for _ in range(args.pool_copies - 1):
        kv.append((kv[0][0].clone(), kv[0][1].clone()))
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    step = lambda i: dec.run(q, qx, *kv[i % len(kv)], w.sm_scale)   # noqa: E731
    part = lambda i: dec.partial(q, qx, *kv[i % len(kv)], w.sm_scale)   # noqa: E731
    out, lse = step(0)
    torch.cuda.synchronize()
    # parity on a sample of query heads (both q groups, every 16-head wave)
    sel = np.array([0, 21, 47, 63, 64, 90, 111, 127])
    sel = sel[sel < w.num_qo_heads]
    ocsr = oracle.csr_from_block_tables(w.block_tables, w.logical_start, w.written_len,
                                        w.page_size)
    cores = len(os.sched_getaffinity(0))
    tc = time.time()
    ref_v, ref_l = oracle.attention_mla(np.ascontiguousarray(w.q[:, sel]),
                                        np.ascontiguousarray(w.q_extra[:, sel]), w.k_pool,
                                        w.k_extra_pool, ocsr, w.page_size, w.sm_scale,
                                        nthreads=cores)
    oracle_s = time.time() - tc
    dv = float(np.max(np.abs(out.cpu().numpy()[:, sel] - ref_v)))
    dl = float(np.max(np.abs(lse.cpu().numpy()[:, sel] - ref_l)))
    if not (dv <= 2e-3 and dl <= 1e-3):
        print(json.dumps({"error": "parity failed", "max_abs_v": dv, "max_abs_lse": dl}))
        sys.exit(1)
    stream = torch.cuda.current_stream()

    def timed(fn):
        t_end = time.time() + args.settle_ms * 1e-3
        i = 0
        while time.time() < t_end:
            for _ in range(20):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / args.steps

    step_s = timed(step)
    part_s = timed(part)
    g_step = PD.graph_time(step, args.steps)
    g_part = PD.graph_time(part, args.steps)
    sweep = None
    if args.sweep_chunks:
        sweep = []
        for c in PD.chunk_candidates(csr["indptr"], dec.info.pages_per_chunk):
            r = PD.MlaDecode(csr, page_size=w.page_size, num_pool_pages=w.k_pool.shape[0],
                             num_qo_heads=w.num_qo_heads, dim=w.dim, extra_dim=w.extra_dim,
                             fixed_pages_per_chunk=c, device=dev)
            o2, l2 = r.run(q, qx, *kv[0], w.sm_scale)
            torch.cuda.synchronize()
            if not (float(np.max(np.abs(o2.cpu().numpy()[:, sel] - ref_v))) <= 2e-3 and
                    float(np.max(np.abs(l2.cpu().numpy()[:, sel] - ref_l))) <= 1e-3):
                print(json.dumps({"error": "parity failed in the chunk sweep", "c": c}))
                sys.exit(1)
            fs = lambda i: r.run(q, qx, *kv[i % len(kv)], w.sm_scale)   # noqa: E731
            sweep.append({"pages_per_chunk": c, "num_chunks": r.info.num_chunks,
                          "units": r.info.num_wgs,
                          "graph_step_us": round(PD.graph_time(fs, args.steps) * 1e6, 2),
                          "default": c == dec.info.pages_per_chunk})
    kv_bytes = w.kv_bytes()
    tokens = int(w.visible_tokens.sum())
    flops = tokens * w.num_qo_heads * 2 * (w.dim + w.extra_dim + w.dim)
    hbm = kv_bytes / part_s / 1e9
    tflops = flops / part_s / 1e12
    bound = "hbm" if kv_bytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_FP16_PEAK_TFLOPS * 1e12) \
        else "mfma"
    value = kv_bytes / step_s / 1e9
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) queries, latent and rope keys)",
        "config": {"workload": w.name, "batch": w.batch, "num_qo_heads": w.num_qo_heads,
                   "num_kv_heads": 1, "dim": w.dim, "extra_dim": w.extra_dim,
                   "row_stride": w.row_stride, "page_size": w.page_size,
                   "visible_tokens": [int(x) for x in w.visible_tokens],
                   "kv_bytes_per_step": int(kv_bytes), "flops_per_step": int(flops),
                   "accumulate": "fp32",
                   "timing": "%d back-to-back steps after %.0f ms of settle steps and %d "
                             "warmup steps; step i reads pool copy i mod %d; events on the "
                             "launch stream" % (args.steps, args.settle_ms, args.warmup,
                                                len(kv)),
                   "plan": dec.plan_summary()},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kv_tokens_per_s": round(tokens / step_s, 1),
        "step_us": round(step_s * 1e6, 2), "partial_us": round(part_s * 1e6, 2),
        "merge_and_gap_us": round((step_s - part_s) * 1e6, 2),
        "graph": {"step_us": round(g_step * 1e6, 2), "partial_us": round(g_part * 1e6, 2)},
        "setup_s": round(setup_s, 1),
        "parity": {"max_abs_v": dv, "max_abs_lse2": dl, "tol_v": 2e-3, "tol_lse2": 1e-3,
                   "ok": True, "heads_checked": sel.tolist()},
        "roofline": {"bound": bound,
                     "achieved": round(hbm, 2) if bound == "hbm" else round(tflops, 2),
                     "peak": HBM_PEAK_GBS if bound == "hbm" else MFMA_FP16_PEAK_TFLOPS,
                     "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                     "frac": round(hbm / HBM_PEAK_GBS if bound == "hbm"
                                   else tflops / MFMA_FP16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "paged_mla_decode_partial",
                     "hbm_gbs": round(hbm, 2), "hbm_frac": round(hbm / HBM_PEAK_GBS, 4),
                     "mfma_tflops": round(tflops, 2),
                     "mfma_frac": round(tflops / MFMA_FP16_PEAK_TFLOPS, 4),
                     "bytes_per_launch": int(kv_bytes), "flops_per_launch": int(flops)},
    }
    if sweep is not None:
        res["chunk_sweep"] = sweep
    if not args.no_cpu_baseline:
        scale = w.num_qo_heads / sel.size
        res["cpu_baseline"] = {"value": round(kv_bytes / (oracle_s * scale) / 1e9, 4),
                               "unit": "GB/s", "cores": cores, "kind": "oracle",
                               "sample": "%d of %d query heads over the whole step, f64 oracle, "
                                         "one run %.3f s, scaled to all heads"
                                         % (sel.size, w.num_qo_heads, oracle_s),
                               "cpu_model": cpu_model()}
    print(json.dumps(res), flush=True)


def block_sparse(args, torch, B, PD, workloads, dev):
    """Block-sparse decode (a selection of KV blocks per KV head): the
    block-granular page table (16-row pages, the default) timed beside the
    token-exact one and the one-page-per-block one."""
    import oracle
    w = workloads.block_sparse_fp16()
    b, hkv, cap, d = w.k_dense.shape
    hq = w.q.shape[1]
    kd = torch.from_numpy(w.k_dense).to(dev)
    vd = torch.from_numpy(w.v_dense).to(dev)
    q = torch.from_numpy(w.q).to(dev)
    ids = torch.from_numpy(w.block_ids).to(dev)
    arms = {False: dict(token_exact=False), True: dict(token_exact=True),
            "block": dict(token_exact=False, page_size=w.block_size)}
    runners = {k: PD.BlockSparseDecode(kd, vd, num_qo_heads=hq, block_size=w.block_size,
                                       blocks_per_request=w.block_ids.shape[1],
                                       kv_len=w.kv_len, target_wgs=args.target_wgs, device=dev,
                                       **kw)
               for k, kw in arms.items()}
    # parity of both granularities against attention over the selected positions
    g = hq // hkv
    t0 = time.time()
    ref_v = np.zeros((b, hq, d))
    ref_l = np.zeros((b, hq))
    pos = [oracle.block_positions(w.block_ids[h], w.block_size, w.kv_len[0]) for h in range(hkv)]
    for i in range(hq):
        h = i // g
        ref_v[0, i], ref_l[0, i] = oracle.attention_dense_f64(w.q[0, i], w.k_dense[0, h, pos[h]],
                                                              w.v_dense[0, h, pos[h]], w.sm_scale)
    oracle_s = time.time() - t0
    worst = (0.0, 0.0)
    for r in runners.values():
        out, lse = r.run(q, ids, w.sm_scale)
        torch.cuda.synchronize()
        dv = float(np.max(np.abs(out.cpu().numpy() - ref_v)))
        dl = float(np.max(np.abs(lse.cpu().numpy() - ref_l)))
        worst = (max(worst[0], dv), max(worst[1], dl))
    if not (worst[0] <= 2e-3 and worst[1] <= 1e-3):
        print(json.dumps({"error": "parity failed", "max_abs_v": worst[0], "max_abs_lse": worst[1]}))
        sys.exit(1)
    stream = torch.cuda.current_stream()

    def timed(fn):
        t_end = time.time() + args.settle_ms * 1e-3
        while time.time() < t_end:
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / args.steps

    t_block = timed(lambda: runners[False].run(q, ids, w.sm_scale))
    t_token = timed(lambda: runners[True].run(q, ids, w.sm_scale))
    t_whole = timed(lambda: runners["block"].run(q, ids, w.sm_scale))
    g_block = PD.graph_time(lambda i: runners[False].run(q, ids, w.sm_scale), args.steps)
    g_token = PD.graph_time(lambda i: runners[True].run(q, ids, w.sm_scale), args.steps)
    g_whole = PD.graph_time(lambda i: runners["block"].run(q, ids, w.sm_scale), args.steps)
    sweep = None
    if args.sweep_chunks:
        sweep = {}
        for exact in (False, True):
            rows = []
            for c in PD.chunk_candidates(runners[exact].dec.indptr,
                                         runners[exact].dec.info.pages_per_chunk):
                r = PD.BlockSparseDecode(kd, vd, num_qo_heads=hq, block_size=w.block_size,
                                         blocks_per_request=w.block_ids.shape[1],
                                         kv_len=w.kv_len, fixed_pages_per_chunk=c, device=dev,
                                         **arms[exact])
                out, lse = r.run(q, ids, w.sm_scale)
                torch.cuda.synchronize()
                if not (float(np.max(np.abs(out.cpu().numpy() - ref_v))) <= 2e-3 and
                        float(np.max(np.abs(lse.cpu().numpy() - ref_l))) <= 1e-3):
                    print(json.dumps({"error": "parity failed in the chunk sweep", "c": c}))
                    sys.exit(1)
                rows.append({"pages_per_chunk": c, "num_chunks": r.dec.info.num_chunks,
                             "step_us": round(timed(lambda: r.run(q, ids, w.sm_scale)) * 1e6, 2),
                             "graph_step_us": round(PD.graph_time(
                                 lambda i: r.run(q, ids, w.sm_scale), args.steps) * 1e6, 2),
                             "default": c == runners[exact].dec.info.pages_per_chunk})
            sweep["token_exact" if exact else "block_granular"] = rows
    tokens = sum(len(p) for p in pos)
    kv_bytes = tokens * d * 2 * 2
    value = kv_bytes / t_block / 1e9
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_block * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) Q/K/V, random distinct blocks plus the final block)",
        "config": {"workload": w.name, "batch": b, "num_qo_heads": hq, "num_kv_heads": hkv,
                   "head_dim": d, "block_size": w.block_size,
                   "blocks_per_kv_head": int(w.block_ids.shape[1]), "kv_len": int(w.kv_len[0]),
                   "selected_positions": int(tokens), "kv_bytes_per_step": int(kv_bytes),
                   "timing": "%d back-to-back steps (block-id expansion + partial + merge) "
                             "after %.0f ms of settle steps; K/V resident (fits the last-level "
                             "cache)" % (args.steps, args.settle_ms),
                   "plan": runners[False].plan_summary()},
        "step_us": round(t_block * 1e6, 2),
        "block_vs_token": {"block_granular_step_us": round(t_block * 1e6, 2),
                           "token_exact_step_us": round(t_token * 1e6, 2),
                           "one_page_per_block_step_us": round(t_whole * 1e6, 2),
                           "speedup": round(t_token / t_block, 3),
                           "graph_block_granular_step_us": round(g_block * 1e6, 2),
                           "graph_token_exact_step_us": round(g_token * 1e6, 2),
                           "graph_one_page_per_block_step_us": round(g_whole * 1e6, 2),
                           "token_exact_plan": runners[True].plan_summary(),
                           "one_page_per_block_plan": runners["block"].plan_summary()},
        "parity": {"max_abs_v": worst[0], "max_abs_lse2": worst[1], "tol_v": 2e-3,
                   "tol_lse2": 1e-3, "ok": True},
        # three launches per step (block-id expansion, partial, merge) over K/V
        # that fits the last-level cache: the figure covers the whole step
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
                     "scope": "step",
                     "kernel": "block-selection step (block-id expansion, partial, merge)",
                     "kernel_sha": kernel_sha(), "bytes_per_launch": int(kv_bytes)},
    }
    if sweep is not None:
        res["chunk_sweep"] = sweep
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = {"value": round(kv_bytes / oracle_s / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": "the whole step (%d selected positions x %d KV heads),"
                                         " f64 dense-position oracle, one run, %.3f s"
                                         % (tokens // hkv, hkv, oracle_s),
                               "cpu_model": cpu_model()}
    print(json.dumps(res), flush=True)


def read_ceiling(torch, B, kv, settle, run_steps, args):
    """Best read rate of the streaming-read probe over the K pool copies
    (each larger than the last-level cache), step i reading copy i mod n, at
    a few grid sizes; returns (GB/s, per-grid-size table)."""
    dev = kv[0][0].device
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = kv[0][0].numel() * kv[0][0].element_size()
    table = {}
    for nt in (True, False):
        for per_cu in (0.5, 1, 2, 4):
            wgs = max(1, int(cus * per_cu))
            sink = torch.empty(wgs, dtype=torch.int32, device=dev)
            fn = lambda i: B.paged_hbm_read_probe(kv[i % len(kv)][0], nbytes, wgs, sink, nt)  # noqa
            settle(fn)
            run_steps(args.warmup, fn)
            t, _ = run_steps(args.steps, fn)
            table["%s x%d" % ("nt" if nt else "plain", wgs)] = round(nbytes / t / 1e9, 1)
    return max(table.values()), {"bytes_per_launch": int(nbytes), "gbs_by_launch": table,
                                 "kernel": "paged_hbm_read_probe (16-byte loads, 512 threads, "
                                           "one contiguous segment per workgroup)"}


def oracle_subset(w, ocsr, rows):
    """The first `rows` requests of the oracle's CSR and their queries."""
    ip = np.asarray(ocsr["indptr"])
    csr = dict(indptr=ip[:rows + 1].copy(), indices=np.asarray(ocsr["indices"])[:ip[rows]],
               last_page_len=np.asarray(ocsr["last_page_len"])[:rows],
               first_page_offset=np.asarray(ocsr["first_page_offset"])[:rows])
    return {"q": np.ascontiguousarray(w.q[:rows]), "csr": csr}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
