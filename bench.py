#!/usr/bin/env python3
"""Benchmark: MoE dispatch + combine on one MI355X, virtual EP ranks.

A step is one pass of the whole hot path over one batch: ep_get_layout ->
ep_dispatch -> ep_combine, inputs resident in HBM.  The three calls only
enqueue kernels, so by default the step is captured once into a HIP graph and
the timed region replays one HIP graph of the K steps (--eager launches every
call from Python instead).  The default workload is the
prefill shape: 4096 tokens x hidden 7168 bf16, 256 experts in 8 groups, top-4
groups then top-8 experts, 8 virtual ranks, expert_alignment 128.  Expert
outputs are a separate seeded bf16 buffer (what an expert GEMM would have
written), so combine does not read the rows dispatch just wrote.

Metric: dispatch+combine algorithmic HBM bytes per step / step time (GB/s), and
tokens/s.  Algorithmic bytes: dispatch 2NH + 2NKH (bf16) or 2NH + NKH +
4NK(H/128) (e4m3), combine 2NKH + 2NH.  Layout time counts inside the step.

Prints ONE JSON line.  Extra keys beside the required ones: tokens_per_s,
hbm_frac, per-kernel times, the roofline of the dominant kernel, the HBM
ceilings measured on the same box (linear copy / write / read, and dispatch's
and combine's own access patterns on the workload's slot map) with each
kernel's fraction of its pattern's ceiling, cold-cache step times and
cold-cache times of each call alone (median / p10 / p90, a 1 GiB flush before
each), the same step times after a 1 GiB write pass (dirty caches), the
device's clocks, and the CPU oracle baseline (threaded and single-threaded).
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "dispatch+combine HBM GB/s and % of peak; tokens/s at 4096×7168 top-8"
KERNEL_SRC = os.path.join(ROOT, "combine_ep_get_amd", "csrc", "ep_get.hip")


def algorithmic_bytes(w):
    N, H, K = w.N, w.H, w.K
    if w.fp8:
        disp = 2 * N * H + N * K * H + 4 * N * K * (H // 128)
    else:
        disp = 2 * N * H + 2 * N * K * H
    comb = 2 * N * K * H + 2 * N * H
    return disp, comb


def source_sha():
    """sha256 of the kernel source with comments and blank space removed, so
    that edits to comments alone do not mark the counter summaries stale."""
    src = open(KERNEL_SRC).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprof counter summary, or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = dict(re.findall(r"^(\w+):\s*(\S+)", open(path).read(), flags=re.M))
    if kv.get("source_sha256") != source_sha():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _cpu_info():
    """Model name and a few identifying fields of the host CPU (/proc/cpuinfo)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if info:
                    break
                continue
            k, v = (t.strip() for t in line.split(":", 1))
            if k in ("model name", "cpu family", "model", "stepping", "cpu MHz") and k not in info:
                info[k] = v
    except OSError:
        pass
    return info


def oracle_threads():
    """CPUs this process may use, at most 16 (a GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, inp, eo_bits, budget_s):
    """The oracle as it stands on the same batch, timed on this host: single
    threaded, and through its threaded driver (layout and slot tags serial,
    dispatch and combine over token ranges on every usable CPU, at most 16).
    Each form runs full steps for about half of ``budget_s``; the outputs of
    the two forms' last steps are compared byte for byte."""
    import oracle
    cap = oracle.capacity(w.N, w.K, w.E, w.A)
    disp_b, comb_b = algorithmic_bytes(w)

    def step(th):
        lay = oracle.layout(inp["topk_idx"], w.E, w.R, w.A)
        if w.fp8:
            d = oracle.dispatch_fp8(inp["x"], lay["slot_of"], cap, threads=th)
        else:
            d = (oracle.dispatch_bf16(inp["x"], lay["slot_of"], cap, threads=th),)
        meta = oracle.recv_meta(lay["slot_of"], inp["topk_weights"], cap)
        y = oracle.combine(eo_bits, lay["slot_of"], inp["topk_weights"], threads=th)
        return [lay["slot_of"], *d, *meta, *y]

    def timed(th):
        reps, t_total, out = 0, 0.0, None
        while t_total < budget_s / 2 or reps == 0:
            out = None
            t0 = time.perf_counter()
            out = step(th)
            t_total += time.perf_counter() - t0
            reps += 1
        return t_total / reps, reps, out

    nth = oracle_threads()
    s1, r1, o1 = timed(1)
    sn, rn, on = timed(nth)
    identical = all(np.array_equal(a.view(np.uint8), b.view(np.uint8)) for a, b in zip(o1, on))
    del o1, on

    def row(step_s, reps, th):
        return {"value": round((disp_b + comb_b) / step_s / 1e9, 3), "unit": "GB/s",
                "cores": th, "tokens_per_s": round(w.N / step_s, 1),
                "ms_per_step": round(step_s * 1e3, 1), "steps": reps}

    res = {"kind": "oracle", **row(sn, rn, nth),
           "sample": f"full steps (layout + dispatch + slot tags + combine) of the {w.name} batch, "
                     f"{w.N} tokens: {rn} with the threaded driver ({nth} threads: layout and "
                     f"tags serial, dispatch and combine over token ranges), {r1} single-"
                     f"threaded; same algorithmic bytes as the GPU figure",
           "single_thread": row(s1, r1, 1),
           "threaded_identical_to_single": bool(identical),
           "cpu": _cpu_info(), "host_cpus": os.cpu_count()}
    return res


def ceilings(per_launch_ms, w, slot_of, x, recv_x, eo, nbytes=1 << 30):
    """What this GPU's HBM delivers, timed like the EP kernels (a graph of
    back-to-back launches): linear copy / write / read over 1 GiB with four or
    one 16-byte accesses per thread, and the two traffic patterns of the path
    on the workload's own slot map -- dispatch's (each token row read once and
    written to its K slots; one wavefront per token, LDS-staged 2 KiB pieces
    (the dispatch kernel's form), and XCD-placed (token, k, piece)
    workgroups, which only win while the rows are in the Infinity Cache) and
    combine's (K slot rows gathered, one row written) --
    with no arithmetic.  GB/s of the patterns use the same algorithmic bytes
    as the kernels they bound."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_ep_get_amd", "_lib", "libepceil.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.epc_copy_p.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    lib.epc_write_p.argtypes = [vp, i64, ctypes.c_uint32, ctypes.c_int, vp]
    lib.epc_read_p.argtypes = [vp, i64, ctypes.c_int, vp, vp]
    lib.epc_scatter.argtypes = [vp, vp, vp, i32, i32, i64, vp]
    lib.epc_scatter_items.argtypes = [vp, vp, vp, i32, i32, i64, vp]
    lib.epc_scatter_pieces.argtypes = [vp, vp, vp, i32, i32, i64, vp]
    lib.epc_gather.argtypes = [vp, vp, vp, i32, i32, i64, vp]

    def cur():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    a = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(256, dtype=torch.int32, device="cuda")
    res = {}
    for name, fn, moved in (
            ("copy", lambda: lib.epc_copy_p(b.data_ptr(), a.data_ptr(), nbytes, 4, cur()), 2),
            ("copy1", lambda: lib.epc_copy_p(b.data_ptr(), a.data_ptr(), nbytes, 1, cur()), 2),
            ("write", lambda: lib.epc_write_p(a.data_ptr(), nbytes, 7, 4, cur()), 1),
            ("write1", lambda: lib.epc_write_p(a.data_ptr(), nbytes, 7, 1, cur()), 1),
            ("read", lambda: lib.epc_read_p(a.data_ptr(), nbytes, 4, sink.data_ptr(), cur()), 1),
            ("read1", lambda: lib.epc_read_p(a.data_ptr(), nbytes, 1, sink.data_ptr(), cur()), 1)):
        assert fn() == 0
        res[name + "_gbs"] = round(moved * nbytes / (per_launch_ms(fn) * 1e-3) / 1e9, 1)
    del a, b
    disp_b, comb_b = algorithmic_bytes(w)
    row_b = 2 * w.H
    if not w.fp8 and row_b <= 16384:
        fn = lambda: lib.epc_scatter(x.data_ptr(), recv_x.data_ptr(), slot_of.data_ptr(),  # noqa: E731
                                     w.N, w.K, row_b, cur())
        assert fn() == 0
        res["scatter_gbs"] = round(disp_b / (per_launch_ms(fn) * 1e-3) / 1e9, 1)
        fn = lambda: lib.epc_scatter_items(x.data_ptr(), recv_x.data_ptr(),  # noqa: E731
                                           slot_of.data_ptr(), w.N, w.K, row_b, cur())
        assert fn() == 0
        res["scatter_items_gbs"] = round(disp_b / (per_launch_ms(fn) * 1e-3) / 1e9, 1)
        fn = lambda: lib.epc_scatter_pieces(x.data_ptr(), recv_x.data_ptr(),  # noqa: E731
                                            slot_of.data_ptr(), w.N, w.K, row_b, cur())
        assert fn() == 0
        res["scatter_pieces_gbs"] = round(disp_b / (per_launch_ms(fn) * 1e-3) / 1e9, 1)
    if w.K <= 8 and row_b <= 16384:
        yt = torch.empty((w.N, w.H), dtype=torch.bfloat16, device="cuda")
        fn = lambda: lib.epc_gather(eo.data_ptr(), yt.data_ptr(), slot_of.data_ptr(),  # noqa: E731
                                    w.N, w.K, row_b, cur())
        assert fn() == 0
        res["gather_gbs"] = round(comb_b / (per_launch_ms(fn) * 1e-3) / 1e9, 1)
    return res


def lds_info():
    """LDS per workgroup (what a CU-budget workgroup reserves) and per CU."""
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_ep_get_amd", "_lib", "libepceil.so"))
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    if lib.epc_lds_info(ctypes.byref(a), ctypes.byref(b)) != 0:
        return None
    res = {"lds_per_workgroup": a.value, "lds_per_cu": b.value}
    c, m, bw = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    if lib.epc_clock_info(ctypes.byref(c), ctypes.byref(m), ctypes.byref(bw)) == 0:
        res.update({"core_clock_mhz": round(c.value / 1e3), "memory_clock_mhz": round(m.value / 1e3),
                    "memory_bus_bits": bw.value})
    return res


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize(args):
    """Write the profiles/ summaries from three rocprofv3 output directories:
    --kernel-trace --stats (trace), --pmc FETCH_SIZE (fetch), --pmc WRITE_SIZE
    (write), all taken on `bench.py --config <id>`.  Counter values are KiB per
    dispatch; each is scaled by what the same counter reads for the benchmark's
    1 GiB plain copy kernel (ceiling measurement) in the same run."""
    from combine_ep_get_amd import workloads as wl
    w = wl.CONFIGS[args.config]
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    # the profiles are taken from /tmp (rocprofv3 writes its scratch there), so
    # bench.py is named by its path; <repo> stands for the repository root
    cmd_base = f"python3 <repo>/bench.py --config {args.config}"
    # kernel trace statistics
    stats = _csv_rows(os.path.join(args.trace_dir, "run_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel statistics: {w.desc}",
             f"# command: cd /tmp && rocprofv3 --kernel-trace --stats -T -f csv -d <out> -o run -- "
             f"{cmd_base} --steps 20 --warmup 5 --cpu-seconds 0 --no-ceiling --cold-steps 0",
             "# <repo> is the repository root; the command runs from /tmp",
             f"# kernel source sha256 (comments and blank space stripped): {source_sha()}",
             f"{'kernel':28s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in stats:
        lines.append(f"{r['Name'][:28]:28s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                     f"{float(r['Percentage']):6.2f}")
    step_us = sum(float(r["AverageNs"]) for r in stats
                  if r["Name"].startswith(("layout_", "dispatch_", "combine_"))) / 1e3
    lines.append(f"sum of per-step kernel averages: {step_us:.2f} us")
    open(os.path.join(out_dir, f"kernel_trace_{w.name}.txt"), "w").write("\n".join(lines) + "\n")

    if not (args.fetch_dir and args.write_dir):
        print(f"wrote the kernel trace summary for {w.name}")
        return

    def per_kernel(path):
        acc = {}
        for r in _csv_rows(path):
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch = per_kernel(os.path.join(args.fetch_dir, "run_counter_collection.csv"))
    write = per_kernel(os.path.join(args.write_dir, "run_counter_collection.csv"))
    copy_kib = (1 << 30) / 1024.0
    f_scale = copy_kib / fetch["copy_kernel"]
    w_scale = copy_kib / write["copy_kernel"]
    disp_b, comb_b = algorithmic_bytes(w)
    dk = "dispatch_fp8_item_kernel" if w.fp8 else "dispatch_piece_kernel"
    for short, kname, alg in (("dispatch_fp8" if w.fp8 else "dispatch_bf16", dk, disp_b),
                              ("combine", "combine_piece_k_kernel", comb_b)):
        fb = fetch[kname] * f_scale * 1024
        wb = write[kname] * w_scale * 1024
        txt = [f"# HBM byte audit (rocprofv3 --pmc), {kname}, {w.desc}",
               f"# commands: cd /tmp && rocprofv3 --pmc FETCH_SIZE -T -f csv -d <out> -o run -- "
               f"{cmd_base} --steps 3 --warmup 1 --cpu-seconds 0 --cold-steps 0",
               f"#           cd /tmp && rocprofv3 --pmc WRITE_SIZE -T -f csv -d <out> -o run -- "
               f"{cmd_base} --steps 3 --warmup 1 --cpu-seconds 0 --cold-steps 0",
               "# <repo> is the repository root; the commands run from /tmp",
               "# scale: counter KiB of the 1 GiB copy kernel in the same run -> bytes",
               "# source_sha256: ep_get.hip with comments and blank space stripped",
               f"kernel: {kname}",
               f"workload: {w.name}",
               f"source_sha256: {source_sha()}",
               f"fetch_kib_per_dispatch: {fetch[kname]:.1f}",
               f"write_kib_per_dispatch: {write[kname]:.1f}",
               f"copy_kernel_fetch_kib: {fetch['copy_kernel']:.1f}",
               f"copy_kernel_write_kib: {write['copy_kernel']:.1f}",
               f"fetch_scale: {f_scale:.5f}",
               f"write_scale: {w_scale:.5f}",
               f"fetch_bytes_per_launch: {fb:.0f}",
               f"write_bytes_per_launch: {wb:.0f}",
               f"traffic_bytes_per_launch: {fb + wb:.0f}",
               f"algorithmic_bytes_per_launch: {alg}",
               f"traffic_over_algorithmic: {(fb + wb) / alg:.4f}"]
        open(os.path.join(out_dir, f"traffic_{short}_{w.name}.txt"), "w").write("\n".join(txt) + "\n")
    print(f"wrote profiles for {w.name}")


def overlap_gemm(args, step, capture):
    """Time K steps (one HIP graph) alone, K bf16 GEMMs alone (eager, on a
    second stream) and both at once, each from one start event to the end of
    both streams."""
    import torch
    m, k, n = (int(v) for v in args.overlap_gemm.lower().split("x"))
    gen = torch.Generator(device="cpu").manual_seed(7)
    a = torch.randn((m, k), generator=gen).to(torch.bfloat16).cuda()
    b = torch.randn((k, n), generator=gen).to(torch.bfloat16).cuda()
    c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    reps = args.steps
    g = capture(step, reps)
    main_s = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def gemms():
        with torch.cuda.stream(side):
            for _ in range(reps):
                torch.mm(a, b, out=c)

    def timed(run_step, run_gemm):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main_s)
        side.wait_event(e0)
        if run_step:
            g.replay()
        if run_gemm:
            gemms()
        done = torch.cuda.Event()
        done.record(side)
        main_s.wait_event(done)
        e1.record(main_s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    timed(True, True)   # warm both paths
    step_ms = timed(True, False)
    gemm_ms = timed(False, True)
    both_ms = timed(True, True)
    tflop = 2.0 * m * k * n / 1e12
    return {"gemm": f"bf16 [{m},{k}]x[{k},{n}]", "cu_budget": args.cu_budget,
            "step_ms": round(step_ms, 4), "gemm_ms": round(gemm_ms, 4),
            "both_ms": round(both_ms, 4),
            "gemm_tflops_alone": round(tflop / (gemm_ms * 1e-3), 1),
            "overlap_saving": round(1.0 - both_ms / (step_ms + gemm_ms), 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="workload id 1..5 (default 3, prefill)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle baseline budget; 0 skips it")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--ll", type=int, default=0, metavar="M",
                    help="low-latency path: ep_ll_dispatch (routing + payload in one launch, "
                         "M rows per (expert, source) sub-block) + ep_combine")
    ap.add_argument("--cu-budget", type=int, default=0, metavar="N",
                    help="run dispatch and combine on at most N CUs (persistent grids, one "
                         "workgroup per CU); 0 = whole GPU")
    ap.add_argument("--overlap-gemm", default="", metavar="MxKxN",
                    help="also time the K steps concurrently with K bf16 GEMMs "
                         "[M,K]x[K,N] on a second stream (e.g. 8192x7168x4096)")
    ap.add_argument("--cold-steps", type=int, default=50, metavar="C",
                    help="also time C single steps, each after an untimed pass over 1 GiB "
                         "that evicts L2 and the Infinity Cache (0 skips)")
    ap.add_argument("--cold-flush", choices=("read", "write"), default="read",
                    help="the eviction pass: read (leaves clean lines) or write (leaves "
                         "dirty lines that are written back during the step)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every call from Python instead of replaying a HIP graph")
    ap.add_argument("--summarize", action="store_true",
                    help="write profiles/ summaries from rocprofv3 output dirs and exit")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return

    if args.gpus != 1:
        print(f"bench.py: this implementation runs on one GPU only (virtual EP ranks inside one GPU's "
              f"HBM); --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_ep_get_amd as ep
    from combine_ep_get_amd import workloads as wl

    w = wl.CONFIGS[args.config]
    print(f"[bench] {w.desc}", file=sys.stderr, flush=True)
    inp = wl.make_inputs(w, args.seed)
    cap = ep.recv_capacity(w.N, w.K, w.E, w.R, w.A)
    eo_bits = wl.make_expert_out(w, cap, args.seed)
    dev = torch.device("cuda")
    idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    wts = torch.from_numpy(inp["topk_weights"]).to(dev)
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(dev)
    eo = torch.from_numpy(eo_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device=dev)
    if args.ll:
        ll_out = ep.alloc_ll(w.N, w.K, w.E, w.R, args.ll, w.H, w.fp8, dev)
        lay = ll_out[0]
        # expert outputs: seeded rows placed at the slots the routing uses (the
        # sub-blocks' unused rows are never read)
        ep.ll_dispatch(x, idx, wts, w.E, w.R, args.ll, w.fp8, out=ll_out)
        used = lay.slot_of.flatten().long()
        used = used[used >= 0]
        rows = torch.from_numpy(wl.make_expert_out(w, int(used.numel()), args.seed)
                                .view(np.int16)).view(torch.bfloat16).to(dev)
        eo = torch.zeros((lay.capacity, w.H), dtype=torch.bfloat16, device=dev)
        eo.index_copy_(0, used, rows)
    else:
        lay = ep.alloc_layout(w.N, w.K, w.E, w.R, w.A, dev)
        recv = ep.alloc_recv(lay, w.H, w.fp8, dev)
    torch.cuda.synchronize()

    def do_layout():
        ep.get_layout(idx, w.E, w.R, w.A, out=lay)

    def do_dispatch():
        if args.ll:
            ep.ll_dispatch(x, idx, wts, w.E, w.R, args.ll, w.fp8, out=ll_out)
        else:
            ep.dispatch(x, wts, lay, w.fp8, out=recv, cu_budget=args.cu_budget)

    def do_combine():
        ep.combine(eo, lay, wts, out=y, cu_budget=args.cu_budget)

    def step():
        if not args.ll:
            do_layout()
        do_dispatch()
        do_combine()

    def capture(fn, reps):
        """HIP graph of `reps` back-to-back calls of fn (the library only
        enqueues kernels on the current stream, so the calls capture)."""
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                for _ in range(reps):
                    fn()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        return g

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if not args.eager:
        # one graph holding the W warmup steps, one holding the K timed steps
        warm_graph = capture(step, max(args.warmup, 1))
        timed_graph = capture(step, args.steps)
        warm_graph.replay()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps "
          f"({'eager' if args.eager else 'one HIP graph of K steps'})", file=sys.stderr,
          flush=True)
    # The timed region: K back-to-back steps, nothing else enqueued between them.
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    if args.eager:
        for i in range(args.steps):
            step()
    else:
        timed_graph.replay()
    g1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    gpu_step_ms = g0.elapsed_time(g1) / args.steps

    # Per-kernel durations: each kernel launched `steps` times back to back
    # (one HIP graph of `steps` launches, replayed between two events on the
    # stream the library launches on), with the inputs the timed steps used.
    def per_launch_ms(fn):
        reps = args.steps
        if args.eager:
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
        else:
            g = capture(fn, reps)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # Cold-cache steps: one step at a time, each after an untimed pass over
    # 1 GiB (more than the 256 MB Infinity Cache plus the L2s), timed by events
    # on the launch stream; median and spread over the steps.
    cold = None
    if args.cold_steps > 0:
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_steps)]
        for i, (a, b) in enumerate(evs):
            if args.cold_flush == "read":
                flush.sum(dtype=torch.int64)
            else:
                flush.fill_(i)
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])

        def spread(v):
            return {"median_us": round(float(np.median(v)), 2),
                    "p10_us": round(float(np.percentile(v, 10)), 2),
                    "p90_us": round(float(np.percentile(v, 90)), 2)}

        # each call of the step alone, after its own flush (the inputs of the
        # later calls are the outputs the steps above left)
        per_call = {}
        calls = (("dispatch", do_dispatch), ("combine", do_combine))
        if not args.ll:
            calls = (("layout", do_layout),) + calls
        for name, fn in calls:
            ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.cold_steps)]
            for i, (a, b) in enumerate(ce):
                if args.cold_flush == "read":
                    flush.sum(dtype=torch.int64)
                else:
                    flush.fill_(i)
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            per_call[name] = spread(np.array([a.elapsed_time(b) * 1e3 for a, b in ce]))
        # whole steps after the other kind of pass too: a write pass leaves
        # dirty lines of other data in the caches, which the step then pays for
        other = "write" if args.cold_flush == "read" else "read"
        oe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.cold_steps)]
        for i, (a, b) in enumerate(oe):
            if other == "read":
                flush.sum(dtype=torch.int64)
            else:
                flush.fill_(i)
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        other_us = np.array([a.elapsed_time(b) * 1e3 for a, b in oe])
        del flush
        disp_b0, comb_b0 = algorithmic_bytes(w)
        cold = dict(spread(us))
        cold.update({"gbs_at_median": round((disp_b0 + comb_b0) / (np.median(us) * 1e-6) / 1e9, 1),
                     "steps": args.cold_steps,
                     "flush": f"1 GiB {args.cold_flush} before each step or call, untimed",
                     "per_call": per_call,
                     f"after_{other}_flush": spread(other_us)})

    lay_ms = 0.0 if args.ll else per_launch_ms(do_layout)
    dis_ms = per_launch_ms(do_dispatch)
    com_ms = per_launch_ms(do_combine)

    disp_b, comb_b = algorithmic_bytes(w)
    total_b = disp_b + comb_b
    gbs = total_b / step_s / 1e9
    if dis_ms >= com_ms:
        dom_b, dom_ms = disp_b, dis_ms
        dom_kernel = "dispatch_fp8" if w.fp8 else "dispatch_bf16"
        if args.ll:
            dom_kernel = "ll_dispatch_fp8" if w.fp8 else "ll_dispatch_bf16"
    else:
        dom_b, dom_ms = comb_b, com_ms
        dom_kernel = "combine"
    achieved = dom_b / (dom_ms * 1e-3) / 1e9
    # the counters were taken on the ordinary grids, not on the CU-budget kernels
    traffic = None if args.cu_budget else read_traffic(dom_kernel, w.name)
    overlap = overlap_gemm(args, step, capture) if args.overlap_gemm else None

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if w.fp8 else "bf16",
        "data": "synthetic (seeded numpy draws with the workload's shapes and routing)",
        "config": {"workload": f"{w.name}: {w.N} tokens x hidden {w.H}, {w.E} experts, "
                               f"top-{w.K}, {w.R} virtual ranks, expert_alignment {w.A}, "
                               f"{'e4m3' if w.fp8 else 'bf16'} dispatch, {w.routing} routing",
                   "num_tokens": w.N, "hidden": w.H, "num_experts": w.E, "num_topk": w.K,
                   "num_ranks": w.R, "expert_alignment": 1 if args.ll else w.A,
                   "seed": args.seed, "path": (f"low-latency (M={args.ll})" if args.ll
                                               else "layout + dispatch + combine"),
                   "cu_budget": args.cu_budget,
                   "parallelism": "1 GPU, virtual EP ranks"},
        "tokens_per_s": round(w.N / step_s, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "bytes_per_step": total_b,
        "gpu_ms_per_step": round(gpu_step_ms, 4),
        "launch": "eager" if args.eager else "one captured HIP graph of the K steps",
        "kernel_ms": {"layout": round(lay_ms, 4), "dispatch": round(dis_ms, 4),
                      "combine": round(com_ms, 4)},
        "kernel_gbs": {"dispatch": round(disp_b / (dis_ms * 1e-3) / 1e9, 1),
                       "combine": round(comb_b / (com_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "kernel": dom_kernel, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic},
    }
    if cold:
        result["cold"] = cold
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                        "compute_units": props.multi_processor_count,
                        "memory_gib": round(props.total_memory / 2 ** 30, 1),
                        "hip": torch.version.hip, "torch": torch.__version__}
    lds = lds_info()
    if lds:
        result["device"].update(lds)
        if args.cu_budget:
            # each CU-budget workgroup reserves lds_per_workgroup bytes; more
            # than half of a CU's LDS means at most one of them per CU
            result["config"]["cu_budget_lds_per_workgroup"] = lds["lds_per_workgroup"]
            result["config"]["cu_budget_one_workgroup_per_cu"] = \
                2 * lds["lds_per_workgroup"] > lds["lds_per_cu"]
    if overlap:
        result["overlap"] = overlap
    if not args.no_ceiling:
        print("[bench] HBM ceilings", file=sys.stderr, flush=True)
        recv_x_t = ll_out[1][0] if args.ll else recv[0]
        c = ceilings(per_launch_ms, w, lay.slot_of, x, recv_x_t, eo)
        result["ceiling"] = c
        best_copy = max(c["copy_gbs"], c["copy1_gbs"])
        result["frac_of_copy_ceiling"] = round(gbs / best_copy, 4)
        frac = {}
        if "scatter_gbs" in c:
            # the best of the scatter forms, all timed warm like the kernel
            best = max(c["scatter_gbs"], c.get("scatter_items_gbs", 0.0),
                       c.get("scatter_pieces_gbs", 0.0))
            frac["dispatch"] = round(result["kernel_gbs"]["dispatch"] / best, 4)
        if "gather_gbs" in c:
            frac["combine"] = round(result["kernel_gbs"]["combine"] / c["gather_gbs"], 4)
        result["frac_of_pattern_ceiling"] = frac
    if args.cpu_seconds > 0:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inp, eo_bits, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
