#!/usr/bin/env python3
"""Benchmark of the fused row-wise normalisation library on one MI355X.

Default run: one JSON line on stdout for the headline workload, residual add-RMSNorm in bf16
storage at [16384, 8192] (x and r Student-t(3) with 1% of rows scaled by 1e3, w ~ N(1, 0.1),
eps 1e-6), inputs resident in HBM. A step is one nrm_add_rms_norm call: load x and r, add,
round and store h, sum of squares, row scalar, normalise, scale by w, round and store out.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--suite] [--no-cpu-baseline]

--suite        also prints one JSON line per workload to stderr, rotating buffer sets when a
               call's working set would fit in the 256 MB Infinity Cache. The synthetic
               configurations (1-5d) carry every measurement field: GPU time, GB/s, % of
               peak, rows/s, copy ceilings of the same bytes, HBM fetch / write MB (stored
               counter summary), and the fp64 oracle over the whole workload in the same run
               (its seconds, cores, GB/s, and the parity of this run's output).
--counters     eager calls of every configuration and of one workload per other operation,
               for rocprofv3 (kernel trace, FETCH_SIZE, WRITE_SIZE runs).
--summarize-configs TRACE_DB FETCH_DB WRITE_DB
               write profiles/suite_configs.md and profiles/traffic_suite_configs.json from
               those three runs of --counters.
--sweep        bandwidth of every operation across row widths (about 256 MB per call), one
               JSON line per case to stderr; no headline line.
--profile      only warm-up and timed calls of the headline kernel plus the copy kernel
               (for rocprofv3 runs); no CPU baseline.
--summarize-trace TRACE_DB
               write profiles/add_rms_norm_bf16_16384x8192.md from the kernel trace of a
               --profile run and the counter summary.
--summarize-counters PMC_DB
               write profiles/valu_issue_suite_kernels.md (VALU issue share per kernel) from
               a `rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE`
               run of `bench.py --only fwd,vjp,sm`.
--summarize-pmc FETCH_FILE WRITE_FILE
               turn two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` outputs (rocpd .db or
               counter_collection.csv) of a
               --profile run into profiles/traffic_add_rms_norm_bf16_16384x8192.json, scaled
               by what the same counters read for the 16-byte copy kernel of known size.

Fields beyond the contract: roofline (algorithmic bytes per launch over the average launch
time measured with HIP events on the launch stream, against 8 TB/s), copy2_ceiling_GBps (two
arrays copied into two, the headline's byte pattern without arithmetic, in that pattern's
fastest shape), copy2_row_ceiling_GBps (the same copy in the row kernel's work unit: each block
loads a row's 16 KB of each array and stores nothing until all of it has arrived),
copy_ceiling_GBps (a plain 16-byte copy of the same byte count), and cpu_baseline (the fp64 oracle on a bounded
sample of the same workload, in a process pool over the host's cores).
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + rows/s, add-RMSNorm bf16 16384x8192"
PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
ROWS, HIDDEN = 16384, 8192
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_add_rms_norm_bf16_16384x8192.json")
HEADLINE_KERNEL = "row_block<true, 1, 2, 1, true>"  # bf16, add-RMSNorm, 2 chunks/thread, w bf16, exact
COPY_KERNEL = "copy16_kernel"
COPY2_KERNEL = "copy16x2_kernel"
COPY2_ROW_KERNEL = "copy16x2_row_kernel"


# Files the headline kernel and the copy kernel that scales the counters are built from.
HEADLINE_SOURCES = ("transformer_row_wise_amd/csrc/common.hpp",
                    "transformer_row_wise_amd/csrc/row_kernels.hpp",
                    "transformer_row_wise_amd/csrc/row_launch.hpp",
                    "transformer_row_wise_amd/csrc/launch.hpp",
                    "transformer_row_wise_amd/csrc/add_rms.hip",
                    "transformer_row_wise_amd/csrc/copy.hip")


def kernel_source_hash():
    """Hash of the headline kernel's sources and compiler flags: a stored counter reading is
    used only for this exact code."""
    from transformer_row_wise_amd import build as nrm_build
    h = hashlib.sha256()
    flags = [f.replace(nrm_build.ROOT, ".") for f in nrm_build.FLAGS]
    h.update(" ".join(flags).encode() + b"\0")
    for rel in HEADLINE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def add_rms_bytes(rows, hidden, es, w_es):
    """Algorithmic bytes of one add-RMSNorm call: read x and r, write out and h, read w."""
    return 4 * rows * hidden * es + hidden * w_es


# --------------------------------------------------------------------------- GPU timing

def time_calls(fn, steps, warmup):
    """Time `steps` back-to-back calls after `warmup` untimed ones.

    Returns (gpu_ms_per_call, wall_ms_per_call). The GPU figure comes from two HIP events on
    torch's current stream (the stream the library launches on) around the whole timed
    region, so it is the average launch duration with nothing recorded between launches.
    The wall figure is the host clock across the same region, bracketed by synchronisation.
    """
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return start.elapsed_time(end) / steps, wall_ms


def time_graph(fn, calls, replays=10):
    """Per-call GPU time (ms) of `calls` back-to-back calls captured in one HIP graph and
    replayed: no host time between kernels, which matters for calls of a few microseconds."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    for _ in range(3):  # untimed replays: let the clocks settle
        g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        per.append(s.elapsed_time(e) / calls)
    del g
    return per


def copy_ceiling(nbytes, steps):
    """GB/s of the library's 16-byte copy moving nbytes/2 bytes in and nbytes/2 out."""
    import torch
    import transformer_row_wise_amd as nrm

    half = (nbytes // 2) // 16 * 16
    src = torch.empty(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    gpu_ms, _ = time_calls(lambda i: nrm.bench_copy(src, dst), steps, steps)
    del src, dst
    return 2 * half / (gpu_ms * 1e-3) / 1e9


def copy2_ceiling(nbytes, steps):
    """GB/s of the library's two-into-two 16-byte copy moving nbytes in all: two arrays of
    nbytes/4 in, two out (the headline's byte pattern without arithmetic)."""
    import torch
    import transformer_row_wise_amd as nrm

    q = (nbytes // 4) // 16 * 16
    s1 = torch.empty(q, dtype=torch.uint8, device="cuda")
    s2, d1, d2 = torch.empty_like(s1), torch.empty_like(s1), torch.empty_like(s1)
    s1.fill_(1)
    s2.fill_(2)
    gpu_ms, _ = time_calls(lambda i: nrm.bench_copy2(s1, s2, d1, d2), steps, steps)
    del s1, s2, d1, d2
    return 4 * q / (gpu_ms * 1e-3) / 1e9


def copy2_row_ceiling(rows, unit_bytes, steps):
    """GB/s of the two-into-two copy in the row kernel's work unit (nrm_bench_copy2_row): two
    arrays of rows units of unit_bytes in, two out, every block waiting for its whole unit
    before it stores (the headline's access pattern in row_block's shape, no arithmetic)."""
    import torch
    import transformer_row_wise_amd as nrm

    q = rows * unit_bytes
    s1 = torch.empty(q, dtype=torch.uint8, device="cuda")
    s2, d1, d2 = torch.empty_like(s1), torch.empty_like(s1), torch.empty_like(s1)
    s1.fill_(1)
    s2.fill_(2)
    gpu_ms, _ = time_calls(lambda i: nrm.bench_copy2_row(s1, s2, d1, d2, unit_bytes), steps, steps)
    del s1, s2, d1, d2
    return 4 * q / (gpu_ms * 1e-3) / 1e9


def stored_traffic(nbytes):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------- CPU baseline

def _oracle_chunk(args):
    """One worker: the fp64 oracle on a slice of rows (bf16 bit patterns in, time out)."""
    import numpy as np

    import oracle

    xb, rb, wb, eps = args

    def decode(b):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    t = time.perf_counter()
    oracle.add_rms_norm(decode(xb), decode(rb), decode(wb), eps, "bf16")
    return time.perf_counter() - t


def cpu_baseline(inp, min_cpu_s=10.0, max_passes=3):
    """The oracle, as it is, over all rows of the workload, spread over a process pool with
    one process per available core (at most 16); whole passes are repeated until at least
    `min_cpu_s` seconds of CPU work are done (at most `max_passes`)."""
    import multiprocessing as mp

    import numpy as np
    import torch

    cores = min(len(os.sched_getaffinity(0)), 16)
    rows = inp.x.shape[0]
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    xb, rb, wb = bits(inp.x), bits(inp.r), bits(inp.w)
    step = 128
    jobs = [(xb[i:i + step], rb[i:i + step], wb, inp.eps) for i in range(0, rows, step)]
    ctx = mp.get_context("spawn")
    busy, passes = 0.0, 0
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_chunk, jobs[:cores])  # start-up and imports, untimed
        t0 = time.perf_counter()
        while passes < max_passes and (passes == 0 or busy < min_cpu_s):
            busy += sum(pool.map(_oracle_chunk, jobs))
            passes += 1
        wall = time.perf_counter() - t0
    nbytes = passes * add_rms_bytes(rows, inp.x.shape[1], 2, 2)
    return {
        "value": round(nbytes / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"all {rows} rows of the same add-RMSNorm bf16 [{rows}, {inp.x.shape[1]}] "
                  f"inputs, {passes} pass(es); fp64 oracle in a pool of {cores} processes "
                  f"(chunks of {step} rows); {busy:.1f} s of CPU work, {wall:.2f} s wall",
        "rows_per_s": round(passes * rows / wall, 1),
        "wall_s": round(wall, 3),
    }


# --------------------------------------------------------------------------- headline

def headline(args):
    import torch

    import transformer_row_wise_amd as nrm
    import workloads

    nrm.load()
    print(f"# generating add-RMSNorm bf16 [{ROWS}, {HIDDEN}] inputs", file=sys.stderr, flush=True)
    inp = workloads.cfg_add_rms_scale(ROWS, HIDDEN, "bf16")
    x, r, w = inp.x.cuda(), inp.r.cuda(), inp.w.cuda()
    out, h = torch.empty_like(x), torch.empty_like(x)
    nbytes = add_rms_bytes(ROWS, HIDDEN, 2, 2)

    def step(_):
        nrm.add_rms_norm(x, r, w, inp.eps, out=out, h=h)

    # The three copy ceilings run first: about 1 s of streaming at the same byte count, which
    # brings the GPU to the clocks it holds under sustained load (it needs about a second), so
    # that the headline's few timed steps are not taken on the way up. Under a profiler they
    # stay short.
    copy_steps = max(100, args.steps // 2) if args.profile else 2000
    print(f"# copy ceilings, {copy_steps} steps each", file=sys.stderr, flush=True)
    ceiling = copy_ceiling(nbytes, copy_steps)
    ceiling2 = copy2_ceiling(nbytes, copy_steps)
    ceiling_row = copy2_row_ceiling(ROWS, HIDDEN * 2, copy_steps)
    print(f"# timing {args.steps} steps after {args.warmup} warm-up", file=sys.stderr, flush=True)
    gpu_ms, wall_ms = time_calls(step, args.steps, args.warmup)
    achieved = nbytes / (gpu_ms * 1e-3) / 1e9
    value = nbytes / (wall_ms * 1e-3) / 1e9
    if args.profile:
        print(json.dumps({"profile_run": True, "avg_launch_us": gpu_ms * 1e3,
                          "achieved_GBps": achieved, "copy_GBps": ceiling,
                          "copy2_GBps": ceiling2, "copy2_row_GBps": ceiling_row}), flush=True)
        return
    traffic = stored_traffic(nbytes)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "add-RMSNorm bf16 [16384, 8192]: x, r Student-t(3) with 1% of rows "
                        "x1e3, w ~ N(1, 0.1) bf16, eps 1e-6",
            "rows": ROWS, "hidden": HIDDEN, "io_dtype": "bf16", "parallelism": "none",
        },
        "pct_peak": round(100 * value / PEAK_GBPS, 2),
        "rows_per_s": round(ROWS / (wall_ms * 1e-3), 1),
        "bytes_per_step": nbytes,
        "kernel_us_mean": round(gpu_ms * 1e3, 2),
        "copy_ceiling_GBps": round(ceiling, 1),
        "copy2_ceiling_GBps": round(ceiling2, 1),
        "copy2_row_ceiling_GBps": round(ceiling_row, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline: the oracle over the workload's rows", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(res), flush=True)


# --------------------------------------------------------------------------- suite

def suite(args):
    """One line per synthetic workload, to stderr. Working sets under 512 MB rotate through
    enough buffer sets to exceed the 256 MB Infinity Cache."""
    import torch

    import transformer_row_wise_amd as nrm
    import workloads

    nrm.load()

    def n_sets(bytes_per_call):
        return max(1, min(16, -(-512 * 2**20 // bytes_per_call)))

    def calls(bytes_per_call):
        """Calls per graph: about 2 GB of traffic, between 16 and 1000 calls."""
        return max(16, min(1000, (2048 * 2**20) // bytes_per_call))

    def emit(cfg, op, shape, nbytes, rows, per):
        avg = statistics.median(per)
        gbps = nbytes / (avg * 1e-3) / 1e9
        print(json.dumps({"cfg": cfg, "op": op, "shape": shape, "bytes": nbytes,
                          "gpu_us_median": round(avg * 1e3, 3),
                          "gpu_us_min": round(min(per) * 1e3, 3),
                          "timing": "HIP graph of back-to-back calls, median of 10 replays",
                          "gpu_GBps": round(gbps, 1), "pct_peak": round(100 * gbps / PEAK_GBPS, 2),
                          "rows_per_s": round(rows / (avg * 1e-3), 1),
                          "fetch_MB": (traffic_entry(cfg) or {}).get("fetch_MB"),
                          "write_MB": (traffic_entry(cfg) or {}).get("write_MB")}),
              file=sys.stderr, flush=True)

    def run_vjp(cfg, inp, ln):
        rows, hidden = inp.x.shape
        es, pes = inp.x.element_size(), inp.w.element_size()
        # read x and g, write dx; read w, write dw (and db)
        nbytes = 3 * rows * hidden * es + hidden * pes * (3 if ln else 2)
        x, g, w = inp.x.cuda(), inp.g.cuda(), inp.w.cuda()
        dx, dw, db = torch.empty_like(x), torch.empty_like(w), torch.empty_like(w)
        ws = torch.empty(nrm.vjp_workspace_bytes(rows, hidden, ln), dtype=torch.uint8,
                         device="cuda")
        if ln:
            fn = lambda i: nrm.layer_norm_vjp(x, w, g, inp.eps, dx=dx, dw=dw, db=db, workspace=ws)
        else:
            fn = lambda i: nrm.rms_norm_vjp(x, w, g, inp.eps, dx=dx, dw=dw, workspace=ws)
        per = time_graph(fn, calls(nbytes))
        emit(cfg, "layer_norm_vjp" if ln else "rms_norm_vjp", [rows, hidden, str(inp.x.dtype)],
             nbytes, rows, per)

    groups = set(args.only.split(",")) if args.only else {"fwd", "vjp", "rope", "sm"}
    if "sm" in groups:
        x = workloads.scores((16384, 8192), "bf16").cuda()
        out = torch.empty_like(x)
        nbytes = 2 * x.numel() * 2
        per = time_graph(lambda i: nrm.softmax(x, out=out), calls(nbytes))
        emit("9a", "softmax", list(x.shape), nbytes, x.shape[0], per)
        del x, out
        B, H, L = 8, 32, 512
        xs = workloads.scores((B * H, L, L), "bf16", seed=1)
        k = n_sets(2 * xs.numel() * 2)
        xl = [xs.cuda() for _ in range(k)]
        ol = [torch.empty_like(xl[0]) for _ in range(k)]
        # Masked scores need not be read: the bytes are the kept scores (row r keeps r + 1
        # of L columns with rows = L) plus the whole output.
        nbytes = B * H * (L * (L + 1) // 2) * 2 + xs.numel() * 2
        per = time_graph(lambda i: nrm.causal_softmax(xl[i % k], L, out=ol[i % k]), calls(nbytes))
        emit("9b", "causal_softmax", [B * H, L, L], nbytes, B * H * L, per)
        del xl, ol
        inp = workloads.cfg_ce_bf16()
        rows, V = workloads.CE_SHAPE
        lg, tg, g = inp.logits.cuda(), inp.targets.cuda(), inp.g.cuda()
        lse = torch.empty(rows, 1, dtype=torch.bfloat16, device="cuda")
        loss = torch.empty(rows, dtype=torch.float32, device="cuda")
        dl = torch.empty_like(lg)
        nb_in = rows * V * 2
        per = time_graph(lambda i: nrm.logsumexp(lg, out=lse), calls(nb_in))
        emit("9c", "logsumexp", [rows, V], nb_in + rows * 2, rows, per)
        per = time_graph(lambda i: nrm.cross_entropy(lg, tg, loss=loss), calls(nb_in))
        emit("9d", "cross_entropy", [rows, V], nb_in + rows * 12, rows, per)
        per = time_graph(lambda i: nrm.cross_entropy_vjp(lg, tg, g, dlogits=dl), calls(2 * nb_in))
        emit("9e", "cross_entropy_vjp", [rows, V], 2 * nb_in + rows * 12, rows, per)
        del lg, dl
    if "rope" in groups:
        inp = workloads.cfg_rope_qk_bf16()
        T, Hq, Hk, D = workloads.ROPE_QK_SHAPE
        freqs, ms = nrm.rope_freqs_llama3(D, workloads.ROPE_QK_BASE)
        nbytes = 2 * T * (Hq + Hk) * D * 2 + T * 8 + D // 2 * 4
        k = n_sets(nbytes)
        qs = [inp.q.cuda() for _ in range(k)]
        ks = [inp.k.cuda() for _ in range(k)]
        pos, fr = inp.positions.cuda(), freqs.cuda()
        outs = [(torch.empty_like(qs[0]), torch.empty_like(ks[0])) for _ in range(k)]
        per = time_graph(lambda i: nrm.rope_positions(pos, qs[i % k], ks[i % k],
                                                      base=workloads.ROPE_QK_BASE, freqs=fr,
                                                      mscale=ms, q_out=outs[i % k][0],
                                                      k_out=outs[i % k][1]), calls(nbytes))
        emit("8a", "rope_positions_llama3", [T, Hq, Hk, D], nbytes, T * (Hq + Hk), per)
        del qs, ks, outs
        rp = workloads.cfg_norm_rope_bf16()
        B, H, L, D = rp.x.shape
        nbytes = 2 * B * H * L * D * 2
        k = n_sets(nbytes)
        xs = [rp.x.cuda() for _ in range(k)]
        dsts = [torch.empty_like(xs[0]) for _ in range(k)]
        per = time_graph(lambda i: nrm.rope(xs[i % k], out=dsts[i % k]), calls(nbytes))
        emit("8b", "rope", [B, H, L, D], nbytes, B * H * L, per)
        del xs, dsts
    if "vjp" in groups:
        for ln, tag in ((False, "6"), (True, "7")):
            f32 = workloads.cfg_ln_vjp(dtype="f32") if ln else workloads.cfg_rms_vjp(dtype="f32")
            bf = workloads.RowInputs(x=f32.x.to(torch.bfloat16), r=None,
                                     w=f32.w.to(torch.bfloat16), b=None, eps=f32.eps,
                                     g=f32.g.to(torch.bfloat16))
            run_vjp(tag + "a", bf, ln)
            run_vjp(tag + "b", f32, ln)
            del f32, bf
    if "fwd" not in groups:
        return
    run_configs(args, nrm, torch, workloads, n_sets, calls, traffic_entry)


# --------------------------------------------------------------------------- synthetic configs

# The synthetic configurations of the benchmark (one line each), and one workload per
# operation of the backward, Rope and softmax groups, in the order the counter runs take them.
CONFIG_IDS = ["1", "2", "3a", "3b", "4a", "4b", "4c", "4d", "5a", "5b", "5c", "5d"]
NEXT_IDS = ["6a", "7a", "8a", "8b", "9a", "9b", "9c", "9d", "9e"]
# Kernel dispatches of one call, where more than one (the backward adds its column sums).
DISPATCHES_PER_CALL = {"6a": 2, "7a": 2}
# The library launches a row call (RMSNorm, add-RMSNorm, LayerNorm on rows of whole 16-byte
# chunks) that streams more than this many bytes over all its arrays as consecutive pieces of
# at most that many (an even number of rows each); the forward configurations' row calls:
# (rows, hidden), element bytes, arrays streamed (x, r, out, h for add-RMSNorm; x, out).
LAUNCH_BYTES = 1 << 30
FWD_ROW_CALLS = {"1": ((64, 512), 4, 4), "2": ((4096, 4096), 2, 4), "3a": ((16384, 8192), 2, 2),
                 "3b": ((16384, 8192), 2, 2), "5a": ((16384, 8192), 2, 4),
                 "5b": ((16384, 8192), 4, 4), "5c": ((65536, 5120), 2, 4),
                 "5d": ((65536, 5120), 4, 4)}


def row_call_launches(rows, hidden, elem_bytes, arrays):
    """Kernel launches of one row call of that shape under the library's split rule."""
    row_bytes = hidden * elem_bytes * arrays
    if rows <= LAUNCH_BYTES // row_bytes:
        return 1
    per = max(2, (LAUNCH_BYTES // row_bytes) & ~1)
    return -(-rows // per)


def dispatches_per_call(cid):
    if cid in FWD_ROW_CALLS:
        (rows, hidden), es, arrays = FWD_ROW_CALLS[cid]
        return row_call_launches(rows, hidden, es, arrays)
    return DISPATCHES_PER_CALL.get(cid, 1)
SUITE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_suite_configs.json")
SUITE_MD = os.path.join(ROOT, "profiles", "suite_configs.md")
CAL_BYTES = 512 * 2**20  # the calibration copy, bytes each way
ORACLE_CHUNK_ROWS = 256


def library_source_hash():
    """Hash of every library source and the compiler flags: a stored per-config counter
    reading is used only for this exact code."""
    import glob

    from transformer_row_wise_amd import build as nrm_build
    h = hashlib.sha256()
    flags = [f.replace(nrm_build.ROOT, ".") for f in nrm_build.FLAGS]
    h.update(" ".join(flags).encode() + b"\0")
    for path in sorted(glob.glob(os.path.join(ROOT, "transformer_row_wise_amd", "csrc", "*"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _np_bits(t):
    """A CPU numpy copy of a tensor's bits: bf16 -> uint16, fp32 -> float32."""
    import numpy as np
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def build_case(cid, nrm, torch, workloads, n_sets):
    """One workload as a dict: op, dtype, shape, algorithmic bytes, rows, the kernel
    dispatches one call issues, `call(i)` (buffer set i % k), and `jobs()` (runs set 0 once
    and returns the oracle's chunks of rows, each with the GPU's output for it; configs only)."""
    import numpy as np

    dev = "cuda"
    if cid in ("1", "2", "5a", "5b", "5c", "5d"):
        if cid == "1":
            inp = workloads.cfg_add_rms_small_f32()
        elif cid == "2":
            inp = workloads.cfg_add_rms_4k_bf16()
        else:
            shape = (16384, 8192) if cid in ("5a", "5b") else (65536, 5120)
            inp = workloads.cfg_add_rms_scale(*shape, dtype="f32")
            if cid in ("5a", "5c"):
                inp = workloads.RowInputs(x=inp.x.to(torch.bfloat16), r=inp.r.to(torch.bfloat16),
                                          w=inp.w.to(torch.bfloat16), b=None, eps=inp.eps)
        rows, hidden = inp.x.shape
        nbytes = add_rms_bytes(rows, hidden, inp.x.element_size(), inp.w.element_size())
        k = n_sets(nbytes)
        sets = [(inp.x.to(dev), inp.r.to(dev)) for _ in range(k)]
        w = inp.w.to(dev)
        outs = [(torch.empty_like(sets[0][0]), torch.empty_like(sets[0][0])) for _ in range(k)]

        def call(i):
            nrm.add_rms_norm(*sets[i % k], w, inp.eps, out=outs[i % k][0], h=outs[i % k][1])

        def jobs():
            call(0)
            torch.cuda.synchronize()
            xb, rb, wb, ob, hb = (_np_bits(t) for t in (inp.x, inp.r, inp.w, outs[0][0], outs[0][1]))
            c = ORACLE_CHUNK_ROWS
            return [("add", xb[i:i + c], rb[i:i + c], wb, inp.eps, ob[i:i + c], hb[i:i + c])
                    for i in range(0, rows, c)]

        return dict(cfg=cid, op="add_rms_norm", dtype=str(inp.x.dtype).replace("torch.", ""),
                    shape=[rows, hidden], bytes=nbytes, rows=rows, dispatches=1, call=call,
                    jobs=jobs, copy2=True)
    if cid in ("3a", "3b"):
        affine = cid == "3a"
        inp = workloads.cfg_layer_norm_bf16(affine=affine)
        rows, hidden = inp.x.shape
        nbytes = 2 * rows * hidden * 2 + (2 * hidden * 2 if affine else 0)
        x = inp.x.to(dev)
        w = inp.w.to(dev) if affine else None
        b = inp.b.to(dev) if affine else None
        out = torch.empty_like(x)

        def call(i):
            nrm.layer_norm(x, w, b, inp.eps, out=out)

        def jobs():
            call(0)
            torch.cuda.synchronize()
            xb, ob = _np_bits(inp.x), _np_bits(out)
            wb = _np_bits(inp.w) if affine else None
            bb = _np_bits(inp.b) if affine else None
            c = ORACLE_CHUNK_ROWS
            return [("ln", xb[i:i + c], wb, bb, inp.eps, ob[i:i + c]) for i in range(0, rows, c)]

        return dict(cfg=cid, op="layer_norm" + ("" if affine else "_no_affine"), dtype="bfloat16",
                    shape=[rows, hidden], bytes=nbytes, rows=rows, dispatches=1, call=call,
                    jobs=jobs, copy2=False)
    if cid in ("4a", "4b", "4c", "4d"):
        cache, trad = cid in ("4c", "4d"), cid in ("4b", "4d")
        rp = workloads.cfg_norm_rope_bf16(offset=workloads.NORM_ROPE_CACHE_OFFSET if cache else 0)
        B, H, L, D = rp.x.shape
        nbytes = 2 * B * H * L * D * 2 + D * 2
        k = n_sets(nbytes)
        xs = [rp.x.to(dev) for _ in range(k)]
        w = rp.w.to(dev)
        if cache:
            dsts = [torch.zeros(B, H, workloads.NORM_ROPE_CACHE_LEN, D, dtype=torch.bfloat16,
                                device=dev) for _ in range(k)]
        else:
            dsts = [torch.empty_like(xs[0]) for _ in range(k)]

        def call(i):
            nrm.norm_rope(xs[i % k], w, eps=rp.eps, dims=rp.dims, traditional=trad,
                          base=rp.base, scale=rp.scale, offset=rp.offset,
                          cache=dsts[i % k] if cache else None, out=None if cache else dsts[i % k])

        def jobs():
            call(0)
            torch.cuda.synchronize()
            xb, wb, ob = _np_bits(rp.x), _np_bits(rp.w), _np_bits(dsts[0])
            p = (rp.eps, rp.dims, trad, rp.base, rp.scale, rp.offset, cache)
            return [("rope", xb[i:i + 1], wb, p, ob[i:i + 1]) for i in range(B)]

        return dict(cfg=cid, op="norm_rope" + ("_cache" if cache else "") +
                    ("_interleaved" if trad else "_half"), dtype="bfloat16", shape=[B, H, L, D],
                    bytes=nbytes, rows=B * H * L, dispatches=1, call=call, jobs=jobs, copy2=False)
    # One workload per operation of the other groups (counter evidence only).
    if cid in ("6a", "7a"):
        ln = cid == "7a"
        f32 = workloads.cfg_ln_vjp(dtype="f32") if ln else workloads.cfg_rms_vjp(dtype="f32")
        x, g = f32.x.to(torch.bfloat16).to(dev), f32.g.to(torch.bfloat16).to(dev)
        w = f32.w.to(torch.bfloat16).to(dev)
        rows, hidden = x.shape
        dx, dw, db = torch.empty_like(x), torch.empty_like(w), torch.empty_like(w)
        ws = torch.empty(nrm.vjp_workspace_bytes(rows, hidden, ln), dtype=torch.uint8, device=dev)
        nbytes = 3 * rows * hidden * 2 + hidden * 2 * (3 if ln else 2)

        def call(i):
            if ln:
                nrm.layer_norm_vjp(x, w, g, f32.eps, dx=dx, dw=dw, db=db, workspace=ws)
            else:
                nrm.rms_norm_vjp(x, w, g, f32.eps, dx=dx, dw=dw, workspace=ws)

        return dict(cfg=cid, op="layer_norm_vjp" if ln else "rms_norm_vjp", dtype="bfloat16",
                    shape=[rows, hidden], bytes=nbytes, rows=rows, dispatches=2, call=call)
    if cid == "8a":
        inp = workloads.cfg_rope_qk_bf16()
        T, Hq, Hk, D = workloads.ROPE_QK_SHAPE
        freqs, ms = nrm.rope_freqs_llama3(D, workloads.ROPE_QK_BASE)
        q, kk, pos, fr = inp.q.to(dev), inp.k.to(dev), inp.positions.to(dev), freqs.to(dev)
        qo, ko = torch.empty_like(q), torch.empty_like(kk)
        nbytes = 2 * T * (Hq + Hk) * D * 2 + T * 8 + D // 2 * 4

        def call(i):
            nrm.rope_positions(pos, q, kk, base=workloads.ROPE_QK_BASE, freqs=fr, mscale=ms,
                               q_out=qo, k_out=ko)

        return dict(cfg=cid, op="rope_positions_llama3", dtype="bfloat16", shape=[T, Hq, Hk, D],
                    bytes=nbytes, rows=T * (Hq + Hk), dispatches=1, call=call)
    if cid == "8b":
        rp = workloads.cfg_norm_rope_bf16()
        x = rp.x.to(dev)
        out = torch.empty_like(x)
        B, H, L, D = x.shape

        def call(i):
            nrm.rope(x, out=out)

        return dict(cfg=cid, op="rope", dtype="bfloat16", shape=[B, H, L, D],
                    bytes=2 * x.numel() * 2, rows=B * H * L, dispatches=1, call=call)
    if cid in ("9a", "9b"):
        causal = cid == "9b"
        shape = (8 * 32, 512, 512) if causal else (16384, 8192)
        x = workloads.scores(shape, "bf16", seed=1 if causal else 0).to(dev)
        out = torch.empty_like(x)
        if causal:
            N, R, L = shape
            nbytes = N * (L * (L + 1) // 2) * 2 + x.numel() * 2
        else:
            nbytes = 2 * x.numel() * 2

        def call(i):
            if causal:
                nrm.causal_softmax(x, shape[1], out=out)
            else:
                nrm.softmax(x, out=out)

        return dict(cfg=cid, op="causal_softmax" if causal else "softmax", dtype="bfloat16",
                    shape=list(shape), bytes=nbytes, rows=x.numel() // shape[-1], dispatches=1,
                    call=call)
    if cid in ("9c", "9d", "9e"):
        inp = workloads.cfg_ce_bf16()
        rows, V = workloads.CE_SHAPE
        lg, tg, g = inp.logits.to(dev), inp.targets.to(dev), inp.g.to(dev)
        nb_in = rows * V * 2
        if cid == "9c":
            lse = torch.empty(rows, 1, dtype=torch.bfloat16, device=dev)
            call, op, nbytes = (lambda i: nrm.logsumexp(lg, out=lse)), "logsumexp", nb_in + rows * 2
        elif cid == "9d":
            loss = torch.empty(rows, dtype=torch.float32, device=dev)
            call = lambda i: nrm.cross_entropy(lg, tg, loss=loss)
            op, nbytes = "cross_entropy", nb_in + rows * 12
        else:
            dl = torch.empty_like(lg)
            call = lambda i: nrm.cross_entropy_vjp(lg, tg, g, dlogits=dl)
            op, nbytes = "cross_entropy_vjp", 2 * nb_in + rows * 12
        return dict(cfg=cid, op=op, dtype="bfloat16", shape=[rows, V], bytes=nbytes, rows=rows,
                    dispatches=1, call=call)
    raise ValueError(cid)


def _bf16_ordered(bits):
    import numpy as np

    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def _f32_ordered(v):
    import numpy as np

    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.int64)
    return np.where(b & 0x80000000, -(b & 0x7FFFFFFF), b & 0x7FFFFFFF)


def _compare(got, want):
    """(largest distance in units in the last place, elements over the bar) of one output
    chunk: bf16 within 1 ulp, fp32 within 1e-5 relative + 1e-6 absolute; NaN only with NaN."""
    import numpy as np

    if got.dtype == np.uint16:
        wb = (np.asarray(want, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        gn = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        wn = ((wb & 0x7F80) == 0x7F80) & ((wb & 0x7F) != 0)
        d = np.abs(_bf16_ordered(got) - _bf16_ordered(wb))
        d = np.where(gn & wn, 0, np.where(gn ^ wn, 1 << 40, d))
        return int(d.max()) if d.size else 0, int(np.count_nonzero(d > 1))
    g = got.astype(np.float64)
    w = np.asarray(want, np.float64)
    gn, wn = np.isnan(g), np.isnan(w)
    d = np.abs(_f32_ordered(got) - _f32_ordered(w.astype(np.float32)))
    d = np.where(gn & wn, 0, np.where(gn ^ wn, 1 << 40, d))
    with np.errstate(invalid="ignore"):
        bad = ~(np.abs(g - w) <= 1e-6 + 1e-5 * np.abs(w))
    bad &= ~(np.isinf(g) & np.isinf(w) & (g == w))
    bad = np.where(gn & wn, False, bad) | (gn ^ wn)
    return int(d.max()) if d.size else 0, int(np.count_nonzero(bad))


def _config_oracle_job(job):
    """One worker: the fp64 oracle on one chunk, timed, then compared with the GPU's output.
    Returns (oracle seconds, max ulp, over the bar, h bits that differ)."""
    import numpy as np

    import oracle

    def dec(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.astype(np.float64)

    kind = job[0]
    t0 = time.perf_counter()
    if kind == "add":
        _, x, r, w, eps, out, h = job
        dt = "bf16" if x.dtype == np.uint16 else "f32"
        want_out, want_h = oracle.add_rms_norm(dec(x), dec(r), dec(w), eps, dt)
        t = time.perf_counter() - t0
        mu, over = _compare(out, want_out)
        if dt == "bf16":
            hb = (np.asarray(want_h, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            hbad = int(np.count_nonzero(hb != h))
        else:
            hbad = int(np.count_nonzero(np.asarray(want_h, np.float64).astype(np.float32).view(np.uint32)
                                        != h.view(np.uint32)))
        return t, mu, over, hbad
    if kind == "ln":
        _, x, w, b, eps, out = job
        want = oracle.layer_norm(dec(x), dec(w), dec(b), eps, "bf16" if x.dtype == np.uint16 else "f32")
        t = time.perf_counter() - t0
        return (t, *_compare(out, want), 0)
    if kind == "rope":
        _, x, w, (eps, dims, trad, base, scale, offset, cache), out = job
        cache_in = np.zeros(out.shape) if cache else None
        want = oracle.norm_rope(dec(x), dec(w), normalize=True, eps=eps, dims=dims,
                                traditional=trad, base=base, scale=scale, offset=offset,
                                forward=True, dtype="bf16", cache=cache_in)
        t = time.perf_counter() - t0
        return (t, *_compare(out, want), 0)
    raise ValueError(kind)


def oracle_parity(jobs):
    """The oracle over every chunk in a spawn process pool over the host's cores (at most
    16), each chunk compared with the GPU's output. Returns the suite fields."""
    import multiprocessing as mp

    cores = min(len(os.sched_getaffinity(0)), 16)
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_config_oracle_job, jobs[:1])  # start-up and imports, untimed
        t0 = time.perf_counter()
        res = pool.map(_config_oracle_job, jobs, chunksize=1)
        wall = time.perf_counter() - t0
    return {"parity_max_ulp": max(r[1] for r in res), "parity_over_tol": sum(r[2] for r in res),
            "h_bits_differ": sum(r[3] for r in res), "oracle_s": round(wall, 3),
            "oracle_cpu_s": round(sum(r[0] for r in res), 2), "oracle_cores": cores}


def traffic_entry(cid):
    """Stored per-config counter figures for the current library sources, else None."""
    try:
        with open(SUITE_TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("library_source_hash") != library_source_hash():
        return None
    return t.get("cases", {}).get(cid)


def run_configs(args, nrm, torch, workloads, n_sets, calls, traffic):
    """One JSON line per synthetic configuration (stderr) with the measurement fields: GPU
    time from a captured HIP graph (median of 10 replays, rotating buffer sets under 512 MB),
    GB/s, % of peak, rows/s, the 16-byte copy of the same bytes (and, for add-RMSNorm, the
    two-into-two copy), HBM fetch / write MB from the stored counter summary, and the oracle
    over the whole workload in the same run: its time, cores, GB/s, and the parity of this
    run's own output (largest ulp distance, elements over the bar, h bits that differ)."""

    def copy_gbps(nbytes, two):
        q = (nbytes // (4 if two else 2)) // 16 * 16
        k = n_sets(nbytes)
        if two:
            bufs = [[torch.ones(q, dtype=torch.uint8, device="cuda") for _ in range(4)] for _ in range(k)]
            fn = lambda i: nrm.bench_copy2(*bufs[i % k])
            moved = 4 * q
        else:
            bufs = [[torch.ones(q, dtype=torch.uint8, device="cuda") for _ in range(2)] for _ in range(k)]
            fn = lambda i: nrm.bench_copy(*bufs[i % k])
            moved = 2 * q
        avg = statistics.median(time_graph(fn, calls(nbytes)))
        del bufs
        return moved / (avg * 1e-3) / 1e9

    for cid in CONFIG_IDS:
        case = build_case(cid, nrm, torch, workloads, n_sets)
        nbytes = case["bytes"]
        per = time_graph(case["call"], calls(nbytes))
        avg = statistics.median(per)
        gbps = nbytes / (avg * 1e-3) / 1e9
        line = {"cfg": cid, "op": case["op"], "dtype": case["dtype"], "shape": case["shape"],
                "bytes": nbytes, "gpu_us_median": round(avg * 1e3, 3),
                "gpu_us_min": round(min(per) * 1e3, 3),
                "timing": "HIP graph of back-to-back calls, median of 10 replays",
                "gpu_GBps": round(gbps, 1), "pct_peak": round(100 * gbps / PEAK_GBPS, 2),
                "rows_per_s": round(case["rows"] / (avg * 1e-3), 1),
                "copy_ceiling_GBps": round(copy_gbps(nbytes, False), 1)}
        if case["copy2"]:
            line["copy2_ceiling_GBps"] = round(copy_gbps(nbytes, True), 1)
        t = traffic(cid)
        line["fetch_MB"] = t["fetch_MB"] if t else None
        line["write_MB"] = t["write_MB"] if t else None
        if not args.no_cpu_baseline:
            par = oracle_parity(case["jobs"]())
            par["oracle_GBps"] = round(nbytes / par["oracle_s"] / 1e9, 4)
            line.update(par)
        print(json.dumps(line), file=sys.stderr, flush=True)
        del case
        torch.cuda.empty_cache()


def counter_run(args):
    """For rocprofv3 (kernel trace, or one --pmc counter per run): the calibration copy, then
    every configuration and one workload per other operation, each called --counter-calls
    times back to back (one synchronisation per workload), in CONFIG_IDS + NEXT_IDS order.
    --summarize-configs attributes the dispatches by that order."""
    import torch

    import transformer_row_wise_amd as nrm
    import workloads

    nrm.load()
    n = args.counter_calls
    src = torch.ones(CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n):
        nrm.bench_copy(src, dst)
    torch.cuda.synchronize()
    del src, dst
    for cid in CONFIG_IDS + NEXT_IDS:
        print(f"# counters: {cid}", file=sys.stderr, flush=True)
        case = build_case(cid, nrm, torch, workloads, lambda nb: 1)
        for i in range(n):
            case["call"](i)
        torch.cuda.synchronize()
        del case
        torch.cuda.empty_cache()


CONFIG_CMDS = [
    "rocprofv3 --kernel-trace -d gpurun_out/cfg_trace -o trace -- python3 bench.py --counters "
    "--counter-calls 20",
    "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/cfg_fetch -o fetch -- python3 bench.py --counters",
    "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/cfg_write -o write -- python3 bench.py --counters",
    "python3 bench.py --summarize-configs gpurun_out/cfg_trace/trace_results.db "
    "gpurun_out/cfg_fetch/fetch_results.db gpurun_out/cfg_write/write_results.db",
]


def _dispatches(db, counter=None):
    """The library's kernel dispatches of a rocpd database in dispatch order: (name, duration
    us, vgprs, accum vgprs, lds bytes, scratch bytes, workgroup size) from a kernel trace, or
    (name, counter value) from a counter run."""
    import sqlite3

    con = sqlite3.connect(db)
    if counter is None:
        q = ("select name, duration, vgpr_count, accum_vgpr_count, lds_size, scratch_size, "
             "workgroup_x * workgroup_y * workgroup_z from kernels order by dispatch_id")
        rows = [(r[0], r[1] / 1000.0, *r[2:]) for r in con.execute(q)]
    else:
        q = ("select kernel_name, sum(value) from counters_collection where counter_name = ? "
             "group by dispatch_id order by dispatch_id")
        rows = list(con.execute(q, (counter,)))
    con.close()
    return [r for r in rows if "nrm::" in r[0]]


def summarize_configs(trace_db, fetch_db, write_db):
    """Per-configuration kernel time, registers, occupancy and HBM bytes (FETCH_SIZE and
    WRITE_SIZE in KiB per dispatch, scaled by what they read for the calibration copy), to
    profiles/traffic_suite_configs.json and profiles/suite_configs.md."""
    import re

    tr = _dispatches(trace_db)
    fe = _dispatches(fetch_db, "FETCH_SIZE")
    wr = _dispatches(write_db, "WRITE_SIZE")

    per_call = 1 + sum(dispatches_per_call(c) for c in CONFIG_IDS + NEXT_IDS)

    def split(rows):
        """Dispatches in run order -> {case: [per-call lists of dispatches]}."""
        calls = len(rows) // per_call
        if calls * per_call != len(rows):
            raise SystemExit(f"{len(rows)} dispatches is not a multiple of {per_call}: the run "
                             "and CONFIG_IDS + NEXT_IDS differ")
        out, i = {"cal": rows[:calls]}, calls
        for cid in CONFIG_IDS + NEXT_IDS:
            nd = dispatches_per_call(cid)
            out[cid] = [rows[i + c * nd:i + (c + 1) * nd] for c in range(calls)]
            i += nd * calls
        return out

    T, F, W = split(tr), split(fe), split(wr)
    for name, *_ in T["cal"] + F["cal"] + W["cal"]:
        assert "copy16_kernel" in name, name
    cal_f = statistics.median(v for _, v in F["cal"])
    cal_w = statistics.median(v for _, v in W["cal"])
    scale_f, scale_w = CAL_BYTES / (cal_f * 1024), CAL_BYTES / (cal_w * 1024)

    def short(n):
        n = re.sub(r"\(nrm::\w+\)$", "", n.replace("void ", "").replace("nrm::", ""))
        n = re.sub(r"\(.*\)$", "", n)
        return n if len(n) < 60 else n[:57] + "..."

    cases = {}
    for cid in CONFIG_IDS + NEXT_IDS:
        calls_t = T[cid]
        main = [c[0] for c in calls_t]
        us = statistics.median(sum(d[1] for d in c) for c in calls_t)
        f_kib = statistics.median(sum(d[1] for d in c) for c in F[cid])
        w_kib = statistics.median(sum(d[1] for d in c) for c in W[cid])
        name, _, vg, avg, lds, scr, wg = main[0]
        # rocprofv3 reports half the compiler's VGPR count on gfx950 (the compiler's 46, 54,
        # 128 and 157 read as 24, 28, 64 and 80): the compiler's count is twice the field.
        vgprs = 2 * (vg + avg)
        waves_per_simd = min(8, 512 // max(8, (vgprs + 7) // 8 * 8))
        cases[cid] = {"kernel": short(name), "dispatches_per_call": len(calls_t[0]),
                      "us_median": round(us, 2), "vgprs": vgprs, "trace_vgpr_count": vg,
                      "accum_vgprs": avg, "lds_bytes": lds, "scratch_bytes_per_lane": scr,
                      "workgroup": wg, "waves_per_simd_by_vgprs": waves_per_simd,
                      "fetch_MB": round(f_kib * 1024 * scale_f / 1e6, 2),
                      "write_MB": round(w_kib * 1024 * scale_w / 1e6, 2)}
    meta = _case_meta()
    for cid, c in cases.items():
        alg = meta[cid]["bytes"]
        c["algorithmic_MB"] = round(alg / 1e6, 2)
        c["traffic_over_algorithmic"] = round((c["fetch_MB"] + c["write_MB"]) * 1e6 / alg, 4)
        c["GBps_trace"] = round(alg / (c["us_median"] * 1e-6) / 1e9, 1)
        c["pct_peak_trace"] = round(100 * alg / (c["us_median"] * 1e-6) / 8e12, 1)
        c["op"] = meta[cid]["op"]
        c["shape"] = meta[cid]["shape"]
    summary = {"library_source_hash": library_source_hash(), "fetch_scale": scale_f,
               "write_scale": scale_w, "calibration_bytes_each_way": CAL_BYTES,
               "commands": CONFIG_CMDS, "cases": cases}
    with open(SUITE_TRAFFIC_FILE, "w") as fh:
        json.dump(summary, fh, indent=1)
    L = ["# Every configuration on one MI355X: kernel time, registers and HBM traffic", "",
         "`bench.py --counters` calls each synthetic configuration (1-5d) and one workload of "
         "each other operation (6a-9e) eagerly, one call at a time; a kernel trace (20 calls "
         "each) gives the time and the registers, and two counter runs (3 calls each) give "
         "FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what it reads for a copy of "
         f"{CAL_BYTES // 2**20} MiB each way (x{scale_f:.3f} fetch, x{scale_w:.3f} write). "
         "The calls of a workload run back to back; workloads under 512 MB run here without "
         "buffer rotation, so their repeat calls may hit the Infinity Cache (the counters "
         "count L2 misses either way), and the suite's graph-timed lines remain the reference "
         "for time.", "",
         f"Library sources hash: `{summary['library_source_hash']}`.", "",
         "From the repository root, with `TMPDIR=/tmp`:", "", "```", *CONFIG_CMDS, "```", "",
         "VGPRs are the compiler's count (rocprofv3's vgpr_count field reads half of it on "
         "gfx950); waves/SIMD is what that count allows (8 at most); scratch is bytes per lane "
         "(register spills). Traffic above 1.0 is the backward's fp64 partial column sums "
         "(16.8 MB per parameter at [16384, 8192], written and read once), register spills, or a second read "
         "that missed the Infinity Cache (the cross-entropy gradient).", "",
         "| cfg | op | kernel | us | % of 8 TB/s | VGPRs | waves/SIMD | scratch B/lane | fetch MB | "
         "write MB | algorithmic MB | traffic / algorithmic |",
         "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for cid, c in cases.items():
        L.append(f"| {cid} | {c['op']} | `{c['kernel']}` | {c['us_median']:.2f} | "
                 f"{c['pct_peak_trace']:.1f} | {c['vgprs']} | {c['waves_per_simd_by_vgprs']} | "
                 f"{c['scratch_bytes_per_lane']} | {c['fetch_MB']:.1f} | {c['write_MB']:.1f} | "
                 f"{c['algorithmic_MB']:.1f} | {c['traffic_over_algorithmic']:.3f} |")
    with open(SUITE_MD, "w") as f:
        f.write("\n".join(L) + "\n")
    print("\n".join(L))


def _case_meta():
    """op, shape and algorithmic bytes of each case, without a GPU (the same formulas as
    build_case)."""
    m = {}
    for cid, shape, es in (("1", (64, 512), 4), ("2", (4096, 4096), 2), ("5a", (16384, 8192), 2),
                           ("5b", (16384, 8192), 4), ("5c", (65536, 5120), 2),
                           ("5d", (65536, 5120), 4)):
        m[cid] = {"op": "add_rms_norm", "shape": list(shape),
                  "bytes": add_rms_bytes(shape[0], shape[1], es, es)}
    m["3a"] = {"op": "layer_norm", "shape": [16384, 8192], "bytes": 2 * 16384 * 8192 * 2 + 2 * 8192 * 2}
    m["3b"] = {"op": "layer_norm_no_affine", "shape": [16384, 8192], "bytes": 2 * 16384 * 8192 * 2}
    for cid, op in (("4a", "norm_rope_half"), ("4b", "norm_rope_interleaved"),
                    ("4c", "norm_rope_cache_half"), ("4d", "norm_rope_cache_interleaved")):
        m[cid] = {"op": op, "shape": [8, 32, 512, 128], "bytes": 2 * 8 * 32 * 512 * 128 * 2 + 128 * 2}
    m["6a"] = {"op": "rms_norm_vjp", "shape": [16384, 8192], "bytes": 3 * 16384 * 8192 * 2 + 8192 * 2 * 2}
    m["7a"] = {"op": "layer_norm_vjp", "shape": [16384, 8192], "bytes": 3 * 16384 * 8192 * 2 + 8192 * 2 * 3}
    m["8a"] = {"op": "rope_positions_llama3", "shape": [16384, 32, 8, 128],
               "bytes": 2 * 16384 * 40 * 128 * 2 + 16384 * 8 + 64 * 4}
    m["8b"] = {"op": "rope", "shape": [8, 32, 512, 128], "bytes": 2 * 8 * 32 * 512 * 128 * 2}
    m["9a"] = {"op": "softmax", "shape": [16384, 8192], "bytes": 2 * 16384 * 8192 * 2}
    m["9b"] = {"op": "causal_softmax", "shape": [256, 512, 512],
               "bytes": 256 * (512 * 513 // 2) * 2 + 256 * 512 * 512 * 2}
    rows, V = 4096, 128256
    m["9c"] = {"op": "logsumexp", "shape": [rows, V], "bytes": rows * V * 2 + rows * 2}
    m["9d"] = {"op": "cross_entropy", "shape": [rows, V], "bytes": rows * V * 2 + rows * 12}
    m["9e"] = {"op": "cross_entropy_vjp", "shape": [rows, V], "bytes": 2 * rows * V * 2 + rows * 12}
    return m


def sweep(args):
    """Bandwidth across row widths: one line per (operation, dtype, width) to stderr, each call
    moving about 256 MB (rows = 256 MB / the row's bytes), timed like the suite lines. It shows
    how each kernel shape holds up away from the benchmark's widths."""
    import torch

    import transformer_row_wise_amd as nrm

    nrm.load()
    target = 256 * 2**20
    dts = {"bf16": torch.bfloat16, "f32": torch.float32}

    def run(op, dt, shape, fn, nbytes):
        avg = statistics.median(time_graph(lambda i: fn(), 24))
        gbps = nbytes / (avg * 1e-3) / 1e9
        print(json.dumps({"sweep": op, "dtype": dt, "shape": shape, "bytes": nbytes,
                          "gpu_us_median": round(avg * 1e3, 2), "gpu_GBps": round(gbps, 1),
                          "pct_peak": round(100 * gbps / PEAK_GBPS, 1)}), file=sys.stderr,
              flush=True)

    for dt in ("bf16", "f32"):
        es = 2 if dt == "bf16" else 4
        for H in (64, 128, 256, 512, 1024, 2048, 4096, 5120, 8192, 12288, 16384, 32768):
            R = max(64, target // (H * es * 4))
            x = torch.randn(R, H, device="cuda").to(dts[dt])
            r = torch.randn(R, H, device="cuda").to(dts[dt])
            w = torch.ones(H, device="cuda").to(dts[dt])
            b = torch.zeros(H, device="cuda").to(dts[dt])
            out, h = torch.empty_like(x), torch.empty_like(x)
            n = x.numel() * es
            run("add_rms_norm", dt, [R, H], lambda: nrm.add_rms_norm(x, r, w, 1e-6, out=out, h=h), 4 * n)
            run("rms_norm", dt, [R, H], lambda: nrm.rms_norm(x, w, 1e-6, out=out), 2 * n)
            run("layer_norm", dt, [R, H], lambda: nrm.layer_norm(x, w, b, 1e-5, out=out), 2 * n)
            del x, r, out, h
        for H in (64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384):
            R = max(64, target // (H * es * 3))
            x = torch.randn(R, H, device="cuda").to(dts[dt])
            g = torch.randn(R, H, device="cuda").to(dts[dt])
            w = torch.ones(H, device="cuda").to(dts[dt])
            dx, dw, db = torch.empty_like(x), torch.empty_like(w), torch.empty_like(w)
            ws = torch.empty(nrm.vjp_workspace_bytes(R, H, True), dtype=torch.uint8, device="cuda")
            n = x.numel() * es
            run("rms_norm_vjp", dt, [R, H],
                lambda: nrm.rms_norm_vjp(x, w, g, 1e-6, dx=dx, dw=dw, workspace=ws), 3 * n)
            run("layer_norm_vjp", dt, [R, H],
                lambda: nrm.layer_norm_vjp(x, w, g, 1e-5, dx=dx, dw=dw, db=db, workspace=ws), 3 * n)
            del x, g, dx
        for V in (128, 512, 2048, 8192, 16384, 32000, 65536, 128256, 151936):
            R = max(64, target // (V * es * 2))
            x = torch.randn(R, V, device="cuda").to(dts[dt])
            out = torch.empty_like(x)
            lse = torch.empty(R, 1, device="cuda").to(dts[dt])
            tg = torch.randint(0, V, (R,), device="cuda")
            gl = torch.ones(R, device="cuda")
            loss = torch.empty(R, device="cuda")
            n = x.numel() * es
            run("softmax", dt, [R, V], lambda: nrm.softmax(x, out=out), 2 * n)
            run("logsumexp", dt, [R, V], lambda: nrm.logsumexp(x, out=lse), n)
            run("cross_entropy", dt, [R, V], lambda: nrm.cross_entropy(x, tg, loss=loss), n)
            run("cross_entropy_vjp", dt, [R, V],
                lambda: nrm.cross_entropy_vjp(x, tg, gl, dlogits=out), 2 * n)
            del x, out
    for B, H, L, D in ((1, 32, 4096, 128), (8, 32, 512, 128), (4, 8, 8192, 64),
                       (2, 16, 2048, 256), (1, 64, 8192, 128)):
        x = torch.randn(B, H, L, D, device="cuda").to(torch.bfloat16)
        out = torch.empty_like(x)
        w = torch.ones(D, device="cuda").to(torch.bfloat16)
        n = x.numel() * 2
        run("rope", "bf16", [B, H, L, D], lambda: nrm.rope(x, out=out), 2 * n)
        run("norm_rope", "bf16", [B, H, L, D], lambda: nrm.norm_rope(x, w, out=out), 2 * n)


# --------------------------------------------------------------------------- counters

def _pmc_per_dispatch(path, counter):
    """{kernel name: [value per dispatch]} from a rocprofv3 counter file: the rocpd SQLite
    database (its `counters_collection` view) or a counter_collection.csv."""
    out = {}
    if path.endswith(".db"):
        import sqlite3

        con = sqlite3.connect(path)
        q = "select kernel_name, value from counters_collection where counter_name = ? order by id"
        for name, value in con.execute(q, (counter,)):
            out.setdefault(name, []).append(float(value))
        con.close()
        return out
    import csv

    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def summarize_pmc(fetch_file, write_file, copy_bytes_half):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the headline kernel, each scaled by the
    ratio of known bytes to the counter's reading for the 16-byte copy kernel."""
    f = _pmc_per_dispatch(fetch_file, "FETCH_SIZE")
    w = _pmc_per_dispatch(write_file, "WRITE_SIZE")

    def pick(d, key):
        ks = [k for k in d if key in k]
        if not ks:
            raise SystemExit(f"no dispatch of {key} in the counter file")
        vals = d[ks[0]]
        return statistics.median(vals), ks[0]

    kf, kname = pick(f, HEADLINE_KERNEL)
    kw, _ = pick(w, HEADLINE_KERNEL)
    cf, _ = pick(f, COPY_KERNEL)
    cw, _ = pick(w, COPY_KERNEL)
    scale_f = copy_bytes_half / (cf * 1024)
    scale_w = copy_bytes_half / (cw * 1024)
    read_b = kf * 1024 * scale_f
    write_b = kw * 1024 * scale_w
    alg = add_rms_bytes(ROWS, HIDDEN, 2, 2)
    summary = {
        "kernel": kname,
        "workload": "add-RMSNorm bf16 [16384, 8192]",
        "kernel_source_hash": kernel_source_hash(),
        "fetch_KiB_per_dispatch": kf, "write_KiB_per_dispatch": kw,
        "copy_fetch_KiB": cf, "copy_write_KiB": cw, "copy_bytes_each_way": copy_bytes_half,
        "fetch_scale": scale_f, "write_scale": scale_w,
        "hbm_read_bytes_per_launch": round(read_b), "hbm_write_bytes_per_launch": round(write_b),
        "hbm_bytes_per_launch": round(read_b + write_b),
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": round((read_b + write_b) / alg, 4),
        "commands": PMC_CMDS,
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(summary, fh, indent=1)
    print(json.dumps(summary, indent=1))


PROFILE_MD = os.path.join(ROOT, "profiles", "add_rms_norm_bf16_16384x8192.md")
TRACE_CMD = ("rocprofv3 --kernel-trace --stats -d gpurun_out/prof_trace -o trace -- "
             "python3 bench.py --profile --steps 100 --warmup 1000")
PMC_CMDS = [
    "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o fetch -- "
    "python3 bench.py --profile --steps 5 --warmup 2",
    "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o write -- "
    "python3 bench.py --profile --steps 5 --warmup 2",
    "python3 bench.py --summarize-pmc gpurun_out/pmc_fetch/fetch_results.db "
    "gpurun_out/pmc_write/write_results.db",
]


def summarize_trace(trace_db):
    """Kernel-trace statistics (rocpd database of a --profile run) plus the counter summary,
    written to profiles/add_rms_norm_bf16_16384x8192.md."""
    import sqlite3

    con = sqlite3.connect(trace_db)
    rows = list(con.execute("select name, total_calls, total_duration, average from top_kernels"))
    durs = {}
    for name, d in con.execute("select name, duration from kernels order by start"):
        durs.setdefault(name, []).append(d / 1000.0)
    con.close()
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    alg = add_rms_bytes(ROWS, HIDDEN, 2, 2)
    L = ["# add-RMSNorm bf16 [16384, 8192] on one MI355X: kernel trace and HBM traffic", "",
         "Workload: x, r Student-t(3) with 1% of rows x1e3, w ~ N(1, 0.1) bf16, eps 1e-6. "
         "`bench.py --profile` first runs the copy ceilings over the same byte count (the "
         "16-byte copy, the two-into-two copy, and the two-into-two copy in the row kernel's "
         "work unit; they also bring the clocks up), then the headline kernel (1000 warm-up + 100 timed calls).", "",
         f"Kernel sources hash (`bench.py` `kernel_source_hash`) of the counter runs: "
         f"`{t['kernel_source_hash']}`.", "",
         "## Kernel trace (`rocprofv3 --kernel-trace --stats`)", "",
         "From the repository root, with `TMPDIR=/tmp`:", "", "```", TRACE_CMD,
         f"python3 bench.py --summarize-trace gpurun_out/prof_trace/trace_results.db", "```", "",
         "| kernel | calls | average us | last 100 average us | min us | max us |",
         "|---|---|---|---|---|---|"]
    for name, calls, _tot, avg in rows:
        d = durs.get(name, [avg])
        tail = d[-100:]
        L.append(f"| `{name}` | {calls} | {avg:.2f} | {sum(tail) / len(tail):.2f} | "
                 f"{min(d):.2f} | {max(d):.2f} |")
    kavg = [r[3] for r in rows if HEADLINE_KERNEL in r[0]][0]
    cavg = [r[3] for r in rows if COPY_KERNEL in r[0] and COPY2_KERNEL not in r[0]][0]
    c2 = [r[3] for r in rows if COPY2_KERNEL in r[0]]
    cb = 2 * ((alg // 2) // 16 * 16)
    cb2 = 4 * ((alg // 4) // 16 * 16)
    two = (f" Two arrays into two (the headline's pattern without arithmetic): "
           f"{cb2 / (c2[0] * 1e-6) / 1e9:.0f} GB/s ({100 * cb2 / (c2[0] * 1e-6) / 8e12:.1f}%)."
           if c2 else "")
    c3 = [r[3] for r in rows if COPY2_ROW_KERNEL in r[0]]
    cb3 = 4 * ROWS * HIDDEN * 2
    two += (f" The same copy in the row kernel's work unit (each 512-thread block loads a row's "
            f"16 KB of each array and stores nothing until all of it has arrived): "
            f"{cb3 / (c3[0] * 1e-6) / 1e9:.0f} GB/s ({100 * cb3 / (c3[0] * 1e-6) / 8e12:.1f}%)."
            if c3 else "")
    L += ["", f"Headline kernel: {alg:,} algorithmic bytes / {kavg:.2f} us = "
          f"{alg / (kavg * 1e-6) / 1e9:.0f} GB/s ({100 * alg / (kavg * 1e-6) / 8e12:.1f}% of 8 TB/s). "
          f"Copy of the same byte count: {cb / (cavg * 1e-6) / 1e9:.0f} GB/s "
          f"({100 * cb / (cavg * 1e-6) / 8e12:.1f}%).{two}", "",
          "## HBM bytes (`rocprofv3 --pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, one counter per run)",
          "", "```", *PMC_CMDS, "```", "",
          "| quantity | FETCH_SIZE | WRITE_SIZE |", "|---|---|---|",
          f"| headline kernel, KiB per dispatch (median) | {t['fetch_KiB_per_dispatch']:.0f} | "
          f"{t['write_KiB_per_dispatch']:.0f} |",
          f"| copy16_kernel, KiB per dispatch (median) | {t['copy_fetch_KiB']:.1f} | "
          f"{t['copy_write_KiB']:.1f} |",
          f"| copy16_kernel, known bytes each way | {t['copy_bytes_each_way']:,} | "
          f"{t['copy_bytes_each_way']:,} |",
          f"| scale = known bytes / counter bytes | {t['fetch_scale']:.4f} | {t['write_scale']:.4f} |",
          f"| headline kernel, scaled bytes per launch | {t['hbm_read_bytes_per_launch']:,} | "
          f"{t['hbm_write_bytes_per_launch']:,} |",
          f"| algorithmic bytes per launch | {2 * ROWS * HIDDEN * 2 + HIDDEN * 2:,} (x, r, w) | "
          f"{2 * ROWS * HIDDEN * 2:,} (out, h) |", "",
          f"Traffic / algorithmic = {t['traffic_over_algorithmic']}: x and r are read from HBM "
          "once and out and h written once; w (16 KiB) comes from L2. On this GPU FETCH_SIZE "
          "counts half of the copy's known read bytes, hence the x2 scale.", ""]
    with open(PROFILE_MD, "w") as f:
        f.write("\n".join(L))
    print("\n".join(L))


SUITE_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -d gpurun_out/prof_suite -o suite -- "
                   "python3 bench.py --only vjp,rope,sm")
SUITE_TRACE_MD = os.path.join(ROOT, "profiles", "suite_kernels_backward_rope_softmax.md")
COUNTERS_CMD = ("rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE "
                "-d gpurun_out/pmc_valu -o valu -- python3 bench.py --only fwd,vjp,sm "
                "--no-cpu-baseline")
COUNTERS_MD = os.path.join(ROOT, "profiles", "valu_issue_suite_kernels.md")


def summarize_suite_trace(trace_db):
    """Per-kernel statistics of a kernel-trace run of the backward, rope and softmax suite
    groups, written to profiles/suite_kernels_backward_rope_softmax.md."""
    import re
    import sqlite3

    con = sqlite3.connect(trace_db)
    rows = list(con.execute("select name, total_calls, average from top_kernels"))
    mins = {n: (lo / 1000.0, hi / 1000.0) for n, lo, hi in
            con.execute("select name, min(duration), max(duration) from kernels group by name")}
    con.close()

    def short(n):
        n = re.sub(r"\(nrm::\w+\)$", "", n.replace("void ", ""))
        return n if len(n) < 90 else n[:87] + "..."

    L = ["# Backward, Rope and softmax-family kernels on one MI355X: kernel trace", "",
         "`bench.py --only vjp,rope,sm` times each workload of those groups from captured HIP "
         "graphs (cfg 6a-9e); under the profiler every kernel launch of those graphs (and of "
         "their warm-up replays) is traced. Average durations here are per launch and "
         "agree with the suite's per-call figures, which add the small column-sum kernel of "
         "the backward.", "", "From the repository root, with `TMPDIR=/tmp`:", "", "```",
         SUITE_TRACE_CMD, "python3 bench.py --summarize-suite-trace "
         "gpurun_out/prof_suite/suite_results.db", "```", "",
         "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for name, calls, avg in rows:
        if not name.startswith("void nrm::") and not name.startswith("nrm::"):
            continue
        lo, hi = mins.get(name, (avg, avg))
        L.append(f"| `{short(name)}` | {calls} | {avg:.2f} | {lo:.2f} | {hi:.2f} |")
    with open(SUITE_TRACE_MD, "w") as f:
        f.write("\n".join(L) + "\n")
    print("\n".join(L))


def summarize_counters(db):
    """VALU issue share per kernel from a `--pmc SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU
    GRBM_GUI_ACTIVE` run of suite groups, written to profiles/valu_issue_suite_kernels.md."""
    import re
    import sqlite3

    con = sqlite3.connect(db)
    vals = {}
    for name, cn, v in con.execute(
            "select kernel_name, counter_name, value from counters_collection order by id"):
        vals.setdefault(name, {}).setdefault(cn, []).append(float(v))
    con.close()

    def short(n):
        n = re.sub(r"\(nrm::\w+\)$", "", n.replace("void ", ""))
        n = re.sub(r"\(double const\*.*\)$", "", n)
        return n if len(n) < 70 else n[:67] + "..."

    L = ["# VALU issue of the suite kernels on one MI355X (`rocprofv3 --pmc`)", "",
         "Counters per dispatch (median over the dispatches of each kernel) of a run of the "
         "forward, backward and softmax suite groups. GRBM_GUI_ACTIVE reads the sum over the "
         "8 XCDs: an eighth of it, at 2.4 GHz, matches each kernel's traced duration. "
         "`VALU share` = SQ_INSTS_VALU x 4 cycles (a wave64 instruction on a 16-lane SIMD) / "
         "(1024 SIMDs x the per-XCD active cycles): near 100% the kernel is bound by "
         "instruction issue, not by HBM. A kernel that serves several workloads (the same "
         "template at several shapes) shows the median over all of its dispatches; under the "
         "counters every dispatch runs alone, so durations exceed the suite's.", "", "From the repository root, with `TMPDIR=/tmp`:",
         "", "```", COUNTERS_CMD, "python3 bench.py --summarize-counters "
         "gpurun_out/pmc_valu/valu_results.db", "```", "",
         "| kernel | dispatches | us (active cycles / 8 / 2.4 GHz) | VALU instructions per wave "
         "| VALU share |", "|---|---|---|---|---|"]
    for name, cs in sorted(vals.items()):
        if "nrm::" not in name or "GRBM_GUI_ACTIVE" not in cs or "SQ_INSTS_VALU" not in cs:
            continue
        gui = statistics.median(cs["GRBM_GUI_ACTIVE"]) / 8
        vi = statistics.median(cs["SQ_INSTS_VALU"])
        waves = statistics.median(cs["SQ_WAVES"])
        share = 4 * vi / 1024 / gui if gui else 0.0
        L.append(f"| `{short(name)}` | {len(cs['SQ_INSTS_VALU'])} | {gui / 2400:.1f} | "
                 f"{vi / waves:.0f} | {100 * share:.0f}% |")
    with open(COUNTERS_MD, "w") as f:
        f.write("\n".join(L) + "\n")
    print("\n".join(L))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--suite", action="store_true")
    ap.add_argument("--only", metavar="GROUPS",
                    help="with --suite: comma-separated groups among fwd, vjp, rope, sm "
                         "(skips the headline line)")
    ap.add_argument("--sweep", action="store_true",
                    help="bandwidth across row widths, one line per case (stderr)")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_FILE", "WRITE_FILE"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DB")
    ap.add_argument("--summarize-suite-trace", metavar="TRACE_DB")
    ap.add_argument("--summarize-counters", metavar="PMC_DB")
    ap.add_argument("--counters", action="store_true",
                    help="eager calls of every configuration, for rocprofv3 runs")
    ap.add_argument("--counter-calls", type=int, default=3)
    ap.add_argument("--summarize-configs", nargs=3, metavar=("TRACE_DB", "FETCH_DB", "WRITE_DB"))
    args = ap.parse_args()
    if args.summarize_configs:
        summarize_configs(*args.summarize_configs)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return 0
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return 0
    if args.summarize_suite_trace:
        summarize_suite_trace(args.summarize_suite_trace)
        return 0
    if args.summarize_pmc:
        half = (add_rms_bytes(ROWS, HIDDEN, 2, 2) // 2) // 16 * 16
        summarize_pmc(*args.summarize_pmc, copy_bytes_half=half)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path (rows are "
              f"independent, so N GPUs would each run this same kernel on their own rows); "
              f"got --gpus {args.gpus}", file=sys.stderr)
        return 2
    if args.sweep:
        sweep(args)
        return 0
    if args.counters:
        counter_run(args)
        return 0
    if not args.only:
        headline(args)
    if args.suite or args.only:
        suite(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
