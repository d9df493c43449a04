#!/usr/bin/env python3
"""Benchmark of the fused row-wise normalisation library on one MI355X.

Default run: one JSON line on stdout for the headline workload, residual add-RMSNorm in bf16
storage at [16384, 8192] (x and r Student-t(3) with 1% of rows scaled by 1e3, w ~ N(1, 0.1),
eps 1e-6), inputs resident in HBM. A step is one nrm_add_rms_norm call: load x and r, add,
round and store h, sum of squares, row scalar, normalise, scale by w, round and store out.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--suite] [--no-cpu-baseline]

--suite        also prints one JSON line per synthetic workload (all four ops) to stderr,
               rotating buffer sets when a call's working set would fit in the 256 MB
               Infinity Cache.
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
arrays copied into two, the headline's byte pattern without arithmetic), copy_ceiling_GBps (a
plain 16-byte copy of the same byte count), and cpu_baseline (the fp64 oracle on a bounded
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

    # The copy ceilings run first: about 1.3 s of streaming at the same byte count, which
    # brings the GPU to the clocks it holds under sustained load (it needs about a second), so
    # that the headline's few timed steps are not taken on the way up. Under a profiler they
    # stay short.
    copy_steps = max(100, args.steps // 2) if args.profile else 2000
    print(f"# copy ceilings, {copy_steps} steps each", file=sys.stderr, flush=True)
    ceiling = copy_ceiling(nbytes, copy_steps)
    ceiling2 = copy2_ceiling(nbytes, copy_steps)
    print(f"# timing {args.steps} steps after {args.warmup} warm-up", file=sys.stderr, flush=True)
    gpu_ms, wall_ms = time_calls(step, args.steps, args.warmup)
    achieved = nbytes / (gpu_ms * 1e-3) / 1e9
    value = nbytes / (wall_ms * 1e-3) / 1e9
    if args.profile:
        print(json.dumps({"profile_run": True, "avg_launch_us": gpu_ms * 1e3,
                          "achieved_GBps": achieved, "copy_GBps": ceiling,
                          "copy2_GBps": ceiling2}), flush=True)
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
                          "rows_per_s": round(rows / (avg * 1e-3), 1)}), file=sys.stderr,
              flush=True)

    def run_add(cfg, inp):
        rows, hidden = inp.x.shape
        es = inp.x.element_size()
        nbytes = add_rms_bytes(rows, hidden, es, inp.w.element_size())
        sets = [(inp.x.cuda(), inp.r.cuda()) for _ in range(n_sets(nbytes))]
        w = inp.w.cuda()
        outs = [(torch.empty_like(s[0]), torch.empty_like(s[0])) for s in sets]
        per = time_graph(lambda i: nrm.add_rms_norm(*sets[i % len(sets)], w, inp.eps,
                                                    out=outs[i % len(sets)][0],
                                                    h=outs[i % len(sets)][1]), calls(nbytes))
        emit(cfg, "add_rms_norm", [rows, hidden, str(inp.x.dtype)], nbytes, rows, per)

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
    run_add("1", workloads.cfg_add_rms_small_f32())
    run_add("2", workloads.cfg_add_rms_4k_bf16())
    for affine in (True, False):
        inp = workloads.cfg_layer_norm_bf16(affine=affine)
        rows, hidden = inp.x.shape
        nbytes = 2 * rows * hidden * 2 + (2 * hidden * 2 if affine else 0)
        x = inp.x.cuda()
        w = inp.w.cuda() if affine else None
        b = inp.b.cuda() if affine else None
        out = torch.empty_like(x)
        per = time_graph(lambda i: nrm.layer_norm(x, w, b, inp.eps, out=out), calls(nbytes))
        emit("3a" if affine else "3b", "layer_norm", [rows, hidden], nbytes, rows, per)
        del x, out
    def run_copy(cfg, nbytes):
        """The 16-byte copy moving the same bytes (half in, half out): the small-call ceiling."""
        half = (nbytes // 2) // 16 * 16
        k = n_sets(nbytes)
        srcs = [torch.ones(half, dtype=torch.uint8, device="cuda") for _ in range(k)]
        dsts = [torch.empty_like(srcs[0]) for _ in range(k)]
        per = time_graph(lambda i: nrm.bench_copy(srcs[i % k], dsts[i % k]), calls(nbytes))
        emit(cfg, "copy (ceiling)", [half], 2 * half, 0, per)

    run_copy("4-copy", 2 * 8 * 32 * 512 * 128 * 2)
    for cache in (False, True):
        for trad in (False, True):
            rp = workloads.cfg_norm_rope_bf16(offset=workloads.NORM_ROPE_CACHE_OFFSET if cache else 0)
            B, H, L, D = rp.x.shape
            nbytes = 2 * B * H * L * D * 2 + D * 2
            k = n_sets(nbytes)
            xs = [rp.x.cuda() for _ in range(k)]
            w = rp.w.cuda()
            if cache:
                dsts = [torch.zeros(B, H, workloads.NORM_ROPE_CACHE_LEN, D, dtype=torch.bfloat16,
                                    device="cuda") for _ in range(k)]
            else:
                dsts = [torch.empty_like(xs[0]) for _ in range(k)]
            per = time_graph(
                lambda i: nrm.norm_rope(xs[i % k], w, eps=rp.eps, traditional=trad,
                                        offset=rp.offset, cache=dsts[i % k] if cache else None,
                                        out=None if cache else dsts[i % k]),
                calls(nbytes))
            emit("4" + "abcd"[2 * cache + trad], "norm_rope" + ("_cache" if cache else "") +
                 ("_interleaved" if trad else "_half"), [B, H, L, D], nbytes, B * H * L, per)
            del xs, dsts
    for shape, tag in (((16384, 8192), "5"), ((65536, 5120), "5")):
        f32 = workloads.cfg_add_rms_scale(*shape, dtype="f32")
        bf = workloads.RowInputs(x=f32.x.to(torch.bfloat16), r=f32.r.to(torch.bfloat16),
                                 w=f32.w.to(torch.bfloat16), b=None, eps=f32.eps)
        run_add(tag + ("a" if shape[1] == 8192 else "c"), bf)
        run_add(tag + ("b" if shape[1] == 8192 else "d"), f32)
        del f32, bf
        torch.cuda.empty_cache()


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
         "`bench.py --profile` runs the headline kernel (1000 warm-up + 100 timed calls) and "
         "then the 16-byte copy of the same byte count.", "",
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
                "-d gpurun_out/pmc_valu -o valu -- python3 bench.py --only fwd,vjp,sm")
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
    args = ap.parse_args()
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
    if not args.only:
        headline(args)
    if args.suite or args.only:
        suite(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
