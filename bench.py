#!/usr/bin/env python3
"""Benchmark one decode step of paged FP8 MLA attention on one MI355X.

A step is the whole hot path on one batch: the step's new latent rows go into
the FP8 cache and the split-KV decode runs in one launch
(mla_decode_paged_append: kv_append_fp8 + mla_decode_paged; an extend chunk of
more than 16 rows per request gets the append's own launch inside that call),
then mla_decode_combine (--separate-append issues kv_append_fp8 on its own).  Steps are
timed twice, launched eagerly and as replays of HIP graphs that each hold one
step on every rotated cache in turn (a serving loop's form: a model's
consecutive layers, each with its own cache, in one graph); the step time is
the faster of the two, both reported.  The decode
kernel's own duration comes from HIP events around a burst of back-to-back
decode launches, and, for its spread, around every launch of the eager pass
(--no-graph times eager steps only).  The default
workload is one request of 64 heads over a 100,000-token FP8 e4m3 cache
(+1 appended row) with a per-tensor scale, randomly permuted 64-token pages.

Inputs sit in HBM before timing starts.  Between steps the benchmark rotates
over several copies of the cache (default 8 x 57.6 MB, more than the 256 MB
last-level cache) so that every step reads its cache from HBM, as consecutive
layers of a model would.

Prints one JSON line: the throughput in KV-tokens/s, plus
* roofline: the decode kernel's algorithmic bytes per launch / its mean
  duration (HIP events around a burst of back-to-back launches on its
  stream) against 8 TB/s;
* cpu_baseline: the CPU oracle timed on a bounded sample of the same workload
  (all cores, and one thread), with the host's CPU model;
* measured_peaks: this GPU's streaming-read, LDS-DMA page-stream and bf16
  MFMA peaks from the library's microbenchmarks (--no-peaks skips them), and
  the roofline fraction against them beside the vendor figure.
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

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "MLA decode KV-tokens/s, HBM TB/s and % roofline, FP8 paged cache @100k ctx"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # steady state: after 20 warm-up steps the replayed steps still ran about 10 % slower than
    # after 1,000 (about 30 ms at 100k tokens); the timed steps are the same either way
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", default="fp8_single_100k")
    ap.add_argument("--rotate", type=int, default=8, help="distinct cache copies cycled over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--cpu-repeats", type=int, default=3, help="at least this many oracle runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="and oracle runs until this much CPU time has passed")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--max-splits", type=int, default=0)
    ap.add_argument("--separate-append", action="store_true",
                    help="kv_append_fp8 as its own launch before mla_decode_paged")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graphs)")
    ap.add_argument("--no-page-check", action="store_true",
                    help="skip timing the KV page-tag check in front of the step")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes --steps times (the "
                         "reference reading for HBM traffic counters) and exit")
    return ap.parse_args()


def copy_probe(nbytes, steps):
    """A plain copy of known size: FETCH_SIZE / WRITE_SIZE read under it calibrate
    the counter units against bytes actually moved."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": steps}), flush=True)


# the sources the FP8 decode kernel is compiled from (host-side planning and
# the other kernels do not change its traffic)
KERNEL_SOURCES = ("mla_decode_fp8.hip", "decode_tile.h", "device_common.h", "launch.h", "page_check.h")


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_mla_amd", "csrc")
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"mla_decode_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, repeats, seconds):
    """The oracle, as it stands, on the same workload: one full step (append of
    the new row + attention of every head over the whole context) for request 0,
    timed with every core numpy's BLAS uses and again with one thread."""
    import numpy as np

    from oracle import mla as omla

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = os.cpu_count()
    if threadpool_info is not None:
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [cores])
    b = 0
    pages = w.pages_of(b)
    ts = w.tensor_scale() if w.scale_mode == "tensor" else None
    if w.cache_dtype == "bf16":
        codes = np.zeros((w.num_pages, 64, 576), np.uint16)  # bf16 bits, the cache as it is
        codes[pages] = w.page_bits(pages)
        scales = None
    else:
        codes = np.zeros((w.num_pages, 64, 576), np.uint8)
        scales = np.zeros((w.num_pages, 64), np.float32)
        c, s = omla.fill_pages_ref(w.page_bits(pages), w.scale_mode, ts)
        codes[pages], scales[pages] = c, s
    new = w.new_row_bits()[b:b + 1] if w.n_new else None
    q = w.q_bits()[b:b + 1]
    bt = w.block_table[b:b + 1]
    sl = w.seq_lens[b:b + 1]

    def run(min_runs, budget):
        times = []
        while len(times) < min_runs or sum(times) < budget:
            t0 = time.perf_counter()
            if new is not None:
                omla.append_ref(new, codes, scales, bt, sl, w.scale_mode, ts)
            omla.decode_ref(q, codes, scales, bt, sl, n_q=w.n_q, H=w.H, cache_dtype=w.cache_dtype,
                            scale_mode=w.scale_mode, softmax_scale=w.softmax_scale, tensor_scale=ts)
            times.append(time.perf_counter() - t0)
        return times

    times = run(repeats, seconds)
    t = float(np.median(times))
    times1 = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            times1 = run(1, 0.0)  # one run: the 1-thread figure is context only
    tokens = int(w.seq_lens[b])
    out = {"value": tokens / t, "unit": "KV-tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": f"request 0 of {w.name}: {'append + ' if w.n_new else ''}all {w.H} heads x {w.n_q} queries x "
                     f"{tokens} tokens, "
                     f"median of {len(times)} runs of {t:.2f} s, {sum(times):.1f} s in all (fp64 numpy)",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
    if times1:
        out["value_1thread"] = tokens / float(np.median(times1))
        out["sample_1thread"] = f"the same request on one thread: {float(np.median(times1)):.2f} s"
    return out


def measured_peaks():
    """This GPU's own peaks, measured by the library's microbenchmarks
    (long_context_mla_amd.peaks): a streaming read of 2 GiB (eight times the
    last-level cache), 36,864-byte pages into LDS by LDS-DMA (the decode
    kernel's staging) at one workgroup per compute unit, and a bf16 MFMA loop."""
    from long_context_mla_amd import peaks

    hbm, _ = peaks.hbm_read(grids=(256, 512), reps=5)
    pages = peaks.page_stream(depths=(2,), reps=5)[2]
    tflops, ghz = peaks.mfma_bf16(waves_per_simd=2)
    return {"hbm_read_GBs": round(hbm, 1), "lds_dma_page_stream_GBs": round(pages, 1),
            "mfma_bf16_TFLOPs": round(tflops, 1), "shader_clock_GHz": round(ghz, 3)}


def time_page_check(args, w, mla, torch, np, dev, stream, cap, step, bt, sl, run_checked, graphs):
    """The KV page-tag check: kv_check_pages alone (back to back inside one HIP
    graph), and the step's HIP graph without the check, with it inside the
    decode launch (mla_decode_paged_append_checked, the default: overhead_frac),
    in front of the decode, and beside the decode on a second stream, replayed
    in alternating rounds (the median round of each)."""
    rng = np.random.default_rng(77)
    tags = rng.integers(0, 2**32, size=w.num_pages, dtype=np.uint64).astype(np.uint32)
    bt_h = w.block_table
    exp = np.where(bt_h >= 0, tags[np.clip(bt_h, 0, w.num_pages - 1)], 0).astype(np.uint32)
    tags_t = torch.from_numpy(tags.view(np.int32)).to(dev)
    exp_t = torch.from_numpy(exp.view(np.int32)).to(dev)
    step.check(tags_t, bt, exp_t, sl, None, stream=stream)
    torch.cuda.synchronize()
    flagged = int((step.status != 0).sum().item())
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the kernel alone: one graph of 20 back-to-back checks (no host launch cost)
    burst = torch.cuda.CUDAGraph()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(burst, stream=cap):
            for _ in range(20):
                step.check(tags_t, bt, exp_t, sl, None, stream=cap)
    stream.wait_stream(cap)
    burst.replay()
    torch.cuda.synchronize()
    reps = max(args.steps // 20, 5)
    start.record(stream)
    for _ in range(reps):
        burst.replay()
    end.record(stream)
    torch.cuda.synchronize()
    k_us = start.elapsed_time(end) / (reps * 20) * 1000
    graphs_by_mode = {"plain": graphs}
    for mode, cm in (("sequential", "front"), ("overlapped", "stream"), ("in_launch", "launch")):
        step.check_mode = cm
        gs = []
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for k in range(args.rotate):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run_checked(k, cap, (tags_t, exp_t, None))
                gs.append(g)
        stream.wait_stream(cap)
        graphs_by_mode[mode] = gs
    step.check_mode = "launch"
    for gs in graphs_by_mode.values():
        for i in range(args.warmup):
            gs[i % args.rotate].replay()
    rounds = {m: [] for m in graphs_by_mode}
    for _ in range(5):
        for name, gs in graphs_by_mode.items():
            torch.cuda.synchronize()
            start.record(stream)
            for i in range(args.steps):
                gs[i % args.rotate].replay()
            end.record(stream)
            torch.cuda.synchronize()
            rounds[name].append(start.elapsed_time(end) / args.steps)
    med = {m: float(np.median(v)) for m, v in rounds.items()}
    torch.cuda.synchronize()
    flagged = max(flagged, int((step.status != 0).sum().item()))
    pages = int(sum(-(-int(L) // 64) for L in w.seq_lens))
    return {
        "kernel": "kv_check_pages_kernel",
        "kernel_us": round(k_us, 3),
        "bytes": pages * 16 + w.B * 12,
        "ms_per_step_graph_plain": round(med["plain"], 5),
        "ms_per_step_graph_check_first": round(med["sequential"], 5),
        "ms_per_step_graph_check_beside": round(med["overlapped"], 5),
        "ms_per_step_graph_check_in_launch": round(med["in_launch"], 5),
        "overhead_frac": round(med["in_launch"] / med["plain"] - 1.0, 4),
        "overhead_frac_check_first": round(med["sequential"] / med["plain"] - 1.0, 4),
        "overhead_frac_check_beside": round(med["overlapped"] / med["plain"] - 1.0, 4),
        "flagged_requests": flagged,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this decode path has "
              "no multi-GPU mode to benchmark.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    import numpy as np
    import torch

    import long_context_mla_amd as mla
    import synth

    dev = torch.device("cuda:0")
    w = synth.make(args.config)
    t_setup = time.time()

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q = bf16(w.q_bits())
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    new_rows = bf16(w.new_row_bits()) if w.n_new else None
    caches, scales = [], []
    fp8 = w.cache_dtype == "fp8"
    for r in range(args.rotate):
        if r == 0:
            if fp8:
                cache = torch.zeros((w.num_pages, 64, 576), dtype=torch.uint8, device=dev)
                if w.scale_mode == "token":
                    sc = torch.zeros((w.num_pages, 64), dtype=torch.float32, device=dev)
                else:
                    sc = torch.tensor([float(w.tensor_scale())], dtype=torch.float32, device=dev)
                for c0 in range(0, w.num_pages, 4096):
                    c1 = min(c0 + 4096, w.num_pages)
                    rows = bf16(w.page_bits(np.arange(c0, c1)).reshape(1, -1, 576))
                    ident = torch.arange(c0, c1, dtype=torch.int32, device=dev).view(1, -1)
                    mla.kv_append_fp8(rows, cache, sc, w.scale_mode, ident,
                                      torch.tensor([(c1 - c0) * 64], dtype=torch.int32, device=dev))
            else:
                cache = torch.empty((w.num_pages, 64, 576), dtype=torch.bfloat16, device=dev)
                for c0 in range(0, w.num_pages, 4096):
                    c1 = min(c0 + 4096, w.num_pages)
                    cache[c0:c1] = bf16(w.page_bits(np.arange(c0, c1)))
                sc = None
        else:
            cache = caches[0].clone()
            sc = None if scales[0] is None else scales[0].clone()
        caches.append(cache)
        scales.append(sc)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    pps = args.pages_per_split or None
    ms = args.max_splits or None
    step = mla.DecodeStep(w.B, w.n_q, w.H, w.max_blocks, int(w.seq_lens.max()), w.total_tokens(), dev,
                          pages_per_split=pps, max_splits=ms, seq_lens_host=w.seq_lens, cache_dtype=w.cache_dtype)
    stream = torch.cuda.current_stream()

    def run(i, ev=None, st=None, lens=None):
        st = st or stream
        sl_ = sl if lens is None else lens
        k = i % args.rotate
        fused = new_rows is not None and not args.separate_append
        if new_rows is not None and not fused:
            mla.kv_append_fp8(new_rows, caches[k], scales[k], w.scale_mode, bt, sl_, stream=st)
        if ev is not None:
            ev[0].record(st)
        if fused:
            mla.mla_decode_paged_append(new_rows, q, caches[k], scales[k], w.scale_mode, bt, sl_,
                                        w.softmax_scale, step.pps, step.max_splits, step.o_partial,
                                        step.lse_partial, step.out, step.lse, stream=st)
        else:
            step.decode(q, caches[k], scales[k], w.scale_mode, bt, sl_, w.softmax_scale, stream=st)
        if ev is not None:
            ev[1].record(st)
        step.combine(sl_, stream=st)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    # Pass 1, eager launches: HIP events around every decode launch on its
    # stream give the decode kernel's duration (the roofline figure).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        run(args.warmup + i, evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_step_eager = start.elapsed_time(end) / args.steps
    k_ms = np.array([a.elapsed_time(b) for a, b in evs])
    k_us = float(k_ms.mean() * 1000)
    ms_step = ms_step_eager
    ms_step_graph = None
    page_check = None
    # Pass 1b: the decode launches alone, back to back on the stream, between
    # one pair of events: the per-launch figure holds the kernel plus the
    # dispatch gap between two kernels, not the latency of an event record.
    def run_decode(i):
        k = i % args.rotate
        if new_rows is not None and not args.separate_append:
            mla.mla_decode_paged_append(new_rows, q, caches[k], scales[k], w.scale_mode, bt, sl,
                                        w.softmax_scale, step.pps, step.max_splits, step.o_partial,
                                        step.lse_partial, step.out, step.lse, stream=stream)
        else:
            step.decode(q, caches[k], scales[k], w.scale_mode, bt, sl, w.softmax_scale, stream=stream)

    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        run_decode(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    k_us_burst = start.elapsed_time(end) / args.steps * 1000
    if not args.no_graph:
        # Pass 2: the steps as HIP graphs replayed back to back, as a serving
        # loop runs a model's layers: one graph holds one step on each rotated
        # cache in turn (consecutive layers, each with its own cache), so the
        # host's launch cost is paid once per `rotate` steps.  A step count
        # that is not a multiple of that ends with a shorter graph.
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graphs = []      # one step per graph (the page-check comparison below)
        multi = {}       # steps per graph -> graph of that many consecutive steps
        with torch.cuda.stream(cap):
            for k in range(args.rotate):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run(k, st=cap)
                graphs.append(g)
            for n in {args.rotate, args.warmup % args.rotate, args.steps % args.rotate} - {0}:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    for k in range(n):
                        run(k, st=cap)
                multi[n] = g
        stream.wait_stream(cap)

        def replay_steps(n):
            for _ in range(n // args.rotate):
                multi[args.rotate].replay()
            if n % args.rotate:
                multi[n % args.rotate].replay()

        replay_steps(args.warmup)
        torch.cuda.synchronize()
        start.record(stream)
        replay_steps(args.steps)
        end.record(stream)
        torch.cuda.synchronize()
        ms_step_graph = start.elapsed_time(end) / args.steps
        # the step as a caller would launch it: the faster of the two forms,
        # both timed above over the same number of steps
        ms_step = min(ms_step_graph, ms_step_eager)
        if not args.no_page_check:
            def run_checked(i, st, check):
                k = i % args.rotate
                step(q, caches[k], scales[k], w.scale_mode, bt, sl, w.softmax_scale, new_rows=new_rows,
                     stream=st, page_check=check)

            page_check = time_page_check(args, w, mla, torch, np, dev, stream, cap, step, bt, sl,
                                         run_checked, graphs)

    tokens = w.total_tokens()
    unique = w.unique_tokens()
    kv_bytes = unique * w.kv_row_bytes()
    fixed_bytes = (w.B * w.n_q * w.H * 576 * 2          # q
                   + int(sum(-(-int(L) // 64) for L in w.seq_lens)) * 4 + w.B * 4  # page map, lengths
                   + w.B * w.n_q * w.H * (512 * 2 + 4))  # out + lse
    alg_bytes = kv_bytes + fixed_bytes
    flops = 2.0 * w.H * (576 + 512) * sum(
        sum(int(L) - w.n_q + i + 1 for i in range(w.n_q)) for L in w.seq_lens)
    achieved_gbs = alg_bytes / (k_us_burst * 1e-6) / 1e9
    achieved_tflops = flops / (k_us_burst * 1e-6) / 1e12
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    roof = {
        "bound": bound,
        "achieved": round(achieved_gbs if bound == "hbm" else achieved_tflops, 1),
        "peak": HBM_PEAK_GBS if bound == "hbm" else MFMA_BF16_PEAK_TFLOPS,
        "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
        "frac": round((achieved_gbs / HBM_PEAK_GBS) if bound == "hbm"
                      else (achieved_tflops / MFMA_BF16_PEAK_TFLOPS), 4),
        "traffic": load_traffic(w.name),
        "kernel": ("decode_fp8_kernel (mla_decode_paged_append)" if fp8 and new_rows is not None
                   and not args.separate_append else
                   "decode_fp8_kernel (mla_decode_paged)" if fp8 else "decode_bf16_kernel (mla_decode_paged)"),
        "kernel_us": round(k_us_burst, 3),
        "kernel_us_event_pair": round(k_us, 3),
        "algorithmic_bytes": int(alg_bytes),
        "mfma_tflops": round(achieved_tflops, 1),
    }
    value = tokens / (ms_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.B, "heads": w.H, "queries": w.n_q,
            "seq_lens_total": tokens, "unique_tokens": unique, "page": 64,
            "cache": f"{w.cache_dtype}" + (f" ({w.scale_mode} scale)" if fp8 else ""),
            "rotated_caches": args.rotate, "pages_per_split": step.pps, "max_splits": step.max_splits,
        },
        "roofline": roof,
        "hbm_tb_s_step": round(alg_bytes / (ms_step * 1e-3) / 1e12, 3),
        "roofline_frac_step": round(max(t_hbm, t_mfma) / (ms_step * 1e-3), 4),
        "decode_kernel_us_p10_p50_p90": [round(float(np.percentile(k_ms, p)) * 1000, 2) for p in (10, 50, 90)],
        "step_launch": (f"hip graphs of {args.rotate} steps (one per rotated cache)"
                        if ms_step_graph is not None and ms_step_graph <= ms_step_eager else "eager launches"),
        "ms_per_step_graph": None if ms_step_graph is None else round(ms_step_graph, 5),
        "append": ("none (the step's rows are already in the cache)" if w.n_new == 0
                   else "separate kv_append_fp8 launch" if args.separate_append
                   else "in the decode launch (mla_decode_paged_append)" if w.n_new <= 16
                   else "mla_decode_paged_append: its own kv_append launch first (more than 16 rows)"),
        "ms_per_step_eager": round(ms_step_eager, 5),
        "setup_s": round(t_setup, 1),
    }
    if page_check is not None:
        line["page_check"] = page_check
    if not args.no_peaks:
        mp = measured_peaks()
        line["measured_peaks"] = mp
        if bound == "hbm":
            roof["frac_vs_measured_hbm_read"] = round(achieved_gbs / mp["hbm_read_GBs"], 4)
            roof["frac_vs_measured_page_stream"] = round(achieved_gbs / mp["lds_dma_page_stream_GBs"], 4)
        else:
            roof["frac_vs_measured_mfma"] = round(achieved_tflops / mp["mfma_bf16_TFLOPs"], 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_repeats, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
