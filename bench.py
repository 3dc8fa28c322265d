#!/usr/bin/env python3
"""Benchmark: MLA speculative-verify decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

One step = one decode call of the whole hot path on resident inputs: the main
kernel (mla_decode_run) plus the split-KV merge (mla_decode_reduce).  The plan
is built once per workload beforehand (a host-side prepared plan).  Before
every timed step a 1 GiB buffer is rewritten so the KV is read from HBM, not
from the 256 MB Infinity Cache (cold-cache timing).  Times come from HIP events
recorded on the stream the kernels are launched on: the per-call time from
events around the whole call only; the main-kernel time (roofline) from a
second set of steps with one more event between the two kernels.

Prints ONE JSON line.  The headline workload is fp8-e4m3 KV, bf16 Q, batch 1,
H=12, q=8, ctx=1048576; `value` is its median us per call.  `per_workload`
adds the other workloads and the q-flatness sweep (ctx=1048576, q=1,2,4,8,
bf16 and fp8), each with the GPU clocks the driver reported around its
timing.  `cpu_baseline` times the fp64 oracle on the host cores after all GPU
timing: the headline workload in full (every output row), and each other
workload on a stated sample of rows (`per_config`), plus single-thread runs of
the two smallest workloads.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
METRIC = "µs/call + KV-read HBM GB/s (% roofline), H=12 q=8 ctx=1M bf16/fp8"
HEADLINE = "h12_1m_fp8"
# The pages' own figure for this shape (B300, cute-dsl fold_sq, H=12 q=8 ctx~1M
# fp8, median us/call): context on other hardware, not a baseline of this run.
PAGES_FP8_1M_US_B300 = 168.2
# sources of the headline's main kernel (fp8 KV): their hash ties a counter
# summary to the code it was taken on
KERNEL_SOURCES = [os.path.join(ROOT, "mla_token_decode_amd", "csrc", f)
                  for f in ("fp8_decode.hip", "fp8_agpr.hpp", "device_common.hpp")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "mla_decode_fp8_h12_q8_1m_hbm_traffic.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Profiling runs (--profile) read no clocks: rocm-smi is a script started
# through env, and under a profiler's preloaded library that start would come
# after the GPU is initialised.
READ_CLOCKS = True


def read_clocks():
    """SCLK / MCLK of GPU 0 as the driver reports them right now (rocm-smi,
    best effort: None with the reason when unavailable)."""
    import re
    import subprocess
    if not READ_CLOCKS:
        return {"error": "not read in profiling runs"}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        data = json.loads(r.stdout[r.stdout.index("{"):])
        card = next(iter(data.values()))
        out = {}
        for key, val in card.items():
            m = re.search(r"(\d+)\s*Mhz", str(val), re.I)
            for name in ("sclk", "mclk", "fclk", "socclk"):
                if key.lower().startswith(name) and m:
                    out[name + "_mhz"] = int(m.group(1))
        return out or {"error": "no clock fields in rocm-smi output"}
    except Exception as e:  # noqa: BLE001 -- a missing tool must not stop the bench
        return {"error": f"{type(e).__name__}: {e}"[:200]}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def to_device(inp):
    import torch
    q = torch.from_numpy(np.ascontiguousarray(inp.q_bits).view(np.int16)).view(torch.bfloat16).cuda()
    if inp.kv_fp8:
        kv = torch.from_numpy(np.ascontiguousarray(inp.kv)).cuda()
    else:
        kv = torch.from_numpy(np.ascontiguousarray(inp.kv).view(np.int16)).view(torch.bfloat16).cuda()
    return q, kv


class CacheFlush:
    """Evicts L2 and the Infinity Cache between timed calls by streaming a
    1 GiB buffer through them (more than the 8 x 4 MB L2 plus the 256 MB
    Infinity Cache).  mode "read" sums the buffer into a scalar: the next
    call reads its KV from HBM and finds no dirty lines to write back.
    mode "write" rewrites the buffer instead, so the next call also pays for
    writing back the dirty lines the flush left (up to the cache sizes)."""

    def __init__(self, mode="read"):
        import torch
        self.mode = mode
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        import torch
        if self.mode == "read":
            torch.sum(self.buf, dim=0, out=self.sink)
        else:
            self.buf.add_(1)


def settle(flush, ms):
    """Untimed: keep the GPU busy with cache-flush reads for `ms` milliseconds
    so that its clocks leave any idle state (input generation on the host
    leaves the GPU idle for seconds) before the warm-up calls."""
    import torch
    if ms <= 0:
        return
    t_end = time.perf_counter() + ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            flush()
        torch.cuda.synchronize()


def measure(inp, dev, steps, warmup, flush, paged=None, settle_ms=0, **plan_opts):
    """Cold-cache timing of run + reduce (mla_decode_run, or mla_decode_run_paged
    when `paged` = (pool, page table) is given).  Returns a stats dict
    (microseconds) with the clocks the driver reported before and after."""
    import torch
    from mla_token_decode_amd import binding as mb

    plan = mb.Plan(inp.H, inp.q_len, inp.kv_len, inp.kv_fp8, **plan_opts)
    q, kv = dev
    o, lse, ws = mb.alloc_outputs(plan, q.device)
    stream = torch.cuda.current_stream()

    def run():
        if paged is None:
            mb.mla_decode_run(plan, q, kv, inp.sm_scale, inp.kv_scale, o, lse, ws, ws.numel(), stream)
        else:
            mb.mla_decode_run_paged(plan, q, paged[0], paged[1], inp.sm_scale, inp.kv_scale, o, lse,
                                    ws, ws.numel(), stream)

    def step():
        run()
        mb.mla_decode_reduce(plan, ws, o, lse, stream)

    settle(flush, settle_ms)
    for _ in range(warmup):
        flush()
        step()
    torch.cuda.synchronize()
    clocks_before = read_clocks()
    # the call: events only around run + reduce
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        flush()  # evict L2 / Infinity Cache (untimed: outside the events)
        ev[k][0].record(stream)
        step()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tot = np.array([ev[k][0].elapsed_time(ev[k][1]) for k in range(steps)]) * 1e3
    # breakdown: a middle event splits the main kernel from the merge
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        flush()
        ev[k][0].record(stream)
        run()
        ev[k][1].record(stream)
        mb.mla_decode_reduce(plan, ws, o, lse, stream)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    main = np.array([ev[k][0].elapsed_time(ev[k][1]) for k in range(steps)]) * 1e3
    red = np.array([ev[k][1].elapsed_time(ev[k][2]) for k in range(steps)]) * 1e3
    kv_bytes = inp.kv.nbytes
    med = float(np.median(tot))
    return {
        "us_per_call": med,
        "p10": float(np.percentile(tot, 10)),
        "p90": float(np.percentile(tot, 90)),
        "main_us_mean": float(main.mean()),
        "main_us_median": float(np.median(main)),
        "reduce_us_mean": float(red.mean()),
        "kv_bytes": int(kv_bytes),
        "kv_gbps": kv_bytes / (med * 1e-6) / 1e9,
        "frac_hbm_peak": kv_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        "units": plan.num_units,
        "split_tiles": plan.num_split_tiles,
        "fold_tiles_splits_L": list(plan.query(0)),
        "wall_s": wall,
        "clocks_before": clocks_before,
        "clocks_after": read_clocks(),
        "_calls_us": tot.tolist(),  # per-call samples (kept out of the JSON line)
        "_main_us": main.tolist(),
    }


def kernel_source_sha256():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per main-kernel launch of the headline workload from the
    committed FETCH_SIZE / WRITE_SIZE counter summary (each counter calibrated
    against the 1 GiB read + write reference kernel of the same run).  None when the
    summary is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    try:
        return {"fetch": int(kv["calibrated_fetch_bytes_per_launch"]),
                "write": int(kv["calibrated_write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


def flops(inp):
    """Algorithmic flops: 2 * rows * visible keys * (576 + 512), causal tail exact."""
    total = 0
    H = inp.H
    for qb, nb in zip(inp.q_len, inp.kv_len):
        for i in range(int(qb)):
            total += 2 * H * (int(nb) - int(qb) + i + 1) * (576 + 512)
    return total


def oracle_time(inp, rows_sample, threads=None, seed=123):
    """Wall time of the fp64 oracle on `rows_sample` output rows (all rows when
    the sample covers them), scaled to the whole call.  Returns a dict."""
    import oracle
    total_rows = int(inp.q_len.sum()) * inp.H
    if rows_sample >= total_rows:
        rows = np.arange(total_rows, dtype=np.int64)
    else:
        rng = np.random.default_rng(seed)
        rows = np.sort(rng.choice(total_rows, size=rows_sample, replace=False))
    if threads is not None:
        oracle.set_num_threads(threads)
    try:
        used = oracle.num_threads()
        t0 = time.perf_counter()
        oracle.mla_decode_rows(inp.q_bits, inp.kv, inp.q_len, inp.kv_len, inp.H, rows,
                               kv_is_fp8=inp.kv_fp8, kv_scale=inp.kv_scale, sm_scale=inp.sm_scale)
        dt = time.perf_counter() - t0
    finally:
        if threads is not None:
            oracle.set_num_threads(len(os.sched_getaffinity(0)))
    return {"us_per_call": dt / len(rows) * total_rows * 1e6, "threads": used,
            "rows_timed": int(len(rows)), "rows_total": total_rows, "timed_s": round(dt, 3)}


# Rows of each workload the oracle is timed on (about 10-30 s of host work in
# total at 16 threads): the headline in full; the others sampled.
ORACLE_ROWS = {"h12_1m_fp8": 96, "small": 24, "h12_131k": 96, "h96_125k": 96, "ragged": 320}
ORACLE_ROWS_1T = {"small": 24, "h12_131k": 12}


def cpu_baseline(head_inp, other_inps):
    import oracle
    oracle.set_num_threads(len(os.sched_getaffinity(0)))
    head = oracle_time(head_inp, ORACLE_ROWS[HEADLINE])
    per = {HEADLINE: head}
    for name, inp in other_inps.items():
        per[name] = oracle_time(inp, ORACLE_ROWS.get(name, 96))
        log(f"  oracle {name}: {per[name]}")
        if name in ORACLE_ROWS_1T:
            per[name + "_1thread"] = oracle_time(inp, ORACLE_ROWS_1T[name], threads=1)
            log(f"  oracle {name} (1 thread): {per[name + '_1thread']}")
    return {
        "value": round(head["us_per_call"], 1),
        "unit": "µs/call",
        "cores": head["threads"],
        "kind": "oracle",
        "sample": f"all {head['rows_total']} output rows of the headline workload "
                  f"(fp64, OpenMP over rows, {head['threads']} threads), timed "
                  f"{head['timed_s']:.2f} s; other workloads on the row samples in per_config",
        "cpu_model": cpu_model(),
        "per_config": per,
    }


STREAM_LIB = os.path.join(ROOT, "mla_token_decode_amd", "libmla_stream.so")


def read_ceiling(flush, nbytes, reps=8):
    """Cold read-stream ceiling: the plain streaming read of
    csrc/stream_read.hip (16-byte non-temporal loads, 8 in flight per lane) over
    nbytes of device memory, the caches flushed before every timed launch, HIP
    events around the launch (as for the decode kernels); the median of `reps`
    launches, best over both layouts and 256 .. 8192 workgroups."""
    import ctypes
    import torch
    lib = ctypes.CDLL(STREAM_LIB)
    lib.mla_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p]
    lib.mla_stream_read.restype = ctypes.c_int
    nbytes -= nbytes % 16
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    for layout in (0, 1):
        for blocks in (256, 512, 1024, 2048, 4096, 8192):
            def run():
                rc = lib.mla_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, layout,
                                         stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"mla_stream_read failed ({rc})")
            for _ in range(2):
                flush()
                run()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
            for k in range(reps):
                flush()
                ev[k][0].record(stream)
                run()
                ev[k][1].record(stream)
            torch.cuda.synchronize()
            us = float(np.median([ev[k][0].elapsed_time(ev[k][1]) for k in range(reps)]) * 1e3)
            gbps = nbytes / (us * 1e-6) / 1e9
            if best is None or gbps > best["gbps"]:
                best = {"gbps": gbps, "blocks": blocks, "layout": layout, "us": us, "bytes": nbytes}
    del buf
    return best


def profile_inputs(name):
    """Inputs and device copies of one named workload (profiling runs)."""
    import torch
    from mla_token_decode_amd import inputs as gen
    if name.startswith("flat_"):
        _, kind, q, _ = name.split("_")
        q = int(q[1:])
        if kind == "fp8":
            base = gen.gen_workload_inputs(gen.workload(HEADLINE))
            kv, scale = base.kv, base.kv_scale
        else:
            kv, scale = gen.gen_kv(6, 1048576, False)
        qb = gen.gen_q_bits(6, q, 12)
        inp = gen.Inputs(12, np.array([q], np.int32), np.array([1048576], np.int32), qb, kv,
                         kind == "fp8", scale)
    else:
        inp = gen.gen_workload_inputs(gen.workload(name))
    return inp, to_device(inp)


SCLK_PEAK_MHZ = 2400.0  # MI355X peak engine clock
CLOCK_GATE = 0.70       # a workload counts only if its shader clock stayed above this share of the peak
REPEAT_GATE = 0.02      # largest relative difference between the two headline measurements


def validity_checks(per, head_us, head_repeat_us):
    """The lowest shader clock read around any timed workload against the
    peak, and the headline's second pass (after every other workload)
    against its first: a clock below CLOCK_GATE x peak, or passes more than
    REPEAT_GATE apart, is flagged.  Nothing is dropped: the reported headline
    is the median over the calls of both passes."""
    fracs = {}
    for name, st in per.items():
        if not isinstance(st, dict):
            continue
        mhz = [c.get("sclk_mhz") for c in (st.get("clocks_before"), st.get("clocks_after"))
               if isinstance(c, dict) and isinstance(c.get("sclk_mhz"), (int, float))]
        if mhz:
            fracs[name] = round(min(mhz) / SCLK_PEAK_MHZ, 4)
    out = {"sclk_peak_mhz": SCLK_PEAK_MHZ, "clock_gate": CLOCK_GATE,
           "sclk_min_frac": min(fracs.values()) if fracs else None,
           "clock_gate_passed": (min(fracs.values()) >= CLOCK_GATE) if fracs else None,
           "clock_gate_failed": sorted(k for k, f in fracs.items() if f < CLOCK_GATE),
           "repeat_gate": REPEAT_GATE, "headline_first_pass_us": round(head_us, 2),
           "headline_repeat_us": None, "repeat_disagreement": None,
           "repeat_gate_passed": None}
    if head_repeat_us is not None:
        d = abs(head_repeat_us - head_us) / head_us
        out.update(headline_repeat_us=round(head_repeat_us, 2), repeat_disagreement=round(d, 4),
                   repeat_gate_passed=d <= REPEAT_GATE)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5, help="untimed calls per workload")
    ap.add_argument("--settle-ms", type=int, default=300,
                    help="untimed cache-flush reads before each workload's warm-up, so the "
                         "GPU clocks leave the idle state of the host-side input generation")
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--profile", metavar="WORKLOAD",
                    help="profiling run: the reference kernel, then --steps cold-cache calls "
                         "of one workload (small, h12_131k, h96_125k, h12_1m_fp8, ragged, or "
                         "flat_{fp8,bf16}_q{1,2,4,8}_1m); prints one JSON line")
    args = ap.parse_args()
    if args.profile:
        global READ_CLOCKS
        READ_CLOCKS = False
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the decode of one sequence shard is the single-GPU kernel; see the design notes "
              "for how the path would shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_token_decode_amd import inputs as gen

    torch.cuda.set_device(0)
    flush = CacheFlush("read")
    # one 1 GiB read + 1 GiB write kernel: the known-size reference that the
    # FETCH_SIZE / WRITE_SIZE counter summaries are calibrated against
    flush.buf.add_(1)
    torch.cuda.synchronize()
    meas = dict(steps=args.steps, warmup=args.warmup, flush=flush, settle_ms=args.settle_ms)
    if args.profile:
        inp, dev = profile_inputs(args.profile)
        st = measure(inp, dev, **meas)
        print(json.dumps({"profile": args.profile, "steps": args.steps, "warmup": args.warmup,
                          **{k: (round(v, 3) if isinstance(v, float) else v) for k, v in st.items()}}),
              flush=True)
        return
    log(f"generating {HEADLINE}")
    w = gen.workload(HEADLINE)
    inp = gen.gen_workload_inputs(w)
    dev = to_device(inp)
    settle(flush, args.settle_ms)
    ceiling = read_ceiling(flush, int(inp.kv.nbytes))
    read_stream_gbps = ceiling["gbps"]
    log(f"cold read stream over {ceiling['bytes']} bytes: {read_stream_gbps:.0f} GB/s "
        f"({ceiling['blocks']} workgroups, layout {ceiling['layout']}, {ceiling['us']:.1f} us)")
    log("timing headline")
    head = measure(inp, dev, **meas)
    log(f"  {head}")
    dirty = None
    if not args.quick:
        dirty = measure(inp, dev, args.steps, args.warmup, CacheFlush("write"),
                        settle_ms=args.settle_ms)["us_per_call"]
        log(f"  after a dirtying flush: {dirty:.1f} us")

    per = {HEADLINE: head}
    others = {}
    if not args.quick:
        # the headline workload from a paged cache: 64-key pages in a seeded random order
        page = 64
        npages = w.kv_len[0] // page
        perm = np.random.default_rng(7).permutation(npages)  # pool slot of each logical page
        pool = torch.empty((npages, page, dev[1].shape[1]), dtype=dev[1].dtype, device="cuda")
        pool[torch.from_numpy(perm).cuda()] = dev[1].view(npages, page, -1)
        table = torch.from_numpy(perm.astype(np.int32)).view(1, npages).cuda()
        name = f"paged_{HEADLINE}_p{page}"
        per[name] = measure(inp, dev, paged=(pool, table), **meas)
        log(f"  {name}: {per[name]['us_per_call']:.1f} us")
        del pool, table
        # q-flatness at ctx=1M, both dtypes (same KV per dtype, Q per q)
        kv_fp8 = inp.kv
        for fp8 in (True, False):
            if fp8:
                kv, scale = kv_fp8, inp.kv_scale
            else:
                log("generating bf16 1M KV")
                kv, scale = gen.gen_kv(6, 1048576, False)
            kv_dev = dev[1] if fp8 else torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16).cuda()
            for q in (1, 2, 4, 8):
                qb = gen.gen_q_bits(6, q, 12)
                sub = gen.Inputs(12, np.array([q], np.int32), np.array([1048576], np.int32), qb, kv,
                                 fp8, scale)
                qd = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).cuda()
                name = f"flat_{'fp8' if fp8 else 'bf16'}_q{q}_1m"
                per[name] = measure(sub, (qd, kv_dev), **meas)
                log(f"  {name}: {per[name]['us_per_call']:.1f} us")
            del kv_dev
        for fp8 in ("fp8", "bf16"):
            q1, q8 = per[f"flat_{fp8}_q1_1m"]["us_per_call"], per[f"flat_{fp8}_q8_1m"]["us_per_call"]
            per[f"flat_{fp8}_q8_over_q1"] = round(q8 / q1, 3)
        for name in ("small", "h12_131k", "h96_125k", "ragged"):
            log(f"generating {name}")
            winp = gen.gen_workload_inputs(gen.workload(name))
            wdev = to_device(winp)
            st = measure(winp, wdev, **meas)
            st["tflops"] = flops(winp) / (st["us_per_call"] * 1e-6) / 1e12
            st["frac_bf16_mfma_peak"] = st["tflops"] / BF16_MFMA_PEAK_TFLOPS
            st["main_tflops"] = flops(winp) / (st["main_us_mean"] * 1e-6) / 1e12
            per[name] = st
            log(f"  {name}: {st['us_per_call']:.1f} us")
            others[name] = winp
            del wdev
            torch.cuda.empty_cache()
        # large batches: the sequence descriptors live in workspace tables (GPU timing only)
        for name in ("batch150", "batch150_fp8"):
            winp = gen.gen_workload_inputs(gen.workload(name))
            wdev = to_device(winp)
            per[name] = measure(winp, wdev, **meas)
            log(f"  {name}: {per[name]['us_per_call']:.1f} us")
            del wdev
            torch.cuda.empty_cache()

    # measurement-validity checks: the headline again after every other
    # workload (repeatability), and the shader clock of every workload
    head_repeat = None
    first_pass_us = head["us_per_call"]
    if not args.quick:
        rep_st = measure(inp, dev, **meas)
        head_repeat = rep_st["us_per_call"]
        log(f"  headline again: {head_repeat:.1f} us")
        # the headline figures are those of both passes' calls together
        calls = np.array(head["_calls_us"] + rep_st["_calls_us"])
        mains = np.array(head["_main_us"] + rep_st["_main_us"])
        med = float(np.median(calls))
        head.update(us_per_call=med, p10=float(np.percentile(calls, 10)),
                    p90=float(np.percentile(calls, 90)), main_us_mean=float(mains.mean()),
                    main_us_median=float(np.median(mains)),
                    kv_gbps=head["kv_bytes"] / (med * 1e-6) / 1e9,
                    frac_hbm_peak=head["kv_bytes"] / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                    calls_timed=len(calls))
    validity = validity_checks(per, first_pass_us, head_repeat)
    log(f"  validity: {validity}")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline")
        cpu = cpu_baseline(inp, others)
    traffic = measured_traffic()

    main_us = head["main_us_mean"]
    achieved = head["kv_bytes"] / (main_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(head["us_per_call"], 2),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_call"] / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded N(0,1)*0.1, fp8-e4m3 KV with per-tensor scale)",
        "config": {"workload": HEADLINE, "description": w.description, "batch": 1, "H": 12,
                   "q": 8, "ctx": 1048576, "kv_dtype": "fp8_e4m3", "q_dtype": "bf16",
                   "arithmetic": "QK^T latent part: e4m3 x e4m3 MFMA (Q quantised per row); "
                                 "QK^T rope part: bf16 MFMA; PV: e4m3 P x e4m3 V MFMA; fp32 "
                                 "accumulation, softmax and merge; bf16 split partials",
                   "kv_gbps": round(head["kv_gbps"], 1),
                   "frac_hbm_roofline": round(head["frac_hbm_peak"], 4),
                   "timing": "cold cache (1 GiB read between steps: no KV and no dirty lines "
                             "left in L2 / Infinity Cache), HIP events, median",
                   "settle_ms": args.settle_ms,
                   "clocks": {"before": head["clocks_before"], "after": head["clocks_after"]},
                   "read_stream_gbps": round(read_stream_gbps, 1),
                   "read_stream": "cold plain streaming read of the headline's KV size "
                                  "(csrc/stream_read.hip, non-temporal 16-byte loads), events, "
                                  "median, best of 2 layouts x 6 grid sizes",
                   "frac_of_read_stream": round(head["kv_gbps"] / read_stream_gbps, 4),
                   "context_pages_b300_us": PAGES_FP8_1M_US_B300,
                   "us_per_call_after_dirty_flush": round(dirty, 2) if dirty else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": (traffic["fetch"] + traffic["write"]) if traffic else None,
                     "traffic_unit": "bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
                     "traffic_fetch": traffic["fetch"] if traffic else None,
                     "traffic_write": traffic["write"] if traffic else None,
                     "kernel": "mla_decode_fp8",
                     "algorithmic_bytes": head["kv_bytes"],
                     "kernel_us_mean": round(main_us, 2),
                     "read_ceiling_gbps": round(read_stream_gbps, 1),
                     "frac_of_read_ceiling": round(achieved / read_stream_gbps, 4),
                     "kernel_source_sha256": kernel_source_sha256()},
        "validity": validity,
        "cpu_baseline": cpu,
        "per_workload": {k: ({kk: (round(vv, 4) if isinstance(vv, float) else vv)
                              for kk, vv in v.items() if not kk.startswith("_")}
                             if isinstance(v, dict) else v)
                         for k, v in per.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
