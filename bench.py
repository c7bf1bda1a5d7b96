#!/usr/bin/env python3
"""KDA prefill throughput on one MI355X, with the roofline of the dominant kernel.

    python bench.py [--steps K] [--warmup W]
                    [--workload packed|single|short|long|decode|decode_tokens]
                    [--conv] [--tokens-mode MODE] [--no-extra] [--no-cpu-baseline]

A step is one kda_chunk_prefill call (intra-chunk kernel + state scan, or the
fused prefill for short sequences) over one 8192-row chunk, with inputs
already resident in HBM.  The default
workload is the packed chunk the metric names: 16 sequences of Dirichlet
lengths in 8192 rows, H=32, d_k=d_v=128, bf16 q/k/v/o, fp32 g/beta, initial
states gathered from a 64-slot fp32 pool by an int32 slot index and final
states scattered back.  Inputs and pools rotate over several device copies so
that the 256 MB last-level cache cannot serve a step from the previous one.
About 150 ms of untimed calls run before the W warmup steps so that clocks
have settled; then exactly K steps are timed between two events.

Prints ONE JSON line.  Besides the throughput it reports:
  roofline      the method's algorithmic bytes per step (q, k, v, g, beta
                read, o written, states read and written) over the dominant
                kernel's time per step (the sum over its launches when a call
                runs as several windows of chunks), against 8 TB/s; the durations come
                from HIP events recorded on the launch stream before, between
                and after the kernels in a second pass of K steps (those
                events cost a few microseconds a step, so the timed steps run
                without them); `traffic` is that kernel's HBM bytes from the
                rocprofv3 FETCH_SIZE / WRITE_SIZE counters per step
                (profiles/traffic.json, reported while the kernel sources
                match), `traffic_ratio` their ratio to the algorithmic bytes,
                and with it `traffic_GBs` and `traffic_frac_of_copy`, the
                counter bytes' rate against the copy ceiling below;
  ceilings      what plain streaming (kda_stream_probe) reaches on this chip
                in the same run: read, copy and in-place update of 512 MiB;
                and the core clocks a bf16 16x16x32 product takes one wave
                with 1, 2 or 8 independent accumulators (kda_mfma_probe);
  path          the whole step against the HBM roof and the bf16 MFMA roof;
  intra_mfma    the intra-chunk contractions' algorithmic flops over the
                intra kernel's time, against the bf16 matrix-core peak;
  cpu_baseline  the fp64 oracle timed on the host cores on the same inputs;
  kernels       the kernels' average durations;
  extra         the other workloads, each with its own roofline and CPU
                baseline: one 8192-row sequence, 128 short sequences in 8192
                rows (the fused prefill), the 262,144-token sequence
                fed as 32 chained 8192-row calls (per call and for all rows),
                the 64-sequence decode step; plus the conv front end and the
                multi-token decode.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "KDA prefill tokens/s on 1 MI355X (8192-row packed chunk) + % MFMA/HBM roof"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources of the two prefill kernels whose HBM traffic profiles/traffic.json
# holds: the stored traffic is reported only while their hash matches
KERNEL_SOURCES = [os.path.join(ROOT, "linear_attention_prefill_amd", "csrc", f)
                  for f in ("kda_prefill.hip", "kda_device.h")]


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def kernel_source_hash() -> str:
    """Hash of the prefill kernels' code, comments and blank lines removed
    (editing a comment leaves the kernels, and their traffic, unchanged)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Algorithmic bytes (what each kernel must move given its inputs and outputs)
# ---------------------------------------------------------------------------

def chunk_count(lengths):
    return int(sum((int(L) + 63) // 64 for L in lengths))


def record_bytes(dk, dv, es):
    """Workspace record of one (chunk, head): w, Q e^Gam, K~^T, A_qk, u in the
    io element size, plus e^{Gam_C} in fp32."""
    return (64 * (3 * dk + dv) + 6 * 512) * es + dk * 4


def intra_bytes(T, H, dk, dv, es, n_chunks):
    reads = T * H * (2 * dk * es + dv * es + dk * 4 + 4)
    writes = n_chunks * H * record_bytes(dk, dv, es)
    return reads + writes


def scan_bytes(T, H, dk, dv, es, n_chunks, n_live, state_in, state_out):
    reads = n_chunks * H * record_bytes(dk, dv, es)
    state = H * dk * dv * 4
    reads += n_live * state if state_in else 0
    writes = T * H * dv * es + (n_live * state if state_out else 0)
    return reads + writes


def path_bytes(T, H, dk, dv, es, n_live, state_in, state_out):
    """The method's own traffic: q, k, v, g, beta in, o out, states in/out."""
    state = H * dk * dv * 4
    return (T * H * (2 * dk * es + dv * es + dk * 4 + 4 + dv * es)
            + (n_live * state if state_in else 0) + (n_live * state if state_out else 0))


def path_flops(lengths, H, dk, dv, intra_only=False):
    """Triangle-aware flops of the chunk form per (chunk, head), summed; with
    intra_only, the intra-chunk contractions alone (A_kk, A_qk, the inverse,
    w and u)."""
    total = 0
    for L in lengths:
        for c0 in range(0, int(L), 64):
            C = min(64, int(L) - c0)
            tri = C * (C + 1) // 2
            f = 2 * tri * dk * 2                 # A_kk, A_qk
            f += 2 * tri * (dk + dv)             # w, u (triangular Tm)
            f += C * C * C // 3                  # inverse (approx.)
            if not intra_only:
                f += 2 * C * dk * dv * 2         # w S, Q~ S
                f += 2 * tri * dv                # A_qk U
                f += 2 * C * dk * dv             # K~^T U
            total += f
    return total * H


# ---------------------------------------------------------------------------

def to_dev(case, copies, torch):
    dt = torch.bfloat16 if case.io_dtype == "bf16" else torch.float32
    base = {
        "q": torch.from_numpy(case.q).to("cuda").to(dt),
        "k": torch.from_numpy(case.k).to("cuda").to(dt),
        "v": torch.from_numpy(case.v).to("cuda").to(dt),
        "g": torch.from_numpy(case.g).to("cuda"),
        "beta": torch.from_numpy(case.beta).to("cuda"),
    }
    sets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(copies - 1)]
    return sets, dt


def prewarm(call, torch, ms=150.0):
    """Untimed calls for about `ms` milliseconds before the warmup steps, so
    that clocks and first-touch costs have settled when timing starts."""
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms and i < 5000:
        call(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_prefill(case, steps, warmup, copies, torch, lap, conv=None):
    """conv: None, or (weight [H,4,C], window pool, activation) for the short
    conv front end; each input copy gets its own window pool."""
    sets, dt = to_dev(case, copies, torch)
    T, H, dk, dv = case.T, case.H, case.d_k, case.d_v
    cu = torch.from_numpy(case.cu_seqlens).to("cuda")
    slots = torch.from_numpy(case.slots).to("cuda") if case.slots is not None else None
    if case.state_pool is not None:
        pools = [torch.from_numpy(case.state_pool).to("cuda") for _ in range(copies)]
        state_in = True
    else:
        pools = [torch.zeros((1, H, dv, dk), dtype=torch.float32, device="cuda")
                 for _ in range(copies)]
        state_in = False
    outs = [torch.empty((T, H, dv), dtype=dt, device="cuda") for _ in range(copies)]
    ws = torch.empty(max(lap.prefill_workspace_size(T, case.N, H, dk, dv, dt, conv=bool(conv)), 16),
                     dtype=torch.uint8, device="cuda")
    ckw = [{} for _ in range(copies)]
    if conv:
        w = torch.from_numpy(conv[0]).to("cuda")
        ckw = [{"conv_weight": w, "conv_window": torch.from_numpy(conv[1]).to("cuda").to(dt),
                "conv_activation": conv[2]} for _ in range(copies)]

    def call(i, events=None):
        s = sets[i % copies]
        p = pools[i % copies]
        lap.chunk_prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], cu,
                          state_in=p if state_in else None, state_out=p, o=outs[i % copies],
                          slots=slots, scale=case.scale, workspace=ws, events=events,
                          **ckw[i % copies])

    prewarm(call, torch)
    for i in range(warmup):
        call(i)
    # the timed steps: plain calls, bracketed by two events
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        call(i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # per-kernel durations: the same steps again with events recorded on the
    # launch stream before the first kernel and after every kernel (intra and
    # scan of each window in turn, then the fused prefill if the call runs
    # it; events between kernels cost a few microseconds a step, so they stay
    # out of the timed steps above)
    nw = lap.prefill_windows(T, case.N, H, dk, dv, dt)
    fused = lap.prefill_fuse_chunks(T, case.N, H, dk, dv, dt) >= 0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nw + 1 + int(fused))]
           for _ in range(steps)]
    for row in evs:           # torch creates the underlying hipEvents on first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(steps):
        call(i, evs[i])
    torch.cuda.synchronize()
    intra = [sum(e[2 * w].elapsed_time(e[2 * w + 1]) for w in range(nw)) for e in evs]
    scan = [sum(e[2 * w + 1].elapsed_time(e[2 * w + 2]) for w in range(nw)) for e in evs]
    fz = [e[2 * nw].elapsed_time(e[2 * nw + 1]) if fused else 0.0 for e in evs]
    return {
        "ms_per_step": total_ms / steps,
        "intra_ms": float(np.mean(intra)), "scan_ms": float(np.mean(scan)),
        "intra_ms_median": float(np.median(intra)), "scan_ms_median": float(np.median(scan)),
        "fused_ms": float(np.mean(fz)), "fused_ms_median": float(np.median(fz)),
        "state_in": state_in, "windows": nw, "fused": fused,
    }


def time_decode(case, steps, warmup, copies, torch, lap, conv=None):
    dt = torch.bfloat16 if case.io_dtype == "bf16" else torch.float32
    q = torch.from_numpy(case.q).to("cuda").to(dt)
    k = torch.from_numpy(case.k).to("cuda").to(dt)
    v = torch.from_numpy(case.v).to("cuda").to(dt)
    g = torch.from_numpy(case.g).to("cuda")
    beta = torch.from_numpy(case.beta).to("cuda")
    slots = torch.from_numpy(case.slots).to("cuda")
    pools = [torch.from_numpy(case.state_pool).to("cuda") for _ in range(copies)]
    o = torch.empty((case.N, case.H, case.d_v), dtype=dt, device="cuda")
    ckw = [{} for _ in range(copies)]
    if conv:
        w = torch.from_numpy(conv[0]).to("cuda")
        ckw = [{"conv_weight": w, "conv_window": torch.from_numpy(conv[1]).to("cuda").to(dt),
                "conv_activation": conv[2]} for _ in range(copies)]
    prewarm(lambda i: lap.decode_step(q, k, v, g, beta, pools[i % copies], slots, o=o,
                                      **ckw[i % copies]), torch)
    for i in range(warmup):
        lap.decode_step(q, k, v, g, beta, pools[i % copies], slots, o=o, **ckw[i % copies])
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        lap.decode_step(q, k, v, g, beta, pools[i % copies], slots, o=o, **ckw[i % copies])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    state = case.H * case.d_k * case.d_v * 4
    es = 2 if case.io_dtype == "bf16" else 4
    nbytes = case.N * (2 * state + case.H * (2 * case.d_k * es + case.d_v * es + case.d_k * 4
                                             + 4 + case.d_v * es))
    if conv:   # windows read and written; the taps, shared by all sequences, read once
        C = 2 * case.d_k + case.d_v
        nbytes += case.N * case.H * C * 2 * 3 * es + case.H * 4 * C * 4
    return {"us": ms * 1e3, "bytes": nbytes, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def time_decode_tokens(case, steps, warmup, copies, torch, lap, only=None):
    """Multi-token decode: fused verify + commit of all tokens, a verify alone
    (state only read) and a commit alone (no outputs); `only` times one."""
    dt = torch.bfloat16
    N, T = case.N, case.meta["tokens"]
    r = lambda x: torch.from_numpy(x.reshape((N, T) + x.shape[1:])).to("cuda")
    q, k, v = r(case.q).to(dt), r(case.k).to(dt), r(case.v).to(dt)
    g, beta = r(case.g), r(case.beta)
    slots = torch.from_numpy(case.slots).to("cuda")
    pools = [torch.from_numpy(case.state_pool).to("cuda") for _ in range(copies)]
    o = torch.empty((N, T, case.H, case.d_v), dtype=dt, device="cuda")
    modes = {"verify_commit": dict(commit=True, outputs=True),
             "verify": dict(commit=False, outputs=True),
             "commit": dict(commit=True, outputs=False)}
    state = case.H * case.d_k * case.d_v * 4
    tok_in = case.H * (2 * case.d_k * 2 + case.d_v * 2 + case.d_k * 4 + 4)
    res = {"tokens": T}
    for name, kw in modes.items():
        if only and name != only:
            continue
        def run(i):
            lap.decode_tokens(q, k, v, g, beta, pools[i % copies], slots,
                              o=o if kw["outputs"] else None, **kw)
        prewarm(run, torch)
        for i in range(warmup):
            run(i)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            run(i)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        nbytes = N * (state * (2 if kw["commit"] else 1)
                      + T * (tok_in - (0 if kw["outputs"] else case.H * case.d_k * 2))
                      + (T * case.H * case.d_v * 2 if kw["outputs"] else 0))
        res[name] = {"us": ms * 1e3, "bytes": nbytes, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                     "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "tokens/s": N * T / (ms * 1e-3)}
    return res


def stream_ceilings(torch, lap, mib=512, grids=(256, 384, 512), reps=10):
    """What plain streaming reaches on this chip (``kda_stream_probe``: 16-byte
    nontemporal grid-stride loops): a read, a copy and an in-place update of
    `mib` MiB, rotating over three buffers so that the 256 MB MALL cannot
    serve a repeat, each the best over `grids` (workgroups of 256 threads;
    the rate varies with the grid by up to 20%, and falls off above 768).
    GB/s of bytes moved (a copy and an update move the buffer twice)."""
    n = mib << 20
    bufs = [torch.ones(n // 4, dtype=torch.float32, device="cuda") for _ in range(3)]
    sink = torch.empty(4 * max(grids), dtype=torch.uint8, device="cuda")
    K = lap.kda
    res = {"buffer_MiB": mib, "grids": list(grids), "kernel": "kda_stream_probe"}
    for name, mode, moved in (("read", K.KDA_STREAM_READ, 1), ("copy", K.KDA_STREAM_COPY, 2),
                              ("update", K.KDA_STREAM_UPDATE, 2)):
        best = (0.0, 0)
        for grid in grids:
            def run(i):
                a, b = bufs[i % 3], bufs[(i + 1) % 3]
                if mode == K.KDA_STREAM_READ:
                    K.stream_probe(mode, a, sink, grid)
                elif mode == K.KDA_STREAM_COPY:
                    K.stream_probe(mode, a, b, grid)
                else:
                    K.stream_probe(mode, None, a, grid)
            for i in range(3):
                run(i)
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for i in range(reps):
                run(i)
            end.record()
            torch.cuda.synchronize()
            gbs = moved * n / (start.elapsed_time(end) / reps * 1e-3) / 1e9
            best = max(best, (gbs, grid))
        res[name + "_GBs"], res[name + "_grid"] = best
    del bufs
    return res


def mfma_rates(lap, iters=4096):
    """Core clocks per bf16 16x16x32 product that one wave a SIMD issues with
    1, 2 and 8 independent accumulators (``kda_mfma_probe``): the dependent
    latency, and the matrix core's throughput, which the published dense
    peak (2.5 PFLOP/s on 256 CUs at 2.4 GHz) puts at 16 clocks."""
    r = {c: lap.kda.mfma_probe(c, iters) for c in (1, 2, 8)}
    return {"kernel": "kda_mfma_probe", "clocks_per_product": {str(c): x["clocks_per_product"]
                                                               for c, x in r.items()},
            "core_MHz": r[8]["core_MHz"]}


def host_cpus():
    """Threads the CPU baseline uses and what they run on: the CPUs this
    process may run on (sched_getaffinity), capped by a cgroup CPU quota when
    one is set (a quota smaller than the affinity mask would only time-slice
    extra threads), and the CPU model."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
            if q != "max":
                quota = max(1, int(int(q) / int(per)))
    except (OSError, ValueError):
        pass
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = aff if quota is None else min(aff, quota)
    return threads, {"affinity_cpus": aff, "cgroup_quota_cpus": quota, "cpu_model": model}


def cpu_baseline(case, seconds, s0=None, label=None):
    """The fp64 oracle on the same inputs, repeated until `seconds` elapse (a
    bounded sample; heads are subsampled if one call would take longer).
    s0: initial states [N, H, d_v, d_k] (the pool rows the call gathers)."""
    from oracle import oracle
    threads, info = host_cpus()
    H = case.H
    # probe one head to size the sample
    t0 = time.perf_counter()
    oracle.recurrence(case.q[:, :1], case.k[:, :1], case.v[:, :1], case.g[:, :1],
                      case.beta[:, :1], case.cu_seqlens,
                      s0=None if s0 is None else s0[:, :1], threads=1)
    per_head = time.perf_counter() - t0
    est_call = per_head * H / min(threads, H * case.N)
    heads = H if est_call <= seconds else max(1, int(H * seconds / est_call))
    sl = slice(0, heads)
    args = (case.q[:, sl], case.k[:, sl], case.v[:, sl], case.g[:, sl], case.beta[:, sl])
    s0s = None if s0 is None else np.ascontiguousarray(s0[:, sl])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrence(*args, case.cu_seqlens, s0=s0s, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    tok_s = case.T * reps * (heads / H) / el
    out = {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "%s: %d of %d heads, %d rows, %d repetition(s) in %.1f s (fp64 "
                     "token-by-token recurrence in C; tokens/s scaled to all heads)"
                     % (label or case.name, heads, H, case.T, reps, el),
           "seconds": el, "tokens_per_s_per_core": tok_s / threads}
    out.update(info)
    return out


def stored_traffic(workload, kernel_name, src_hash):
    """HBM bytes per step of a kernel on a workload (all its launches in the
    step), from the FETCH_SIZE / WRITE_SIZE counters stored in
    profiles/traffic.json, while the kernel sources they were taken at
    match."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != src_hash:
        return None
    w = t.get("workloads", {}).get(workload, {})
    k = w.get("kernels", {}).get(kernel_name)
    # counters are per dispatch; a step launches each kernel once per window
    return None if k is None else k.get("bytes_per_launch") * w.get("windows_per_step", 1)


def prefill_line(case, r, src_hash, conv=False):
    """Throughput, kernels, roofline and path figures of one prefill workload
    from its timings."""
    lengths = np.diff(case.cu_seqlens).tolist()
    T, H, dk, dv = case.T, case.H, case.d_k, case.d_v
    es = 2 if case.io_dtype == "bf16" else 4
    n_live = case.N
    pb = path_bytes(T, H, dk, dv, es, n_live, r["state_in"], True)
    pf = path_flops(lengths, H, dk, dv)
    kern = {
        "kda_intra_kernel": {"us": r["intra_ms"] * 1e3, "us_median": r["intra_ms_median"] * 1e3},
        "kda_scan_kernel": {"us": r["scan_ms"] * 1e3, "us_median": r["scan_ms_median"] * 1e3},
    }
    if r.get("fused"):
        kern["kda_fused_prefill_kernel"] = {"us": r["fused_ms"] * 1e3,
                                            "us_median": r["fused_ms_median"] * 1e3}
    dom = max(kern, key=lambda n: kern[n]["us"])
    t_dom = kern[dom]["us"] * 1e-6
    achieved = pb / t_dom / 1e9
    traffic = None if conv else stored_traffic(case.name, dom, src_hash)
    step_s = r["ms_per_step"] * 1e-3
    line = {
        "workload": case.name + ("+conv3_silu" if conv else ""),
        "value": T / step_s, "unit": "tokens/s", "ms_per_step": r["ms_per_step"],
        "windows": r.get("windows", 1),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_ratio": None if traffic is None else traffic / pb,
                     "kernel": dom, "algorithmic_bytes": pb},
        "kernels": kern,
        "path": {"bytes_per_step": pb, "GB/s": pb / step_s / 1e9,
                 "frac_hbm": pb / step_s / 1e9 / HBM_PEAK_GBS,
                 "flops_per_step": pf,
                 "TFLOP/s": pf / step_s / 1e12,
                 "frac_mfma_bf16": pf / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS},
    }
    if r["intra_ms"] > 0:
        # the intra-chunk contractions against the bf16 matrix-core peak, over
        # the intra kernel's whole time (its loads, stores and VALU work
        # included; profiles/ holds the counter-measured MFMA figures)
        fi = path_flops(lengths, H, dk, dv, intra_only=True)
        ti = r["intra_ms"] * 1e-3
        line["intra_mfma"] = {"kernel": "kda_intra_kernel", "algorithmic_flops": fi,
                              "TFLOP/s": fi / ti / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                              "frac": fi / ti / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    return line


def short_seqs_prefill():
    """128 sequences (Dirichlet lengths, longest 285 rows) in 8192 rows, H = 32,
    d = 128, bf16, states from a 128-slot pool: a call the library runs in the
    fused prefill."""
    from linear_attention_prefill_amd import workloads as W
    return W.packed_varlen_prefill(n=128, num_slots=128)


def time_long_context(steps, warmup, torch, lap, log_fn):
    """The 262,144-token sequence as 32 chained 8192-row calls (state carried
    in a one-slot pool).  A pass is all 32 calls; `steps` passes are timed
    after `warmup` ones.  Each call reads its own rows, so no call finds its
    inputs in the last-level cache."""
    from linear_attention_prefill_amd import workloads as W
    n_calls, L, H, d = W.LONG_CONTEXT_CALLS, 8192, 32, 128
    t0 = time.time()
    calls = [W.long_context_call(c) for c in range(n_calls)]
    log_fn("generated the 32 long-context calls in %.1f s" % (time.time() - t0))
    T = n_calls * L
    Q = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    K, V = torch.empty_like(Q), torch.empty_like(Q)
    G = torch.empty((T, H, d), dtype=torch.float32, device="cuda")
    B = torch.empty((T, H), dtype=torch.float32, device="cuda")
    for c, case in enumerate(calls):
        rows = slice(c * L, (c + 1) * L)
        Q[rows] = torch.from_numpy(case.q).to("cuda").to(torch.bfloat16)
        K[rows] = torch.from_numpy(case.k).to("cuda").to(torch.bfloat16)
        V[rows] = torch.from_numpy(case.v).to("cuda").to(torch.bfloat16)
        G[rows] = torch.from_numpy(case.g).to("cuda")
        B[rows] = torch.from_numpy(case.beta).to("cuda")
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    slot0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = torch.zeros((1, H, d, d), dtype=torch.float32, device="cuda")
    o = torch.empty((L, H, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lap.prefill_workspace_size(L, 1, H, d, d, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")

    def one_pass():
        pool.zero_()
        for c in range(n_calls):
            rows = slice(c * L, (c + 1) * L)
            lap.chunk_prefill(Q[rows], K[rows], V[rows], G[rows], B[rows], cu, state_in=pool,
                              state_out=pool, o=o, slots=slot0, workspace=ws)

    prewarm(lambda i: one_pass(), torch)
    for _ in range(warmup):
        one_pass()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        one_pass()
    end.record()
    torch.cuda.synchronize()
    pass_ms = start.elapsed_time(end) / steps
    return calls, {"pass_ms": pass_ms, "call_ms": pass_ms / n_calls, "rows": T}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["packed", "single", "short", "long", "decode",
                                           "decode_tokens"],
                    default="packed",
                    help="packed: 16 sequences in 8192 rows (default, the metric's chunk); "
                         "single: 1 x 8192 rows; long: 262,144 rows as 32 chained calls; "
                         "decode: 64 sequences x 1 token (profiling the decode kernel); "
                         "decode_tokens: 64 sequences x 4 draft tokens (multi-token decode)")
    ap.add_argument("--copies", type=int, default=3, help="rotated device copies of the inputs")
    ap.add_argument("--conv", action="store_true",
                    help="prefill workloads: run the short conv front end (SiLU) before the path")
    ap.add_argument("--tokens-mode", choices=["verify_commit", "verify", "commit"], default=None,
                    help="decode_tokens workload: time only this mode (default: all three)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU baseline of the headline workload (the extra workloads get a third)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one elementwise copy of this size (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: the KDA path here is built and "
                         "measured on a single MI355X (no multi-GPU sharding); run with --gpus 1.\n")
        sys.exit(2)

    import torch
    import linear_attention_prefill_amd as lap
    from linear_attention_prefill_amd import workloads as W

    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a GPU\n")
        sys.exit(1)
    lap.load_library()
    src_hash = kernel_source_hash()
    extra_cpu_s = args.cpu_seconds / 3

    def decode_line(dc, rd, conv=False):
        line = {"workload": dc.name + ("+conv3_silu" if conv else ""),
                "value": dc.N / (rd["us"] * 1e-6), "unit": "tokens/s",
                "ms_per_step": rd["us"] * 1e-3,
                "roofline": {"bound": "hbm", "achieved": rd["GB/s"], "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": rd["frac_hbm"], "traffic": None,
                             "kernel": "kda_decode_conv_kernel" if conv else "kda_decode_kernel",
                             "algorithmic_bytes": rd["bytes"]}}
        return line

    if args.workload == "decode":
        dc = W.decode_case()
        conv = None
        if args.conv:
            cw = W.draw_conv(12, dc.state_pool.shape[0], dc.H, dc.d_k, dc.d_v, dc.io_dtype)
            conv = (cw[0], cw[1], "silu")
        rd = time_decode(dc, args.steps, args.warmup, 4, torch, lap, conv=conv)
        ln = decode_line(dc, rd, bool(conv))
        out = {"metric": "KDA decode step: state read-modify-write bandwidth on 1 MI355X",
               "value": rd["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": rd["us"] * 1e-3, "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
               "config": {"workload": ln["workload"], "num_seqs": dc.N,
                          "heads": dc.H, "d_k": dc.d_k, "d_v": dc.d_v, "pools_rotated": 4},
               "roofline": ln["roofline"]}
        print(json.dumps(out), flush=True)
        return
    if args.workload == "decode_tokens":
        mc = W.decode_tokens_case()
        rm = time_decode_tokens(mc, args.steps, args.warmup, 4, torch, lap, args.tokens_mode)
        f = rm[args.tokens_mode or "verify_commit"]
        out = {"metric": "KDA multi-token decode (%s): draft tokens per second on 1 MI355X"
                         % (args.tokens_mode or "verify_commit"),
               "value": f["tokens/s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": f["us"] * 1e-3, "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
               "config": {"workload": mc.name, "num_seqs": mc.N, "tokens": rm["tokens"],
                          "heads": mc.H, "d_k": mc.d_k, "d_v": mc.d_v, "pools_rotated": 4},
               "roofline": {"bound": "hbm", "achieved": f["GB/s"], "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": f["frac_hbm"], "traffic": None,
                            "kernel": "kda_decode_tokens_kernel"},
               "modes": rm}
        print(json.dumps(out), flush=True)
        return
    if args.workload == "long":
        calls, rl = time_long_context(args.steps, args.warmup, torch, lap, log)
        out = {"metric": "KDA prefill tokens/s on 1 MI355X, 262,144-token sequence as 32 chained "
                         "8192-row calls",
               "value": rl["rows"] / (rl["pass_ms"] * 1e-3), "unit": "tokens/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": rl["pass_ms"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
               "data": "synthetic",
               "config": {"workload": "long_context_32x8192_H32_d128_bf16", "calls": len(calls)},
               "per_call_ms": rl["call_ms"]}
        print(json.dumps(out), flush=True)
        return

    ceil = stream_ceilings(torch, lap)
    log("streaming ceilings: read %.0f GB/s, copy %.0f GB/s, in-place update %.0f GB/s"
        % (ceil["read_GBs"], ceil["copy_GBs"], ceil["update_GBs"]))
    ceil["mfma_bf16_16x16x32"] = mfma_rates(lap)
    log("bf16 16x16x32 products, one wave a SIMD: %s core clocks each (1, 2, 8 accumulators)"
        % ", ".join("%.1f" % x for x in ceil["mfma_bf16_16x16x32"]["clocks_per_product"].values()))
    t0 = time.time()
    case = {"packed": W.packed_varlen_prefill, "single": W.single_seq_prefill,
            "short": short_seqs_prefill}[args.workload]()
    log("generated %s in %.1f s" % (case.name, time.time() - t0))
    T, H, dk, dv = case.T, case.H, case.d_k, case.d_v

    conv = None
    if args.conv:
        cw = W.draw_conv(11, 1 if case.state_pool is None else case.state_pool.shape[0], H, dk,
                         dv, case.io_dtype)
        conv = (cw[0], cw[1], "silu")
    r = time_prefill(case, args.steps, args.warmup, args.copies, torch, lap, conv=conv)
    log("%s%s: %.1f us/step (intra %.1f us, scan %.1f us)"
        % (case.name, " with conv" if conv else "", r["ms_per_step"] * 1e3, r["intra_ms"] * 1e3,
           r["scan_ms"] * 1e3))
    head = prefill_line(case, r, src_hash, conv=bool(conv))
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "total_rows": T, "num_seqs": case.N,
                   "heads": H, "d_k": dk, "d_v": dv, "chunk": 64, "io_dtype": case.io_dtype,
                   "state": "fp32",
                   "initial_state": "pool-gathered" if r["state_in"] else "zero",
                   "input_copies_rotated": args.copies},
        "roofline": head["roofline"],
        "intra_mfma": head.get("intra_mfma"),
        "kernels": head["kernels"],
        "path": head["path"],
        "ceilings": ceil,
        "kernel_source_hash": src_hash,
    }
    if head["roofline"]["traffic"] is not None:
        # the dominant kernel's counter-measured bytes against the copy ceiling
        t_dom = head["kernels"][head["roofline"]["kernel"]]["us"] * 1e-6
        out["roofline"]["traffic_GBs"] = head["roofline"]["traffic"] / t_dom / 1e9
        out["roofline"]["traffic_frac_of_copy"] = out["roofline"]["traffic_GBs"] / ceil["copy_GBs"]
    slots0 = lambda c: None if c.state_pool is None else c.state_pool[c.slots]
    if not args.no_extra:
        extra = {}
        other = W.single_seq_prefill() if args.workload == "packed" else W.packed_varlen_prefill()
        ro = time_prefill(other, args.steps, args.warmup, args.copies, torch, lap)
        lo = prefill_line(other, ro, src_hash)
        log("%s: %.1f us/step" % (other.name, ro["ms_per_step"] * 1e3))
        if not args.no_cpu_baseline:
            lo["cpu_baseline"] = cpu_baseline(other, extra_cpu_s, s0=slots0(other))
        extra["single" if args.workload == "packed" else "packed"] = lo

        sc = short_seqs_prefill()
        rs = time_prefill(sc, args.steps, args.warmup, args.copies, torch, lap)
        ls = prefill_line(sc, rs, src_hash)
        ls["fuse_chunks"] = lap.prefill_fuse_chunks(sc.T, sc.N, sc.H, sc.d_k, sc.d_v)
        log("%s: %.1f us/step (fused %.1f us)" % (sc.name, rs["ms_per_step"] * 1e3,
                                                  rs["fused_ms"] * 1e3))
        if not args.no_cpu_baseline:
            ls["cpu_baseline"] = cpu_baseline(sc, extra_cpu_s, s0=slots0(sc))
        extra["short_seqs"] = ls

        calls, rl = time_long_context(max(3, args.steps // 4), 1, torch, lap, log)
        ll = {"workload": "long_context_32x8192_H32_d128_bf16",
              "value": rl["rows"] / (rl["pass_ms"] * 1e-3), "unit": "tokens/s",
              "ms_all_rows": rl["pass_ms"], "ms_per_call": rl["call_ms"],
              "per_call_tokens/s": 8192 / (rl["call_ms"] * 1e-3),
              "path": {"bytes_per_call": path_bytes(8192, 32, 128, 128, 2, 1, True, True),
                       "frac_hbm": path_bytes(8192, 32, 128, 128, 2, 1, True, True)
                       / (rl["call_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        log("long context: %.2f ms for 262,144 rows, %.1f us a call"
            % (rl["pass_ms"], rl["call_ms"] * 1e3))
        if not args.no_cpu_baseline:
            c0 = calls[0]
            ll["cpu_baseline"] = cpu_baseline(c0, extra_cpu_s,
                                              label="long-context call 0 (per-row cost is that "
                                                    "of every call)")
        extra["long_context"] = ll
        del calls

        dc = W.decode_case()
        rd = time_decode(dc, max(10, args.steps), 3, 4, torch, lap)
        ld = decode_line(dc, rd)
        log("decode %.1f us, %.0f GB/s" % (rd["us"], rd["GB/s"]))
        if not args.no_cpu_baseline:
            ld["cpu_baseline"] = cpu_baseline(dc, extra_cpu_s, s0=slots0(dc))
        extra["decode"] = ld

        cw = W.draw_conv(11, 1 if case.state_pool is None else case.state_pool.shape[0], H, dk,
                         dv, case.io_dtype)
        rc = time_prefill(case, max(5, args.steps // 2), 2, args.copies, torch, lap,
                          conv=(cw[0], cw[1], "silu"))
        lc = prefill_line(case, rc, src_hash, conv=True)
        lc["conv_us"] = (rc["ms_per_step"] - rc["intra_ms"] - rc["scan_ms"] - rc["fused_ms"]) * 1e3
        extra["prefill_conv"] = lc
        log("%s with conv %.1f us/step (conv front end %.1f us)"
            % (case.name, rc["ms_per_step"] * 1e3, lc["conv_us"]))
        cw = W.draw_conv(12, dc.state_pool.shape[0], dc.H, dc.d_k, dc.d_v, dc.io_dtype)
        rdc = time_decode(dc, max(10, args.steps), 3, 4, torch, lap, conv=(cw[0], cw[1], "silu"))
        extra["decode_conv"] = decode_line(dc, rdc, conv=True)
        log("decode with conv %.1f us, %.0f GB/s" % (rdc["us"], rdc["GB/s"]))
        mc = W.decode_tokens_case()
        rm = time_decode_tokens(mc, max(10, args.steps), 3, 4, torch, lap)
        rm["workload"] = mc.name
        extra["decode_tokens"] = rm
        log("decode_tokens T=%d: verify+commit %.1f us (%.0f GB/s), verify %.1f us, commit %.1f us"
            % (rm["tokens"], rm["verify_commit"]["us"], rm["verify_commit"]["GB/s"],
               rm["verify"]["us"], rm["commit"]["us"]))
        out["extra"] = extra
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        torch.add(x, 1.0, out=y)
        torch.cuda.synchronize()
        out["calibration"] = {"kernel": "torch add (elementwise)", "read_bytes": 4 * n,
                              "write_bytes": 4 * n}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(case, args.cpu_seconds, s0=slots0(case))
        log("cpu baseline %.0f tokens/s on %d threads (%s)" % (cb["value"], cb["cores"],
                                                               cb["cpu_model"]))
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
