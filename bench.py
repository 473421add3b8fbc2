#!/usr/bin/env python3
"""Throughput of large-beam GDN decoding on one MI355X.

One bench step = one whole decode of a synthetic batch: gdn_beam_init, then for
every SID step t: gdn_beam_step (fused projection + replay + update + record
append) and gdn_beam_select (scoring, exact global top-W, ancestry remap).
value = beam transitions (sum over steps of R*H*W_t) per second of wall time.

The headline workload is the large-beam stress decode (R = 64, H = 16, d = 128,
W = 1024, V = 8192, T = 4) with its heavy fan-out parent maps (forced mode: 80% of
the children draw from the top 10% of the parents).  The growing-width decode
(d_v = 256, W 64 -> 1024) and the batch decode (W = 256, V = 1024) run after it in
the same process and are reported under "extra", each in its own default mode.

The timed decodes run back to back with nothing else on the stream.  A second run
of the same decodes has every step launch record its own start and end (HIP events
stamped by the dispatch, gdn_beam_time_steps); the step kernel's achieved
algorithmic bandwidth over those launches is reported against the 8 TB/s HBM peak.
A third pass times the select calls between HIP events.  The CPU oracle (float64
FullState) is timed on a bounded sample of the headline workload.

    python bench.py [--workload stress|growing|batch|...] [--mode forced|select]
                    [--extra growing,batch] [--steps K] [--warmup W]

Counter summaries (host side, after rocprofv3 runs of this script):

    python bench.py --traffic-from FETCH_DIR WRITE_DIR --bench-json FILE --workload NAME
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN beam-transitions/sec (R×H×W per SID step) at 1 MI355X; % HBM roofline"
HBM_PEAK_GBS = 8000.0
# the step kernel's compiled machine code (written by the build): counter runs taken on
# other code are stale
STEP_HASH_FILE = os.path.join(ROOT, "linear_attention_beam_amd", "step_kernel_code.sha")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="stress")
    p.add_argument("--mode", choices=["select", "forced"], default=None,
                   help="forced: the workload's seed-fixed parent maps drive the beams (the "
                        "top-W is still computed); select: the top-W drives them.  Default: "
                        "forced for heavy fan-out parent maps, select otherwise")
    p.add_argument("--extra", default="growing,batch",
                   help="comma-separated workloads run after the headline one and reported "
                        "under 'extra' ('' for none)")
    p.add_argument("--path", choices=["records", "fullstate"], default="records",
                   help="records: transition records and replay (gdn_beam_step); fullstate: "
                        "the per-beam state baseline (gdn_fullstate_step)")
    p.add_argument("--groups", type=int, default=2,
                   help="timed decodes: the requests split into this many equal groups, one "
                        "decoder and one stream each (requests are independent; one group's "
                        "selection overlaps another's step); 1: one decoder on one stream")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="target CPU oracle time")
    p.add_argument("--quiet", action="store_true")
    p.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                   help="first copy MIB MiB device-to-device 3 times (a plain copy of known size "
                        "for scaling hardware byte counters)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                   help="host only: summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) "
                        "of this script into profiles/step_kernel_<workload>_traffic.json")
    p.add_argument("--bench-json", default=None,
                   help="with --traffic-from: the JSON line the profiled run printed")
    p.add_argument("--projection-stamps", action="store_true",
                   help="after the timed decodes, one decode whose step launches stamp every "
                        "projection phase (gdn_beam_stamp_projection): MFMA utilisation of the "
                        "S_ctx projection per SIMD, reported as projection_mfma")
    p.add_argument("--flush-mall", choices=["read", "write"], default=None,
                   help="cold-cache timing: read (or write) 1 GiB of scratch before every step "
                        "launch, so neither L2 nor the 256 MiB last-level cache holds its inputs; "
                        "every launch is timed alone between events, and value counts only the "
                        "event-timed init, step and select work")
    return p.parse_args()


def log(args, *a):
    if not args.quiet:
        print("[bench]", *a, file=sys.stderr, flush=True)


def step_bytes(wl, t, distinct):
    """Algorithmic HBM bytes of one gdn_beam_step launch at step t.

    Per (request, value head): S_ctx once (4 d_v d_k); per beam: v (e d_v), alpha,
    beta (8), the new record's alpha and delta (4 + 4 d_v) and o_t (4 d_v).  Per
    (request, key head) and beam: q, k (e d_k each) and the new record's key (e d_k).
    Per distinct ancestor record referenced: 4 + 4 d_v per value head, e d_k per key
    head.  Per request: t ancestry indices per beam (4 t W_t).  `distinct[r]` =
    distinct (step, slot) records request r's beams reference at step t.
    """
    e = 2 if wl.io == "bf16" else 4
    W = wl.width(t)
    per_rh = 4 * wl.d_v * wl.d_k + W * (e * wl.d_v + 8 + (4 + 4 * wl.d_v) + 4 * wl.d_v)
    per_rk = W * 3 * e * wl.d_k
    total = wl.R * (wl.H * per_rh + wl.hk * per_rk) + 4 * t * W * wl.R
    total += (wl.H * (4 + 4 * wl.d_v) + wl.hk * e * wl.d_k) * int(np.sum(distinct))
    return total


def fullstate_bytes(wl, t, parents=None):
    """Algorithmic HBM bytes of one gdn_fullstate_step launch at step t.

    Per beam: the new state (4 d_v d_k), q, k, v (e each), alpha, beta (8) and o_t
    (4 d_v).  Parent states are read once each: at t = 0 the shared S_ctx once per
    (request, head); at t >= 1 every distinct parent state once per head, where
    `parents[r]` = distinct parents of request r's beams (siblings share their
    parent's state).  Per request at t >= 1: the parent indices (4 W_t).
    """
    e = 2 if wl.io == "bf16" else 4
    W = wl.width(t)
    st = 4 * wl.d_v * wl.d_k
    per_beam = st + e * (2 * wl.d_k + wl.d_v) + 8 + 4 * wl.d_v
    total = wl.R * wl.H * W * per_beam
    if t == 0:
        total += wl.R * wl.H * st
    else:
        n_par = wl.R * W if parents is None else int(np.sum(parents))
        total += wl.H * st * n_par + 4 * W * wl.R
    return total


def step_flops(wl, t):
    W = wl.width(t)
    return wl.R * wl.H * W * (4 * wl.d_v * wl.d_k + t * (4 * wl.d_k + 4 * wl.d_v) + 8 * wl.d_v)


MFMA_BF16_PEAK = 2.5e15                  # dense bf16 MFMA, flop/s
MFMA_F32_PEAK = 157.3e12                 # dense fp32 MFMA, flop/s


def decode_floor_s(wl, bytes_t):
    """Lower bound on one decode: each launch at max(algorithmic bytes / 8 TB/s, its
    MFMA flops / the dense peak of their dtype), summed over init, the T step launches
    and the T selections.

    init: S_ctx read and its fragments written (4 d_v d_k + 4 max(d_v, 32) d_k per
    (request, head)).  step: bytes_t (the step kernel is HBM-bound: its intensity is far
    below the MFMA ridge).  select(t): o_t read (4 H W_t d_v per request), cumulative
    scores, the codebook (once), the top-W outputs (12 W_next) and the new ancestry and
    SID prefixes (8 (t + 1) W_next); flops: the logits W_t x d_v x V, 2 per element,
    twice for a bf16 codebook (z in two fp16 terms against the codebook rescaled into
    fp16, which keeps fp32 precision; fp32 MFMA for an fp32 codebook).
    """
    bw = HBM_PEAK_GBS * 1e9
    dvp = max(wl.d_v, 32)
    total = wl.R * wl.H * (4 * wl.d_v * wl.d_k + 4 * dvp * wl.d_k) / bw
    for t in range(wl.T):
        total += bytes_t[t] / bw + select_floor_s(wl, t)
    return total


def select_floor_s(wl, t):
    """Floor of one select(t) call: max(bytes / 8 TB/s, MFMA flops / dense peak)."""
    bw = HBM_PEAK_GBS * 1e9
    ew = 2 if wl.wout == "bf16" else 4
    W, Wn = wl.width(t), wl.width(t + 1)
    sel_bytes = wl.R * (4 * wl.H * W * wl.d_v + 4 * W + 12 * Wn + 8 * (t + 1) * Wn) + wl.d_v * wl.V * ew
    if wl.wout == "bf16":
        sel_flops, peak = 2 * 2 * wl.R * W * wl.d_v * wl.V, MFMA_BF16_PEAK
    else:
        sel_flops, peak = 2 * wl.R * W * wl.d_v * wl.V, MFMA_F32_PEAK
    return max(sel_bytes / bw, sel_flops / peak)


def copy_bandwidth(torch, dev, mib=1024, reps=10):
    """Read+write GB/s of a plain device-to-device copy: the bandwidth a kernel with
    mixed reads and writes can reach on this GPU (context for the 8 TB/s peak)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def stream_bandwidth(torch, dev, mib=1024, reps=6):
    """GB/s of the library's streaming probe (gdn_beam_stream_probe): a copy (every byte
    read and written) and a read of `mib` MiB with 16-byte non-temporal accesses, and a
    write of `mib` MiB in the fused step's store pattern, four workgroups per compute
    unit; the fastest of `reps` launches after the first."""
    from linear_attention_beam_amd import binding as Bb
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    out = {}
    for mode, name, moved in ((0, "copy", 2 * n), (1, "read", n), (2, "write", n)):
        Bb.gdn_beam_stream_probe(dst, src, n, mode, stream)
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            Bb.gdn_beam_stream_probe(dst, src, n, mode, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        out[name] = moved / (best * 1e-3) / 1e9
    del src, dst
    return out


def kernel_hash(dims=None):
    """sha256[:16] of the built step kernel's machine code: of the instantiations of head
    dims (d_k, d_v) when given, else of all of them (None before a build)."""
    try:
        d = json.load(open(STEP_HASH_FILE))
    except (OSError, ValueError):
        return None
    return d.get("all" if dims is None else f"{dims[0]}x{dims[1]}")


def _dims(wl_name):
    import synth
    try:
        wl = synth.get(wl_name)
    except KeyError:
        return None
    return (wl.d_k, wl.d_v)


def load_traffic(wl_name):
    """HBM bytes of the step kernel per decode (summed over its T launches, like
    bytes_per_decode) from committed rocprofv3 counter runs, if they were taken on the
    current kernel source."""
    f = os.path.join(ROOT, "profiles", f"step_kernel_{wl_name}_traffic.json")
    if not os.path.exists(f):
        return None
    try:
        d = json.load(open(f))
    except Exception:
        return None
    h = kernel_hash(_dims(wl_name))
    if h is None or d.get("kernel_sha") != h:
        return None
    return d.get("bytes_per_decode")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((int(d.get("num_threads", 0)) for d in threadpool_info()
                    if d.get("user_api") == "blas"), default=None)
    except Exception:
        return None


def cpu_baseline(args, wl, mode):
    """Time the float64 FullState oracle on the first requests of the workload."""
    import resource
    import oracle
    from synth import gen

    Wout = gen.wout(wl).value.astype(np.float64)
    # one request first, to size the sample
    rs = 0
    t_tot = 0.0
    cpu0 = resource.getrusage(resource.RUSAGE_SELF)
    while True:
        S = oracle.prefill_request(wl, rs)          # input preparation, not timed
        inputs = [oracle.run.step_arrays(wl, rs, t) for t in range(wl.T)]
        forced = [(gen.forced_parents(wl, rs, t), gen.forced_tokens(wl, rs, t)) for t in range(wl.T)]
        dec = oracle.FullStateDecoder(S.astype(np.float64), wl.width(0))
        t0 = time.perf_counter()
        for t in range(wl.T):
            o, _ = dec.step(t, *inputs[t])
            fp, ft = forced[t] if mode == "forced" else (None, None)
            dec.select(t, o, Wout, wl.width(t + 1), fp, ft)
        t_tot += time.perf_counter() - t0
        del dec, inputs
        rs += 1
        log(args, f"cpu oracle: {rs} request(s), {t_tot:.1f} s")
        if rs >= wl.R or t_tot >= args.cpu_seconds or t_tot / rs * (rs + 1) > 2 * args.cpu_seconds:
            break
    cpu1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu_s = (cpu1.ru_utime - cpu0.ru_utime) + (cpu1.ru_stime - cpu0.ru_stime)
    trans = rs * wl.H * sum(wl.width(t) for t in range(wl.T))
    # busy cores: process CPU time over wall time (the prefill of each sampled request
    # is outside the timed interval and inside the CPU-time window, a small excess)
    threads = max(1, round(cpu_s / max(t_tot, 1e-9)))
    return {"value": trans / t_tot, "unit": "beam-transitions/s", "cores": threads,
            "kind": "oracle", "requests_sampled": rs,
            "cpu_model": _cpu_model(), "blas_threads": _blas_threads(),
            "cores_available": len(os.sched_getaffinity(0)),
            "sample": f"{rs} of {wl.R} requests (all {wl.H} heads, {wl.T} steps, {mode} mode) of the "
                      f"{wl.name} workload, float64 FullState numpy, {t_tot:.1f} s of decode steps; "
                      f"requests are independent, so the rate scales to the whole batch"}


def prefill_bytes(wl, N):
    """Algorithmic HBM bytes of one prefill: the stacked prompts read once (k per key
    head, v, alpha, beta in fp32, the offsets) and S_ctx written once."""
    return (N * (wl.hk * wl.d_k + wl.H * wl.d_v + 2 * wl.H) * 4 + (wl.R + 1) * 4
            + wl.R * wl.H * wl.d_v * wl.d_k * 4)


def measure_prefill(args, wl, p, S_ctx, prefill, B, torch, stream, n=5):
    """Prefill of the workload's stacked prompts (eq. 3 over every prompt token) in both
    forms, each timed between HIP events on the launch stream (mean of n calls after one
    untimed call); S_ctx keeps the chunked form's result."""
    N = p["N"]
    ws = torch.empty(B.gdn_beam_prefill_workspace_bytes(wl.H, wl.d_k, wl.d_v, N), dtype=torch.uint8,
                     device=S_ctx.device)
    args_p = (p["k"], p["v"], p["alpha"], p["beta"], p["offsets"])

    def timed(chunked, reps):
        prefill(S_ctx, *args_p, stream=stream, chunked=chunked, workspace=ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            prefill(S_ctx, *args_p, stream=stream, chunked=chunked, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    token_ms = timed(False, 1)
    ms = timed(True, n)                   # last: S_ctx holds the chunked result
    nbytes = prefill_bytes(wl, N)
    flops = 4.0 * N * wl.H * wl.d_k * wl.d_v          # eq. (3): S k and the rank-1 update
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(args, f"prefill of {N} prompt tokens x {wl.H} heads: chunked {ms:.3f} ms, "
              f"token-sequential {token_ms:.3f} ms; {gbs:.0f} GB/s of algorithmic bytes")
    return {"ms": ms, "ms_token_sequential": token_ms, "tokens": int(N),
            "tokens_per_s": N / (ms * 1e-3), "bytes": int(nbytes), "achieved_GBs": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS, "eq3_TFLOPs": flops / (ms * 1e-3) / 1e12,
            "timing": f"mean of {n} calls between HIP events, workspace allocated beforehand"}


def run_workload(args, wl, mode, torch, copy_gbs):
    """Whole decodes of one workload: returns the measurement dict."""
    import synth  # noqa: F401
    from synth import device as sdev
    from linear_attention_beam_amd import binding as B
    from linear_attention_beam_amd.decoder import BeamDecoder, prefill

    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    log(args, f"workload {wl.name} ({mode} mode): {wl.summary}")

    # ---- inputs resident in HBM before timing
    dec = BeamDecoder(wl.R, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, wl.io, wl.wout, H_K=wl.H_K)
    p = sdev.prompts(wl, dev)
    S_ctx = torch.empty((wl.R, wl.H, wl.d_v, wl.d_k), dtype=torch.float32, device=dev)
    pre = measure_prefill(args, wl, p, S_ctx, prefill, B, torch, stream)
    del p
    Wout = sdev.wout(wl, dev)
    inputs = [sdev.step_inputs(wl, t, dev) for t in range(wl.T)]
    outs = [torch.empty((wl.R, wl.H, wl.width(t), wl.d_v), dtype=torch.float32, device=dev)
            for t in range(wl.T)]
    sels = [{n: torch.empty((wl.R, wl.width(t + 1)), dtype=dt, device=dev) for n, dt in
             (("parent", torch.int32), ("token", torch.int32), ("score", torch.float32))}
            for t in range(wl.T)]
    forced = [(None, None)] * wl.T
    if mode == "forced":
        from synth import gen
        forced = [(torch.from_numpy(np.stack([gen.forced_parents(wl, r, t) for r in range(wl.R)])).to(dev),
                   torch.from_numpy(np.stack([gen.forced_tokens(wl, r, t) for r in range(wl.R)])).to(dev))
                  for t in range(wl.T)]
    torch.cuda.synchronize()

    states = dec.alloc_states() if args.path == "fullstate" else None
    # request groups for the timed decodes (records path): G decoders of R / G requests,
    # each on its own stream (default priority), fed slices of the same input tensors
    G = args.groups if (args.groups > 1 and wl.R % args.groups == 0 and states is None) else 1
    if G != args.groups:
        log(args, f"request groups: 1 ({wl.R} requests, path {args.path})")
    gdecs, gstreams, gsl = [], [], []
    if G > 1:
        Rg = wl.R // G
        gdecs = [BeamDecoder(Rg, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, wl.io, wl.wout, H_K=wl.H_K)
                 for _ in range(G)]
        gstreams = [stream] + [torch.cuda.Stream(device=dev) for _ in range(G - 1)]
        gsl = [slice(g * Rg, (g + 1) * Rg) for g in range(G)]

    def gdn_step(t, x):
        if states is None:
            dec.step(t, x["q"], x["k"], x["v"], x["alpha"], x["beta"], outs[t], stream)
        else:
            dec.fullstate_step(t, S_ctx if t == 0 else None, x["q"], x["k"], x["v"], x["alpha"],
                               x["beta"], outs[t], states, stream)

    def decode():
        dec.init(S_ctx, wl.width(0), stream)
        for t in range(wl.T):
            x = inputs[t]
            gdn_step(t, x)
            s = sels[t]
            dec.select(t, outs[t], Wout, wl.V, wl.width(t + 1), s["parent"], s["token"],
                       s["score"], forced[t][0], forced[t][1], stream)

    def decode_grouped():
        """One decode of every request: the groups' launches interleaved per SID step,
        each group on its own stream (no group waits for another)."""
        for g in range(G):
            gdecs[g].init(S_ctx[gsl[g]], wl.width(0), gstreams[g])
        for t in range(wl.T):
            x, s = inputs[t], sels[t]
            for g in range(G):
                q, st = gsl[g], gstreams[g]
                gdecs[g].step(t, x["q"][q], x["k"][q], x["v"][q], x["alpha"][q], x["beta"][q],
                              outs[t][q], st)
                fp = forced[t][0][q] if forced[t][0] is not None else None
                ft = forced[t][1][q] if forced[t][1] is not None else None
                gdecs[g].select(t, outs[t][q], Wout, wl.V, wl.width(t + 1), s["parent"][q],
                                s["token"][q], s["score"][q], fp, ft, st)

    timed_decode = decode_grouped if G > 1 else decode

    # ---- distinct ancestor records and distinct parents per step (deterministic: the
    # same every decode)
    distinct, parents = [], []
    dec.init(S_ctx, wl.width(0), stream)
    for t in range(wl.T):
        anc = dec.export(B.GDN_EXPORT_ANCESTRY).cpu().numpy()
        W = wl.width(t)
        d = np.zeros(wl.R, dtype=np.int64)
        pa = np.zeros(wl.R, dtype=np.int64)
        if t > 0:
            for r in range(wl.R):
                d[r] = sum(len(np.unique(anc[r, :W, j])) for j in range(t))
                pa[r] = len(np.unique(anc[r, :W, t - 1]))
        distinct.append(d)
        parents.append(pa)
        x = inputs[t]
        gdn_step(t, x)
        s = sels[t]
        dec.select(t, outs[t], Wout, wl.V, wl.width(t + 1), s["parent"], s["token"], s["score"],
                   forced[t][0], forced[t][1], stream)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        decode()
        if G > 1:
            decode_grouped()
    torch.cuda.synchronize()

    # ---- per-call times: an instrumented pass of the same decodes, HIP events recorded
    # on the launch stream around init, every step(t) and every select(t).  The select
    # and init times come from here; the step times reported come from the stamped
    # launches, except with a flush buffer.  With a flush buffer, 1 GiB of it is read or
    # written before every step launch (outside the events), so the launch finds none of
    # its inputs in any cache.
    def instrumented(n, flush_buf=None):
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(wl.T)]
               for _ in range(n)]
        evi = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for i in range(n):
            evi[i][0].record(stream)
            dec.init(S_ctx, wl.width(0), stream)
            evi[i][1].record(stream)
            for t in range(wl.T):
                x = inputs[t]
                if flush_buf is not None:
                    if args.flush_mall == "write":
                        flush_buf.zero_()
                    else:
                        flush_buf.sum()
                evs[i][t][0].record(stream)
                gdn_step(t, x)
                evs[i][t][1].record(stream)
                s = sels[t]
                dec.select(t, outs[t], Wout, wl.V, wl.width(t + 1), s["parent"], s["token"],
                           s["score"], forced[t][0], forced[t][1], stream)
                evs[i][t][2].record(stream)
        torch.cuda.synchronize()
        st, se, it = np.zeros(wl.T), np.zeros(wl.T), 0.0
        for i in range(n):
            it += evi[i][0].elapsed_time(evi[i][1])
            for t in range(wl.T):
                st[t] += evs[i][t][0].elapsed_time(evs[i][t][1])
                se[t] += evs[i][t][1].elapsed_time(evs[i][t][2])
        return st / n, se / n, it / n

    trans = wl.transitions()
    if not args.flush_mall:
        # ---- timed region: K whole decodes back to back, nothing else on the streams
        # (a timing event between kernels costs a stream a few microseconds, and the idle
        # gap changes what the next launch finds in the caches); with request groups,
        # each group's decodes follow each other on its own stream
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            timed_decode()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        # ---- step kernel times: the same decodes back to back again, every step launch
        # stamping its own start and end (the stamps cost the stream a few microseconds
        # per launch, so this pass is not the one `value` comes from)
        n_flow = max(3, min(args.steps, 10))
        dec.time_steps(n_flow * wl.T)
        for i in range(n_flow):
            decode()
        times, n_timed = dec.step_times(n_flow * wl.T)
        dec.time_steps(0)
        assert n_timed == n_flow * wl.T, n_timed
        step_ms = np.asarray(times, dtype=np.float64).reshape(n_flow, wl.T).mean(0)
        alone_ms, sel_ms, _ = instrumented(n_flow)
        log(args, f"step kernel ms per SID step alone between events: {np.round(alone_ms, 4).tolist()}")
    else:
        # ---- cold caches: K decodes whose every step launch follows a 1 GiB read or
        # write; the decode time is the sum of its event-timed init, step and select
        # intervals
        flush_buf = torch.zeros(256 << 20, dtype=torch.float32, device=dev)
        step_ms, sel_ms, init_ms = instrumented(args.steps, flush_buf)
        elapsed = (init_ms + step_ms.sum() + sel_ms.sum()) * 1e-3 * args.steps
        del flush_buf
    value = trans * args.steps / elapsed
    if states is None:
        bytes_t = [step_bytes(wl, t, distinct[t]) for t in range(wl.T)]
    else:
        bytes_t = [fullstate_bytes(wl, t, parents[t]) for t in range(wl.T)]
    achieved = sum(bytes_t) / (step_ms.sum() * 1e-3) / 1e9
    traffic = load_traffic(wl.name) if states is None else None
    gdn_rate = trans / (step_ms.sum() * 1e-3)
    if states is None:
        flops = sum(step_flops(wl, t) for t in range(wl.T))
    else:   # P k and P q, alpha P + delta k^T per state element
        flops = sum(wl.R * wl.H * wl.width(t) * 6 * wl.d_v * wl.d_k for t in range(wl.T))
    where = "each after a 1 GiB flush, between HIP events" if args.flush_mall else "in back-to-back decodes"
    log(args, f"step kernel ms per SID step ({where}): {np.round(step_ms, 4).tolist()}  select ms: "
              f"{np.round(sel_ms, 4).tolist()}")
    log(args, f"algorithmic bytes per step launch: {bytes_t}; distinct ancestors per request "
              f"(mean) {[float(d.mean()) for d in distinct]}")
    ms_decode = elapsed / args.steps * 1e3
    sel_floor = [select_floor_s(wl, t) * 1e3 for t in range(wl.T)]
    res = {
        "value": value, "ms_per_decode": ms_decode, "ms_per_sid_step": ms_decode / wl.T,
        "dtype": wl.io,
        "config": {"workload": wl.name, "R": wl.R, "H": wl.H, "H_K": wl.hk, "d_k": wl.d_k,
                   "d_v": wl.d_v, "T": wl.T, "W_t": list(wl.widths), "V": wl.V, "io_dtype": wl.io,
                   "state_dtype": "f32", "mode": mode,
                   "parents": wl.parents if mode == "forced" else "top-W", "path": args.path,
                   "parallelism": "single GPU",
                   "request_groups": G if not args.flush_mall else 1,
                   "cache": f"cold ({args.flush_mall} flush)" if args.flush_mall else "pipeline"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gdn step_kernel" if states is None else "gdn fullstate_kernel",
                     "scope": "the step kernel's launches only (select excluded; see decode_roofline)",
                     "bytes_per_decode": int(sum(bytes_t)),
                     "bytes_per_launch": [int(b) for b in bytes_t],
                     "copy_GBs": copy_gbs,
                     "launches_per_decode": wl.T},
        "gdn_step_rate": gdn_rate,
        "gdn_step_ms": float(step_ms.sum()),
        "step_ms_per_t": [float(x) for x in step_ms],
        "select_ms": float(sel_ms.sum()),
        "select_ms_per_t": [float(x) for x in sel_ms],
        "select_floor_ms_per_t": sel_floor,
        "prefill": pre,
        "step_tflops": flops / (step_ms.sum() * 1e-3) / 1e12,
        "decode_roofline": (None if states is not None else
                            {"floor_ms": decode_floor_s(wl, bytes_t) * 1e3,
                             "frac": decode_floor_s(wl, bytes_t) / (elapsed / args.steps),
                             "basis": "sum over init, step and select launches of max(algorithmic "
                                      "bytes / 8 TB/s, MFMA flops / dense peak)"}),
    }
    if getattr(args, "projection_stamps", False) and states is None:
        # one more decode, every step launch stamping its projection phases
        from linear_attention_beam_amd import binding as Bb
        per_t = []
        dec.init(S_ctx, wl.width(0), stream)
        for t in range(wl.T):
            n = stamp_records(wl, t)
            buf = torch.zeros(n * 8, dtype=torch.int32, device=dev)
            Bb.gdn_beam_stamp_projection(buf, n * 32)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            gdn_step(t, inputs[t])
            ev1.record(stream)
            s_ = sels[t]
            dec.select(t, outs[t], Wout, wl.V, wl.width(t + 1), s_["parent"], s_["token"], s_["score"],
                       forced[t][0], forced[t][1], stream)
            torch.cuda.synchronize()
            u = projection_utilisation(buf.cpu().numpy().view(np.uint32).reshape(n, 8),
                                       MFMA_FLOPS_PER_SIMD_CYCLE[wl.io])
            u["t"] = t
            u["W"] = wl.width(t)
            u["stamped_launch_ms"] = ev0.elapsed_time(ev1)
            proj_flops = 2 * (2 if wl.io == "bf16" else 1) * 2 * wl.R * wl.H * wl.width(t) * wl.d_v * wl.d_k
            u["projection_share_of_launch"] = (proj_flops / (MFMA_BF16_PEAK if wl.io == "bf16" else MFMA_F32_PEAK)
                                               / (step_ms[t] * 1e-3))
            per_t.append(u)
            log(args, f"projection phases t={t}: MFMA utilisation {u['util']:.3f} over {u['simds']} SIMDs, "
                      f"{u['mean_phase_cycles']:.0f} cycles per phase for {u['mfma_cycles_per_phase']:.0f} "
                      f"MFMA cycles")
        res["projection_mfma"] = {
            "per_t": per_t,
            "method": "in-kernel stamps (gdn_beam_stamp_projection): per SIMD, MFMA cycles of the "
                      "projection phases (flops / dense flops per SIMD cycle) over the union of the "
                      "phases' s_memtime intervals; projection_share_of_launch = executed projection "
                      "MFMA flops / dense peak / the unstamped launch time"}
    dec.close()
    return res


# dense MFMA flops per cycle of one SIMD (published peak / (1024 SIMDs x 2.4 GHz))
MFMA_FLOPS_PER_SIMD_CYCLE = {"bf16": MFMA_BF16_PEAK / (1024 * 2.4e9), "f32": MFMA_F32_PEAK / (1024 * 2.4e9)}


def stamp_records(wl, t):
    """Projection-stamp records of one step launch: work items x waves x chunks."""
    dvp = max(wl.d_v, 32)
    nrb = dvp // 256 if dvp > 256 else 1
    nw = min(dvp, 256) // 32
    return wl.R * wl.H * nrb * nw * ((wl.width(t) + 31) // 32)


def projection_utilisation(rec, flops_per_cycle):
    """MFMA utilisation of the projection phases from stamp records [N, 8] uint32.

    Per SIMD (XCC_ID, and HW_ID bits 4..15: SIMD, CU, shader array, engine), the union of
    its waves' [begin, end] cycle intervals; utilisation = the phases' MFMA cycles (flops /
    flops per SIMD cycle) over that union, summed over SIMDs.  Also the mean phase length
    per chunk and the SIMD count."""
    rec = np.asarray(rec, dtype=np.uint64)
    t0 = rec[:, 0] | (rec[:, 1] << np.uint64(32))
    t1 = rec[:, 2] | (rec[:, 3] << np.uint64(32))
    ok = (t1 > t0) & (rec[:, 6] > 0)
    t0, t1, rec = t0[ok].astype(np.int64), t1[ok].astype(np.int64), rec[ok]
    key = (rec[:, 5].astype(np.int64) << 16) | ((rec[:, 4].astype(np.int64) >> 4) & 0xFFF)
    order = np.lexsort((t0, key))
    t0, t1, key, fl = t0[order], t1[order], key[order], rec[order, 6].astype(np.float64)
    union = 0
    start = np.r_[0, np.flatnonzero(np.diff(key)) + 1, len(key)]
    for a, b in zip(start[:-1], start[1:]):
        cur_s, cur_e = t0[a], t1[a]
        for i in range(a + 1, b):
            if t0[i] > cur_e:
                union += cur_e - cur_s
                cur_s, cur_e = t0[i], t1[i]
            else:
                cur_e = max(cur_e, t1[i])
        union += cur_e - cur_s
    mfma_cycles = float(fl.sum()) / flops_per_cycle
    return {"util": mfma_cycles / max(union, 1), "phases": int(len(t0)), "simds": int(len(start) - 1),
            "mean_phase_cycles": float(np.mean(t1 - t0)) if len(t0) else 0.0,
            "mfma_cycles_per_phase": float(fl.mean() / flops_per_cycle) if len(t0) else 0.0}


def default_mode(wl, asked):
    if asked is not None:
        return asked
    return "forced" if wl.parents == "heavy" else "select"


def main():
    args = parse()
    if args.traffic_from:
        sys.exit(traffic_summary(args))
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): requests are "
              "independent, so the one-GPU rate is one GPU's share of a sharded job.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth

    wl = synth.get(args.workload)
    mode = default_mode(wl, args.mode)
    dev = torch.device("cuda")
    if args.copy_calib:
        n = args.copy_calib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(args, f"copy calibration: 3 x {args.copy_calib} MiB device-to-device")
        del src, dst
    copy_gbs = copy_bandwidth(torch, dev)
    log(args, f"device copy (read + write): {copy_gbs:.0f} GB/s")
    stream_gbs = stream_bandwidth(torch, dev)
    log(args, f"streaming probe: copy {stream_gbs['copy']:.0f} GB/s, read {stream_gbs['read']:.0f} GB/s, "
              f"write {stream_gbs['write']:.0f} GB/s")

    head = run_workload(args, wl, mode, torch, copy_gbs)

    def with_stream(rf):
        # the step kernel's achieved rate against the streaming probe (not the peak)
        rf["stream_copy_GBs"] = stream_gbs["copy"]
        rf["stream_read_GBs"] = stream_gbs["read"]
        rf["stream_write_GBs"] = stream_gbs["write"]
        rf["frac_of_stream_copy"] = rf["achieved"] / stream_gbs["copy"]
        return rf

    with_stream(head["roofline"])
    torch.cuda.empty_cache()
    extra = {}
    for name in [x for x in args.extra.split(",") if x and x != wl.name]:
        ew = synth.get(name)
        r = run_workload(args, ew, default_mode(ew, None), torch, copy_gbs)
        torch.cuda.empty_cache()
        extra[name] = {k: r[k] for k in ("value", "ms_per_decode", "ms_per_sid_step", "gdn_step_ms",
                                         "select_ms_per_t", "select_floor_ms_per_t", "step_ms_per_t",
                                         "gdn_step_rate")}
        extra[name]["config"] = r["config"]
        extra[name]["roofline"] = with_stream({k: r["roofline"][k] for k in ("achieved", "frac", "traffic",
                                                                             "bytes_per_decode")})
        extra[name]["decode_roofline"] = r["decode_roofline"]
        extra[name]["prefill"] = r["prefill"]
        if "projection_mfma" in r:
            extra[name]["projection_mfma"] = r["projection_mfma"]
        log(args, f"extra {name}: {r['value']:.4g} beam-transitions/s, step frac "
                  f"{r['roofline']['frac']:.3f}")

    res = {
        "metric": METRIC, "value": head["value"], "unit": "beam-transitions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        # one bench step is one whole decode (init + T SID steps of step and select)
        "ms_per_step": head["ms_per_decode"], "ms_per_decode": head["ms_per_decode"],
        "ms_per_sid_step": head["ms_per_sid_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"],
        "data": "synthetic (seeded draws of the pages' input laws; no dataset or weights)",
        "config": head["config"],
    }
    for k in ("roofline", "gdn_step_rate", "gdn_step_ms", "step_ms_per_t", "select_ms",
              "select_ms_per_t", "select_floor_ms_per_t", "step_tflops", "decode_roofline",
              "projection_mfma", "prefill"):
        if k in head:
            res[k] = head[k]
    if extra:
        res["extra"] = extra
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, wl, mode)
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------- counter summaries

def read_counters(d):
    """rocprofv3 --pmc csv output under directory d: per dispatch (in dispatch order)
    [kernel name, {counter: value summed over the rows of that dispatch}]."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {d}")
    rows = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                did = int(row.get("Dispatch_Id") or row["Correlation_Id"])
                ent = rows.setdefault(did, [row["Kernel_Name"], {}])
                name = row["Counter_Name"]
                ent[1][name] = ent[1].get(name, 0.0) + float(row["Counter_Value"])
    return [rows[k] for k in sorted(rows)]


def step_t_of(kernel_name):
    """SID step of a step_kernel<DK, DV, BF16, t> dispatch (None for other kernels)."""
    if "step_kernel<" not in kernel_name or "fullstate" in kernel_name:
        return None
    inner = kernel_name.split("step_kernel<", 1)[1].split(">", 1)[0]
    return int(inner.split(",")[-1].strip())


def traffic_summary(args):
    """profiles/step_kernel_<workload>_traffic.json from a FETCH_SIZE and a WRITE_SIZE run
    of this script with --copy-calib MIB (its first three copy dispatches are MIB MiB
    device copies: each reads and writes MIB MiB, which scales the counters to bytes)."""
    fetch_dir, write_dir = args.traffic_from
    fetch, write = read_counters(fetch_dir), read_counters(write_dir)
    if not args.bench_json:
        print("--traffic-from needs --bench-json (the profiled run's JSON line)", file=sys.stderr)
        return 2
    bj = None
    for line in open(args.bench_json):
        line = line.strip()
        if line.startswith("{"):
            bj = json.loads(line)
    alg = bj["roofline"]["bytes_per_launch"]
    if not args.copy_calib:
        print("--traffic-from needs --copy-calib MIB (the size the profiled run copied)", file=sys.stderr)
        return 2
    kib = args.copy_calib * 1024.0
    # the calibration copies: the first three copy dispatches (a fill that allocates the
    # copy's source comes before them)
    fcal = [c["FETCH_SIZE"] for n, c in fetch if "copy" in n.lower()][:3]
    wcal = [c["WRITE_SIZE"] for n, c in write if "copy" in n.lower()][:3]
    if len(fcal) < 3 or len(wcal) < 3:
        print("fewer than three copy dispatches in the counter runs", file=sys.stderr)
        return 2
    ff, wf = kib / np.mean(fcal), kib / np.mean(wcal)
    per_t = {}
    for (name, c) in fetch:
        t = step_t_of(name)
        if t is not None:
            per_t.setdefault(t, [[], []])[0].append(c["FETCH_SIZE"])
    for (name, c) in write:
        t = step_t_of(name)
        if t is not None:
            per_t.setdefault(t, [[], []])[1].append(c["WRITE_SIZE"])
    T = len(alg)
    hbm = []
    rows = []
    for t in range(T):
        fk, wk = float(np.mean(per_t[t][0])), float(np.mean(per_t[t][1]))
        b = (fk * ff + wk * wf) * 1024.0
        hbm.append(int(b))
        rows.append(f"| {t} | {fk:.0f} | {wk:.0f} | {alg[t] / 1e6:.1f} | {b / 1e6:.1f} | {b / alg[t]:.3f} |")
    cfg = bj.get("config", {})
    dims = (cfg["d_k"], cfg["d_v"]) if "d_k" in cfg and "d_v" in cfg else _dims(args.workload)
    out = {"kernel_sha": kernel_hash(dims), "workload": args.workload, "unit": "bytes",
           "bytes_per_launch": hbm, "bytes_per_decode": int(sum(hbm)),
           "algorithmic_per_launch": [int(a) for a in alg],
           "fetch_factor": float(ff), "write_factor": float(wf),
           "dispatches_per_t": [len(per_t[t][0]) for t in range(T)],
           "source": f"profiles/step_kernel_{args.workload}_counters.md"}
    path = os.path.join(ROOT, "profiles", f"step_kernel_{args.workload}_traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"wrote {path}")
    print(f"fetch factor {ff:.4f}, write factor {wf:.4f}")
    print("| t | FETCH_SIZE KiB | WRITE_SIZE KiB | algorithmic MB | HBM MB | ratio |")
    print("|---|---|---|---|---|---|")
    print("\n".join(rows))
    tot_a, tot_b = sum(alg), sum(hbm)
    print(f"| sum | | | {tot_a / 1e6:.1f} | {tot_b / 1e6:.1f} | {tot_b / tot_a:.3f} |")
    return 0


if __name__ == "__main__":
    main()
