#!/usr/bin/env python3
"""Throughput of large-beam GDN decoding on one MI355X.

One bench step = one whole decode of a synthetic batch: gdn_beam_init, then for
every SID step t: gdn_beam_step (fused projection + replay + update + record
append) and gdn_beam_select (scoring, exact global top-W, ancestry remap).
value = beam transitions (sum over steps of R*H*W_t) per second of wall time.

The timed decodes run back to back with nothing else on the stream.  A second run
of the same decodes has every step launch record its own start and end (HIP events
stamped by the dispatch, gdn_beam_time_steps); the step kernel's achieved
algorithmic bandwidth over those launches is reported against the 8 TB/s HBM peak.
A third pass times the select calls between HIP events.  The CPU oracle (float64 FullState) is timed on a
bounded sample of the same workload.

    python bench.py [--workload batch|stress|growing|single|tiny] [--steps K] [--warmup W]
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

METRIC = "GDN beam-transitions/sec (R×H×W per SID step) at 1 MI355X; % HBM roofline"
HBM_PEAK_GBS = 8000.0
# the step kernel and everything it includes: counter runs taken on other sources are stale
STEP_SOURCES = [os.path.join(ROOT, "linear_attention_beam_amd", "csrc", f)
                for f in ("gdn_step.hip", "gdn_device.h", "gdn_layout.h")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="batch")
    p.add_argument("--mode", choices=["select", "forced"], default="select")
    p.add_argument("--path", choices=["records", "fullstate"], default="records",
                   help="records: transition records and replay (gdn_beam_step); fullstate: "
                        "the per-beam state baseline (gdn_fullstate_step)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="target CPU oracle time")
    p.add_argument("--quiet", action="store_true")
    p.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                   help="first copy MIB MiB device-to-device 3 times (a plain copy of known size "
                        "for scaling hardware byte counters)")
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


def fullstate_bytes(wl, t):
    """Algorithmic HBM bytes of one gdn_fullstate_step launch at step t: per beam the
    parent's state (4 d_v d_k; at t = 0 the shared S_ctx, once per (request, head)),
    the new state (4 d_v d_k), q, k, v (e each), alpha, beta (8) and o_t (4 d_v); per
    request the parent indices (4 W_t)."""
    e = 2 if wl.io == "bf16" else 4
    W = wl.width(t)
    st = 4 * wl.d_v * wl.d_k
    per_rh = W * (st + e * (2 * wl.d_k + wl.d_v) + 8 + 4 * wl.d_v) + (st if t == 0 else W * st)
    return wl.R * wl.H * per_rh + (4 * W * wl.R if t > 0 else 0)


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
    three times with z split into three bf16 terms for a bf16 codebook (fp32 MFMA
    otherwise), which the selection needs to stay exact at fp32 precision.
    """
    bw = HBM_PEAK_GBS * 1e9
    ew = 2 if wl.wout == "bf16" else 4
    dvp = max(wl.d_v, 32)
    total = wl.R * wl.H * (4 * wl.d_v * wl.d_k + 4 * dvp * wl.d_k) / bw
    for t in range(wl.T):
        W, Wn = wl.width(t), wl.width(t + 1)
        total += bytes_t[t] / bw
        sel_bytes = wl.R * (4 * wl.H * W * wl.d_v + 4 * W + 12 * Wn + 8 * (t + 1) * Wn) + wl.d_v * wl.V * ew
        if wl.wout == "bf16":
            sel_flops, peak = 3 * 2 * wl.R * W * wl.d_v * wl.V, MFMA_BF16_PEAK
        else:
            sel_flops, peak = 2 * wl.R * W * wl.d_v * wl.V, MFMA_F32_PEAK
        total += max(sel_bytes / bw, sel_flops / peak)
    return total


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


def kernel_hash():
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


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
    if d.get("kernel_sha") != kernel_hash():
        return None
    return d.get("bytes_per_decode")


def cpu_baseline(args, wl):
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
            fp, ft = forced[t] if args.mode == "forced" else (None, None)
            dec.select(t, o, Wout, wl.width(t + 1), fp, ft)
        t_tot += time.perf_counter() - t0
        rs += 1
        log(args, f"cpu oracle: {rs} request(s), {t_tot:.1f} s")
        if rs >= wl.R or t_tot >= args.cpu_seconds or t_tot / rs * (rs + 1) > 2 * args.cpu_seconds:
            break
    cpu1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu_s = (cpu1.ru_utime - cpu0.ru_utime) + (cpu1.ru_stime - cpu0.ru_stime)
    trans = rs * wl.H * sum(wl.width(t) for t in range(wl.T))
    threads = max(1, round(cpu_s / max(t_tot, 1e-9)))
    return {"value": trans / t_tot, "unit": "beam-transitions/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rs} of {wl.R} requests (all {wl.H} heads, {wl.T} steps, {args.mode} mode), "
                      f"float64 FullState numpy, {t_tot:.1f} s; host has "
                      f"{len(os.sched_getaffinity(0))} cores available"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): requests are "
              "independent, so the one-GPU rate is one GPU's share of a sharded job.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from synth import device as sdev
    from linear_attention_beam_amd import binding as B
    from linear_attention_beam_amd.decoder import BeamDecoder, prefill

    wl = synth.get(args.workload)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    if args.copy_calib:
        n = args.copy_calib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(args, f"copy calibration: 3 x {args.copy_calib} MiB device-to-device")
        del src, dst
    log(args, f"workload {wl.name}: {wl.summary}")
    copy_gbs = copy_bandwidth(torch, dev)
    log(args, f"device copy (read + write): {copy_gbs:.0f} GB/s")

    # ---- inputs resident in HBM before timing
    dec = BeamDecoder(wl.R, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, wl.io, wl.wout, H_K=wl.H_K)
    p = sdev.prompts(wl, dev)
    S_ctx = torch.empty((wl.R, wl.H, wl.d_v, wl.d_k), dtype=torch.float32, device=dev)
    t0 = time.perf_counter()
    prefill(S_ctx, p["k"], p["v"], p["alpha"], p["beta"], p["offsets"])
    torch.cuda.synchronize()
    log(args, f"prefill of {p['N']} prompt tokens x {wl.H} heads: {time.perf_counter() - t0:.3f} s")
    del p
    Wout = sdev.wout(wl, dev)
    inputs = [sdev.step_inputs(wl, t, dev) for t in range(wl.T)]
    outs = [torch.empty((wl.R, wl.H, wl.width(t), wl.d_v), dtype=torch.float32, device=dev)
            for t in range(wl.T)]
    sels = [{n: torch.empty((wl.R, wl.width(t + 1)), dtype=dt, device=dev) for n, dt in
             (("parent", torch.int32), ("token", torch.int32), ("score", torch.float32))}
            for t in range(wl.T)]
    forced = [(None, None)] * wl.T
    if args.mode == "forced":
        from synth import gen
        forced = [(torch.from_numpy(np.stack([gen.forced_parents(wl, r, t) for r in range(wl.R)])).to(dev),
                   torch.from_numpy(np.stack([gen.forced_tokens(wl, r, t) for r in range(wl.R)])).to(dev))
                  for t in range(wl.T)]
    torch.cuda.synchronize()

    states = dec.alloc_states() if args.path == "fullstate" else None

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

    # ---- distinct ancestor records per step (deterministic: same every decode)
    distinct = []
    dec.init(S_ctx, wl.width(0), stream)
    for t in range(wl.T):
        anc = dec.export(B.GDN_EXPORT_ANCESTRY).cpu().numpy()
        W = wl.width(t)
        d = np.zeros(wl.R, dtype=np.int64)
        if t > 0:
            for r in range(wl.R):
                d[r] = sum(len(np.unique(anc[r, :W, j])) for j in range(t))
        distinct.append(d)
        x = inputs[t]
        gdn_step(t, x)
        s = sels[t]
        dec.select(t, outs[t], Wout, wl.V, wl.width(t + 1), s["parent"], s["token"], s["score"],
                   forced[t][0], forced[t][1], stream)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        decode()
    torch.cuda.synchronize()

    # ---- per-call times: an instrumented pass of the same decodes, HIP events recorded
    # on the launch stream.  Each step(t) is issued rep times back to back between one
    # pair of events (re-issuing step(t) rewrites the same values); select(t) runs once
    # between its pair.  The select and init times come from here; the step times
    # reported come from the timed decodes, except with a flush buffer.
    # With a flush buffer, 1 GiB of it is read or written before every step launch
    # (outside the events), so the launch finds none of its inputs in any cache.
    def instrumented(n, rep, flush_buf=None):
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
                for _ in range(rep):
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
                st[t] += evs[i][t][0].elapsed_time(evs[i][t][1]) / rep
                se[t] += evs[i][t][1].elapsed_time(evs[i][t][2])
        return st / n, se / n, it / n

    trans = wl.transitions()
    if not args.flush_mall:
        # ---- timed region: K whole decodes back to back on the stream, nothing else on
        # it (a timing event between kernels costs the stream a few microseconds, and the
        # idle gap changes what the next launch finds in the caches)
        # it)
        t0 = time.perf_counter()
        for i in range(args.steps):
            decode()
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
        alone_ms, sel_ms, _ = instrumented(n_flow, 1)
        log(args, f"step kernel ms per SID step alone between events: {np.round(alone_ms, 4).tolist()}")
    else:
        # ---- cold caches: K decodes whose every step launch follows a 1 GiB read or
        # write; the decode time is the sum of its event-timed init, step and select
        # intervals
        flush_buf = torch.zeros(256 << 20, dtype=torch.float32, device=dev)
        step_ms, sel_ms, init_ms = instrumented(args.steps, 1, flush_buf)
        elapsed = (init_ms + step_ms.sum() + sel_ms.sum()) * 1e-3 * args.steps
        del flush_buf
    value = trans * args.steps / elapsed
    if states is None:
        bytes_t = [step_bytes(wl, t, distinct[t]) for t in range(wl.T)]
    else:
        bytes_t = [fullstate_bytes(wl, t) for t in range(wl.T)]
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

    res = {
        "metric": METRIC, "value": value, "unit": "beam-transitions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "R": wl.R, "H": wl.H, "d_k": wl.d_k, "d_v": wl.d_v,
                   "T": wl.T, "W_t": list(wl.widths), "V": wl.V, "io_dtype": wl.io,
                   "state_dtype": "f32", "mode": args.mode, "path": args.path,
                   "parallelism": "single GPU", "cache": f"cold ({args.flush_mall} flush)" if args.flush_mall else "pipeline"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gdn step_kernel" if states is None else "gdn fullstate_kernel",
                     "bytes_per_decode": int(sum(bytes_t)),
                     "copy_GBs": copy_gbs,
                     "launches_per_decode": wl.T},
        "gdn_step_rate": gdn_rate,
        "gdn_step_ms": float(step_ms.sum()),
        "step_ms_per_t": [float(x) for x in step_ms],
        "select_ms": float(sel_ms.sum()),
        "step_tflops": flops / (step_ms.sum() * 1e-3) / 1e12,
        "decode_roofline": (None if states is not None else
                            {"floor_ms": decode_floor_s(wl, bytes_t) * 1e3,
                             "frac": decode_floor_s(wl, bytes_t) / (elapsed / args.steps),
                             "basis": "sum over init, step and select launches of max(algorithmic "
                                      "bytes / 8 TB/s, MFMA flops / dense peak)"}),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
