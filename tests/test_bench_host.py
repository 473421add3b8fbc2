"""bench.py's host-side contract, on the CPU: one GPU only, the algorithmic byte
model of the step and FullState launches term by term, hardware counters reported
only when they were taken on the current step-kernel sources, and the oracle leg
(cpu_baseline) on a tiny workload."""
import argparse
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name,H_K", [("batch", None), ("batch", 4), ("growing", None)])
def test_step_bytes_term_by_term(name, H_K):
    """Every byte the step launch must move, summed beam by beam and record by record."""
    b = _bench()
    wl = synth.get(name)
    if H_K:
        wl = wl.scaled(name=f"{name}_hk{H_K}", H_K=H_K)
    e = 2 if wl.io == "bf16" else 4
    rng = np.random.default_rng(7)
    for t in range(wl.T):
        W = wl.width(t)
        distinct = rng.integers(0, t * W + 1, size=wl.R) if t else np.zeros(wl.R, np.int64)
        expect = 0
        for r in range(wl.R):
            expect += wl.H * 4 * wl.d_v * wl.d_k                     # S_ctx, once per (r, h)
            for _ in range(W):
                expect += wl.H * (e * wl.d_v                          # v_t
                                  + 4 + 4                             # alpha_t, beta_t
                                  + 4 + 4 * wl.d_v                    # record: alpha, delta
                                  + 4 * wl.d_v)                       # o_t
                expect += wl.hk * (2 * e * wl.d_k                     # q_t, k_t
                                   + e * wl.d_k)                      # record: key
                expect += 4 * t                                       # ancestry indices
            expect += int(distinct[r]) * (wl.H * (4 + 4 * wl.d_v) + wl.hk * e * wl.d_k)
        assert b.step_bytes(wl, t, distinct) == expect, (name, H_K, t)


def test_fullstate_bytes_term_by_term():
    b = _bench()
    wl = synth.get("batch")
    e = 2
    st = 4 * wl.d_v * wl.d_k
    for t in range(wl.T):
        W = wl.width(t)
        per_beam = st + st + e * (2 * wl.d_k + wl.d_v) + 8 + 4 * wl.d_v   # parent, new, q k v, gates, o
        expect = wl.R * wl.H * W * per_beam
        if t == 0:
            expect += wl.R * wl.H * st - wl.R * wl.H * W * st          # parents: S_ctx once
        else:
            expect += 4 * W * wl.R                                      # parent indices
        assert b.fullstate_bytes(wl, t) == expect


def test_traffic_needs_the_current_sources(monkeypatch):
    """Counter bytes are reported only when the file's hash of the step kernel's sources
    is the current one (else `traffic` is null)."""
    b = _bench()
    f = os.path.join(ROOT, "profiles", "step_kernel_batch_traffic.json")
    d = json.load(open(f))
    monkeypatch.setattr(b, "kernel_hash", lambda: d["kernel_sha"])
    assert b.load_traffic("batch") == d["bytes_per_decode"]
    monkeypatch.setattr(b, "kernel_hash", lambda: "0" * 16)
    assert b.load_traffic("batch") is None
    assert b.load_traffic("no_such_workload") is None


def test_cpu_baseline_on_tiny():
    b = _bench()
    args = argparse.Namespace(mode="select", cpu_seconds=2.0, quiet=True)
    wl = synth.get("tiny")
    res = b.cpu_baseline(args, wl)
    assert res["kind"] == "oracle" and res["unit"] == "beam-transitions/s"
    assert res["value"] > 0 and res["cores"] >= 1
    assert "1 of 1 requests" in res["sample"]


@pytest.mark.parametrize("name", ["batch", "tiny", "growing"])
def test_decode_floor_term_by_term(name):
    """The full-decode floor: init, every step launch and every selection, each at the
    larger of its bytes over 8 TB/s and its MFMA flops over the dense peak."""
    b = _bench()
    wl = synth.get(name)
    bytes_t = [b.step_bytes(wl, t, np.zeros(wl.R, np.int64)) for t in range(wl.T)]
    bw = 8000e9
    ew = 2 if wl.wout == "bf16" else 4
    init = wl.R * wl.H * (4 * wl.d_v * wl.d_k + 4 * max(wl.d_v, 32) * wl.d_k) / bw
    steps = sum(bytes_t) / bw
    sel = 0.0
    for t in range(wl.T):
        W, Wn = wl.width(t), wl.width(t + 1)
        moved = (wl.R * wl.H * W * wl.d_v * 4           # o_t
                 + wl.R * W * 4                          # cumulative scores
                 + wl.d_v * wl.V * ew                    # codebook
                 + wl.R * Wn * (4 + 4 + 4)               # parent, token, score
                 + wl.R * Wn * (t + 1) * (4 + 4))        # ancestry, SID prefixes
        flops = 2 * wl.R * W * wl.d_v * wl.V
        peak = 2.5e15 if wl.wout == "bf16" else 157.3e12
        if wl.wout == "bf16":
            flops *= 3
        sel += max(moved / bw, flops / peak)
    assert b.decode_floor_s(wl, bytes_t) == pytest.approx(init + steps + sel, rel=1e-12)
