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
    """Every beam writes its state; each distinct parent state is read once per head
    (S_ctx once per (request, head) at t = 0)."""
    b = _bench()
    wl = synth.get("batch")
    e = 2
    st = 4 * wl.d_v * wl.d_k
    rng = np.random.default_rng(3)
    for t in range(wl.T):
        W = wl.width(t)
        parents = rng.integers(1, W + 1, size=wl.R) if t else np.zeros(wl.R, np.int64)
        expect = 0
        for r in range(wl.R):
            for _ in range(W):
                expect += wl.H * (st                                   # the new state
                                  + e * (2 * wl.d_k + wl.d_v)          # q, k, v
                                  + 8                                  # alpha, beta
                                  + 4 * wl.d_v)                        # o_t
            if t == 0:
                expect += wl.H * st                                    # S_ctx, once
            else:
                expect += wl.H * st * int(parents[r])                  # each distinct parent once
                expect += 4 * W                                        # parent indices
        assert b.fullstate_bytes(wl, t, parents) == expect
    # siblings share a parent: fewer distinct parents, fewer bytes
    assert b.fullstate_bytes(wl, 1, np.full(wl.R, 10)) < b.fullstate_bytes(wl, 1, np.full(wl.R, 200))


def test_traffic_needs_the_current_sources(monkeypatch):
    """Counter bytes are reported only when the file's hash of the step kernel's sources
    is the current one (else `traffic` is null)."""
    b = _bench()
    f = os.path.join(ROOT, "profiles", "step_kernel_batch_traffic.json")
    d = json.load(open(f))
    monkeypatch.setattr(b, "kernel_hash", lambda dims=None: d["kernel_sha"] if dims == (128, 128) else None)
    assert b.load_traffic("batch") == d["bytes_per_decode"]
    monkeypatch.setattr(b, "kernel_hash", lambda dims=None: "0" * 16)
    assert b.load_traffic("batch") is None
    assert b.load_traffic("no_such_workload") is None


@pytest.mark.parametrize("mode", ["select", "forced"])
def test_cpu_baseline_on_tiny(mode):
    b = _bench()
    args = argparse.Namespace(cpu_seconds=2.0, quiet=True)
    wl = synth.get("tiny")
    res = b.cpu_baseline(args, wl, mode)
    assert res["kind"] == "oracle" and res["unit"] == "beam-transitions/s"
    assert res["value"] > 0 and res["cores"] >= 1
    assert res["requests_sampled"] == 1 and "1 of 1 requests" in res["sample"]
    assert mode in res["sample"]
    assert res["cores_available"] >= 1 and isinstance(res["cpu_model"], str)


def test_default_modes():
    """The heavy fan-out workload runs on its seed-fixed parent maps by default; the
    others let the top-W drive the beams."""
    b = _bench()
    assert b.default_mode(synth.get("stress"), None) == "forced"
    assert b.default_mode(synth.get("batch"), None) == "select"
    assert b.default_mode(synth.get("growing"), None) == "select"
    assert b.default_mode(synth.get("stress"), "select") == "select"


def _write_pmc(d, counter, per_dispatch):
    """A rocprofv3-style counter csv: one row per (dispatch, dimension)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w") as f:
        f.write("Correlation_Id,Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, val) in enumerate(per_dispatch):
            # the value split over two rows of the same dispatch, as per-XCD dimensions are
            f.write(f'{i},{i + 1},"{name}",{counter},{val / 2}\n')
            f.write(f'{i},{i + 1},"{name}",{counter},{val / 2}\n')


def test_traffic_summary_from_counters(tmp_path, monkeypatch):
    """Counter bytes per step launch: FETCH_SIZE and WRITE_SIZE averaged per SID step
    over the step kernel's dispatches, scaled by three device copies of known size."""
    b = _bench()
    copy = [("copy", 0)] * 3
    fetch = [("fill_kernel", 5.0)] + [("copy_kernel", 1000.0)] * 3 + [
        ("void gdn::step_kernel<128, 128, true, 0>(gdn::StepK)", 100.0),
        ("void gdn::logits_kernel<128, true>(gdn::LogitsK)", 7.0),
        ("void gdn::step_kernel<128, 128, true, 1>(gdn::StepK)", 150.0),
        ("void gdn::step_kernel<128, 128, true, 0>(gdn::StepK)", 120.0),
        ("void gdn::step_kernel<128, 128, true, 1>(gdn::StepK)", 170.0)]
    write = [("fill_kernel", 4000.0)] + [("copy_kernel", 4000.0)] * 3 + [(n, 2 * v) for n, v in fetch[4:]]
    del copy
    _write_pmc(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_pmc(str(tmp_path / "w"), "WRITE_SIZE", write)
    bj = tmp_path / "b.json"
    bj.write_text("noise\n" + json.dumps({"roofline": {"bytes_per_launch": [1e6, 2e6]}}) + "\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    args = argparse.Namespace(traffic_from=[str(tmp_path / "f"), str(tmp_path / "w")],
                              bench_json=str(bj), copy_calib=4, workload="wl")
    assert b.traffic_summary(args) == 0
    d = json.load(open(tmp_path / "profiles" / "step_kernel_wl_traffic.json"))
    ff, wf = 4096.0 / 1000.0, 4096.0 / 4000.0
    assert d["fetch_factor"] == pytest.approx(ff) and d["write_factor"] == pytest.approx(wf)
    exp0 = (110.0 * ff + 220.0 * wf) * 1024
    exp1 = (160.0 * ff + 320.0 * wf) * 1024
    assert d["bytes_per_launch"] == [int(exp0), int(exp1)]
    assert d["dispatches_per_t"] == [2, 2]
    assert d["kernel_sha"] == b.kernel_hash()


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
            flops *= 2                                   # z in two fp16 terms
        sel += max(moved / bw, flops / peak)
    assert b.decode_floor_s(wl, bytes_t) == pytest.approx(init + steps + sel, rel=1e-12)


def test_projection_utilisation_on_synthetic_stamps():
    """Per SIMD, MFMA cycles over the union of the phase intervals: two SIMDs, one with two
    overlapping phases, one with two disjoint ones; records never written are ignored."""
    b = _bench()
    def rec(t0, t1, hw, xcc, flops):
        return [t0 & 0xFFFFFFFF, t0 >> 32, t1 & 0xFFFFFFFF, t1 >> 32, hw, xcc, flops, 0]
    f = 1024.0
    r = np.array([
        rec(1000, 1400, 0x10, 0, 200 * 1024),      # SIMD (0, 1): [1000, 1600] after merging
        rec(1200, 1600, 0x13, 0, 300 * 1024),      # same SIMD (wave id in the low bits)
        rec(5000, 5100, 0x20, 1, 50 * 1024),       # SIMD (1, 2): two disjoint phases, 100 + 100
        rec(6000, 6100, 0x20, 1, 50 * 1024),
        [0] * 8,                                   # not written
    ], dtype=np.uint64)
    u = b.projection_utilisation(r, f)
    assert u["simds"] == 2 and u["phases"] == 4
    assert u["util"] == pytest.approx((200 + 300 + 50 + 50) / (600 + 200))
    assert u["mean_phase_cycles"] == pytest.approx((400 + 400 + 100 + 100) / 4)


def test_stamp_records_count():
    b = _bench()
    wl = synth.get("batch")
    assert b.stamp_records(wl, 0) == wl.R * wl.H * 4 * 8          # 4 waves, 8 chunks of 32
    wv = synth.get("wide_v")                                      # d_v = 512: two row blocks of 8 waves
    assert b.stamp_records(wv, 0) == wv.R * wv.H * 2 * 8 * 8


def test_step_kernel_code_hash_matches_the_build():
    """The hashes the build writes are the machine code of the step_kernel instantiations
    in the gfx950 device object, all of them and per head geometry, and bench.py reads
    that file; a workload's traffic file is keyed to its own geometry's hash."""
    import importlib.util as iu
    spec = iu.spec_from_file_location("gdn_build", os.path.join(ROOT, "linear_attention_beam_amd", "build.py"))
    m = iu.module_from_spec(spec)
    spec.loader.exec_module(m)
    dev = os.path.join(ROOT, "linear_attention_beam_amd", "_build", "gdn_step.gfx950.o")
    if not os.path.exists(dev) or not os.path.exists(m.STEP_HASH):
        pytest.skip("the library is not built")
    hs = json.load(open(m.STEP_HASH))
    assert hs == m.step_kernel_hashes(dev)
    assert hs["all"] == m.step_kernel_code_hash(dev) and len(hs["all"]) == 16
    assert {"128x128", "128x256", "256x256", "128x512", "256x512", "16x16"} <= set(hs)
    assert len(set(hs.values())) == len(hs)
    b = _bench()
    assert b.kernel_hash() == hs["all"] and b.kernel_hash((128, 256)) == hs["128x256"]
    syms, _ = m._elf_symbols(open(dev, "rb").read())
    names = [x[0] for x in syms if "step_kernel" in x[0] and x[3] > 0]
    assert any("step_kernelILi128ELi128ELb1ELi3E" in n for n in names)


def test_prefill_bytes_counts_keys_per_key_head():
    """A prefill reads every prompt token's k once per key head (not per value head), its
    v, alpha and beta per value head, and writes one fp32 state per (request, head)."""
    bench = _bench()
    wl = synth.get("grouped")                  # 32 value heads on 16 key heads
    N = 1000
    per_token = (wl.hk * wl.d_k + wl.H * wl.d_v + 2 * wl.H) * 4
    assert bench.prefill_bytes(wl, N) == N * per_token + (wl.R + 1) * 4 + wl.R * wl.H * wl.d_v * wl.d_k * 4
    assert bench.prefill_bytes(wl, 2 * N) - bench.prefill_bytes(wl, N) == N * per_token
