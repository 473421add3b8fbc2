"""GPU-side helpers for the parity tests: drive the C ABI over a synthetic workload
and compare against the CPU oracle.

Requests listed in `exact` get synth.gen's inputs (bit-identical to what the oracle
consumes) and the oracle's fp32 prefill state; the other requests get device-drawn
inputs of the same laws and a short device prefill, and are checked through
properties only.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from synth import device as sdev
from synth import gen
from linear_attention_beam_amd import binding as B
from linear_attention_beam_amd.decoder import BeamDecoder, prefill

# Max per-vector relative inf-norm error of o_t and delta_t.  The bf16-io bar stated for
# the method is 2e-2 (bf16 inputs, fp32 accumulation); these tests hold the path to 1e-4
# in both cases.  With bf16 io the inputs are exact, and the error comes from fp32
# arithmetic and from S_ctx entering the MFMA as two bf16 terms (hi + lo, 16 significant
# bits): about 1e-5 measured.
TOL = {"f32": 1e-4, "bf16": 1e-4}
TOL_STATED = {"f32": 1e-4, "bf16": 2e-2}
NEAR_TIE = 1e-6                       # selection near-tie band, relative to max(1, |theta|)


def say(*a):
    print("[gpu]", *a, file=sys.stderr, flush=True)


def rel_err(got, ref):
    """max over vectors of |got - ref|_inf / |ref|_inf (last axis is the vector)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(num / np.maximum(den, 1e-30)))


def to_np(x: torch.Tensor) -> np.ndarray:
    if x.dtype == torch.bfloat16:
        x = x.float()
    return x.detach().cpu().numpy()


class GpuDecode:
    def __init__(self, wl, R=None, exact=(0,), short_prompt=64, exact_heads=None):
        self.wl = wl
        self.R = wl.R if R is None else R
        self.exact = tuple(r for r in exact if r < self.R)
        dev = torch.device("cuda")
        self.dev = dev
        say(f"workload={wl.name} R={self.R} exact={self.exact} H={wl.H} d_k={wl.d_k} d_v={wl.d_v} "
            f"io={wl.io} T={wl.T} widths={wl.widths} V={wl.V}")
        self.dec = BeamDecoder(self.R, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, wl.io, wl.wout,
                               H_K=wl.H_K)
        # S_ctx: device prefill over short random prompts, exact requests from the oracle
        lengths = [short_prompt] * self.R
        p = sdev.prompts(wl, dev, R=self.R, lengths=lengths)
        self.S_ctx = torch.empty((self.R, wl.H, wl.d_v, wl.d_k), dtype=torch.float32, device=dev)
        say("prefill (device, short prompts)")
        prefill(self.S_ctx, p["k"], p["v"], p["alpha"], p["beta"], p["offsets"])
        self.S_exact = {}
        # exact_heads: only those value heads of the exact requests get the oracle's state
        # (the others keep the device prefill and are not compared)
        hs = list(range(wl.H)) if exact_heads is None else list(exact_heads)
        for r in self.exact:
            S = oracle.prefill_request(wl, r, heads=hs)
            self.S_exact[r] = S
            self.S_ctx[r, hs] = torch.from_numpy(S).to(dev)
        self.Wout = sdev.wout(wl, dev)
        self.Wout64 = gen.wout(wl).value.astype(np.float64)
        self.inputs = []
        for t in range(wl.T):
            x = sdev.step_inputs(wl, t, dev, R=self.R)
            for r in self.exact:
                sdev.upload_request(x, wl, r, t)
            self.inputs.append(x)
        self.o = [torch.empty((self.R, wl.H, wl.width(t), wl.d_v), dtype=torch.float32, device=dev)
                  for t in range(wl.T)]
        self.sel = []
        for t in range(wl.T):
            K = wl.width(t + 1)
            self.sel.append({n: torch.empty((self.R, K), dtype=dt, device=dev) for n, dt in
                             (("parent", torch.int32), ("token", torch.int32), ("score", torch.float32))})
        torch.cuda.synchronize()

    def init(self):
        say(f"gdn_beam_init W0={self.wl.width(0)}")
        self.dec.init(self.S_ctx, self.wl.width(0))

    def step(self, t):
        x = self.inputs[t]
        say(f"gdn_beam_step t={t} W={self.wl.width(t)}")
        self.dec.step(t, x["q"], x["k"], x["v"], x["alpha"], x["beta"], self.o[t])
        torch.cuda.synchronize()
        return self.o[t]

    def forced_maps(self, t):
        fp = np.stack([gen.forced_parents(self.wl, r, t) for r in range(self.R)])
        ft = np.stack([gen.forced_tokens(self.wl, r, t) for r in range(self.R)])
        return fp, ft

    def select(self, t, forced=None):
        s = self.sel[t]
        fpd = ftd = None
        if forced is not None:
            fpd = torch.from_numpy(np.ascontiguousarray(forced[0], np.int32)).to(self.dev)
            ftd = torch.from_numpy(np.ascontiguousarray(forced[1], np.int32)).to(self.dev)
        say(f"gdn_beam_select t={t} V={self.wl.V} W_next={self.wl.width(t + 1)} forced={forced is not None}")
        self.dec.select(t, self.o[t], self.Wout, self.wl.V, self.wl.width(t + 1), s["parent"],
                        s["token"], s["score"], fpd, ftd)
        torch.cuda.synchronize()
        return {k: to_np(v) for k, v in s.items()}

    def export(self, what):
        x = self.dec.export(what)
        torch.cuda.synchronize()
        return to_np(x)

    def step_inputs64(self, r, t):
        return oracle.run.step_arrays(self.wl, r, t)


def check_selection(o_r, cum_r, Wout64, K, sel_r, where=""):
    """GPU top-K against the exact top-K of float64 scores rebuilt from the GPU's own
    o_t and cumulative scores: equal except for candidates within the near-tie band of
    the threshold; scores within the band; canonical order."""
    s = oracle.step_scores(np.asarray(o_r, np.float64), Wout64, np.asarray(cum_r, np.float64))
    V = s.shape[1]
    rp, rt, rs = oracle.top_w(s, K)
    theta = rs[-1]
    band = NEAR_TIE * max(1.0, abs(theta))
    gflat = sel_r["parent"].astype(np.int64) * V + sel_r["token"]
    rflat = rp.astype(np.int64) * V + rt
    assert len(set(gflat.tolist())) == K, f"{where}: duplicate candidates"
    assert np.all((sel_r["parent"] >= 0) & (sel_r["parent"] < s.shape[0])), where
    diff = set(gflat.tolist()) ^ set(rflat.tolist())
    for f in diff:
        assert abs(s.reshape(-1)[f] - theta) <= band, \
            f"{where}: candidate {f} (score {s.reshape(-1)[f]!r}) differs, theta {theta!r}"
    exact = s.reshape(-1)[gflat]
    err = np.abs(sel_r["score"].astype(np.float64) - exact)
    assert np.all(err <= NEAR_TIE * np.maximum(1.0, np.abs(exact))), \
        f"{where}: score error {err.max()} (band {band})"
    sc = sel_r["score"]
    ok = (sc[:-1] > sc[1:]) | ((sc[:-1] == sc[1:]) & (gflat[:-1] < gflat[1:]))
    assert np.all(ok), f"{where}: order is not score-descending / flat-ascending"
    return len(diff)


def xcd_spread(R, n=8):
    """n requests spread over R so that the step kernel's workgroups of the first
    request of every eighth of the grid are among them: requests i R / n + i mod (R / n),
    one in each block of R / 8 consecutive requests, which the XCD-aware block order
    hands to one XCD."""
    if R <= n:
        return tuple(range(R))
    q = R // n
    return tuple(sorted({i * q + (i % q) for i in range(n)}))


def score_perturbation(o_gpu, cum_gpu, o_ref, cum_ref, Wout64):
    """Largest |s_gpu - s_ref| over every candidate of a request, both scored in float64:
    s_gpu from the GPU's o_t and cumulative scores, s_ref from the oracle's."""
    s_gpu = oracle.step_scores(np.asarray(o_gpu, np.float64), Wout64, np.asarray(cum_gpu, np.float64))
    s_ref = oracle.step_scores(np.asarray(o_ref, np.float64), Wout64, np.asarray(cum_ref, np.float64))
    return float(np.max(np.abs(s_gpu - s_ref))), s_ref


def decode_record(name="batch", R=4, time_cap=None):
    """One select-mode decode of workload `name` on its first R requests: every step's
    o_t and selection, then the ancestry, SID prefixes, cumulative scores and record
    pool.  Inputs are seeded, so another process records the same decode.  With
    time_cap, the first time_cap step launches stamp their own start and end
    (gdn_beam_time_steps) and the last entry is (durations, number recorded)."""
    import synth
    wl = synth.get(name)
    g = GpuDecode(wl, R=R, exact=())
    g.init()
    if time_cap is not None:
        g.dec.time_steps(time_cap)
    rec = []
    for t in range(wl.T):
        rec.append(to_np(g.step(t)).copy())
        sel = g.select(t)
        rec += [sel["parent"].copy(), sel["token"].copy(), sel["score"].copy()]
    for what in (B.GDN_EXPORT_ANCESTRY, B.GDN_EXPORT_TOKENS, B.GDN_EXPORT_CUM,
                 B.GDN_EXPORT_GTR_DELTA, B.GDN_EXPORT_GTR_KEY):
        rec.append(g.export(what).copy())
    if time_cap is not None:
        rec.append(g.dec.step_times(wl.T))
        g.dec.time_steps(0)
    return rec


def same_bits(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))
