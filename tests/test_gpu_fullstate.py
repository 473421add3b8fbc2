"""GPU parity of the FullState step (gdn_fullstate_step): the baseline semantics of
the OneLA reading note (section 1.3, Fig. 2; eq. 4), every beam with its own state,
against the CPU oracle and against the transition-record step on the same inputs.

Bars as for the record path: o_t within 1e-4 max per-vector relative error for fp32
io, 2e-2 for bf16 io; ancestry and SID prefixes bit-exact under fixed parent maps.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from linear_attention_beam_amd import binding as B
from gpu_harness import GpuDecode, TOL, check_selection, rel_err, say, to_np

pytestmark = pytest.mark.gpu


def _fullstate(g, states, t):
    x = g.inputs[t]
    say(f"gdn_fullstate_step t={t} W={g.wl.width(t)}")
    g.dec.fullstate_step(t, g.S_ctx if t == 0 else None, x["q"], x["k"], x["v"], x["alpha"],
                         x["beta"], g.o[t], states)
    torch.cuda.synchronize()
    return g.o[t]


VARIANTS = {"single_gqa": ("single", dict(H_K=2)),
            "single_dk256": ("single", dict(d_k=256, d_v=256, io="bf16", wout="bf16")),
            "single_dv512": ("single", dict(d_v=512, io="bf16", wout="bf16"))}


@pytest.mark.parametrize("name,R", [("tiny", 1), ("single", 1), ("batch", 2), ("single_gqa", 1),
                                    ("single_dk256", 1), ("single_dv512", 1)])
def test_fullstate_forced_parity(name, R):
    """Fixed parent maps: o_t of every step against the float64 FullState oracle;
    ancestry and SID prefixes bit-exact."""
    if name in VARIANTS:
        base, kw = VARIANTS[name]
        wl = synth.get(base).scaled(name=name, **kw)
    else:
        wl = synth.get(name)
    g = GpuDecode(wl, R=R, exact=range(R))
    tol = TOL[wl.io]
    states = g.dec.alloc_states()
    decs = {r: oracle.FullStateDecoder(g.S_exact[r].astype(np.float64), wl.width(0)) for r in range(R)}
    g.init()
    for t in range(wl.T):
        o = to_np(_fullstate(g, states, t))
        fp, ft = g.forced_maps(t)
        g.select(t, forced=(fp, ft))
        anc = g.export(B.GDN_EXPORT_ANCESTRY)
        tok = g.export(B.GDN_EXPORT_TOKENS)
        K = wl.width(t + 1)
        for r in range(R):
            o_ref, _ = decs[r].step(t, *g.step_inputs64(r, t))
            e = rel_err(o[r], o_ref)
            say(f"r={r} t={t} rel err o={e:.3e}")
            assert e <= tol, e
            decs[r].select(t, o_ref, g.Wout64, K, fp[r], ft[r])
            np.testing.assert_array_equal(anc[r][:K, :t + 1], decs[r].anc)
            np.testing.assert_array_equal(tok[r][:K, :t + 1], decs[r].tokens)


@pytest.mark.parametrize("name,R", [("tiny", 1), ("single", 1)])
def test_fullstate_select_mode(name, R):
    """Top-W drives the FullState beams: the selection is checked against the exact
    top-W of the GPU's own o_t, and the oracle follows the GPU's choice."""
    wl = synth.get(name)
    g = GpuDecode(wl, R=R, exact=range(R))
    tol = TOL[wl.io]
    states = g.dec.alloc_states()
    decs = {r: oracle.FullStateDecoder(g.S_exact[r].astype(np.float64), wl.width(0)) for r in range(R)}
    g.init()
    for t in range(wl.T):
        o = to_np(_fullstate(g, states, t))
        cum_before = g.export(B.GDN_EXPORT_CUM)
        sel = g.select(t)
        K = wl.width(t + 1)
        for r in range(R):
            o_ref, _ = decs[r].step(t, *g.step_inputs64(r, t))
            assert rel_err(o[r], o_ref) <= tol
            sel_r = {k: v[r] for k, v in sel.items()}
            check_selection(o[r], cum_before[r][:wl.width(t)], g.Wout64, K, sel_r, f"r={r} t={t}")
            s_ref = oracle.step_scores(o_ref, g.Wout64, decs[r].cum)
            decs[r].advance(t, sel_r["parent"], sel_r["token"], s_ref[sel_r["parent"], sel_r["token"]])


@pytest.mark.parametrize("name", ["batch", "growing"])
def test_fullstate_matches_record_path(name):
    """Full-size launch: the FullState step and the transition-record step give the
    same o_t on the same inputs and parent maps, every request and head (they are
    two orderings of the same arithmetic; the record path's S_ctx is split into two
    bf16 terms, so they agree to that split's precision, ~1e-5)."""
    wl = synth.get(name)
    if name == "growing":       # two generations of 1024 states per head: keep it small
        wl = wl.scaled(name="growing_r8", R=8)
    g = GpuDecode(wl, exact=())
    states = g.dec.alloc_states()
    outs = {}
    for path in ("records", "full"):
        g.init()
        outs[path] = []
        for t in range(wl.T):
            if path == "records":
                o = g.step(t)
            else:
                o = _fullstate(g, states, t)
            outs[path].append(to_np(o).copy())
            fp, ft = g.forced_maps(t)
            g.select(t, forced=(fp, ft))
    for t in range(wl.T):
        e = rel_err(outs["full"][t], outs["records"][t])
        say(f"t={t} FullState vs records rel err {e:.3e}")
        assert e <= 1e-3, e


def test_fullstate_state_machine():
    wl = synth.get("tiny")
    g = GpuDecode(wl, R=1, exact=(0,))
    states = g.dec.alloc_states()
    nbytes = states.numel() * 4
    x = g.inputs[0]
    stream = torch.cuda.current_stream().cuda_stream

    def full(t, S, buf, size):
        return B.raw_status("gdn_fullstate_step", g.dec.ctx, t, S, x["q"].data_ptr(), x["k"].data_ptr(),
                            x["v"].data_ptr(), x["alpha"].data_ptr(), x["beta"].data_ptr(),
                            g.o[0].data_ptr(), buf, size, stream)

    g.init()
    assert full(0, None, states.data_ptr(), nbytes) == B.GDN_ERR_INVALID_ARG       # no S_ctx at t = 0
    assert full(0, g.S_ctx.data_ptr(), states.data_ptr(), nbytes - 4) == B.GDN_ERR_WORKSPACE
    assert full(1, g.S_ctx.data_ptr(), states.data_ptr(), nbytes) == B.GDN_ERR_BAD_STATE
    assert full(0, g.S_ctx.data_ptr(), states.data_ptr(), nbytes) == B.GDN_OK
    g.select(0)
    other = torch.empty_like(states)
    assert full(1, None, other.data_ptr(), nbytes) == B.GDN_ERR_BAD_STATE           # parents live in `states`
    step = B.raw_status("gdn_beam_step", g.dec.ctx, 1, x["q"].data_ptr(), x["k"].data_ptr(),
                        x["v"].data_ptr(), x["alpha"].data_ptr(), x["beta"].data_ptr(),
                        g.o[0].data_ptr(), stream)
    assert step == B.GDN_ERR_BAD_STATE                                             # no mixing
    g.init()
    g.step(0)
    assert full(0, g.S_ctx.data_ptr(), states.data_ptr(), nbytes) == B.GDN_ERR_BAD_STATE
    torch.cuda.synchronize()


def test_fullstate_timed_launches_same_bits():
    """FullState launches that stamp their own start and end (gdn_beam_time_steps) give
    the same outputs and selections, bit for bit, as untimed ones."""
    wl = synth.get("single")

    def run(timed):
        g = GpuDecode(wl, R=1, exact=())
        states = g.dec.alloc_states()
        g.init()
        if timed:
            g.dec.time_steps(wl.T)
        rec = []
        for t in range(wl.T):
            rec.append(to_np(_fullstate(g, states, t)).copy())
            sel = g.select(t)
            rec += [sel["parent"].copy(), sel["token"].copy(), sel["score"].copy()]
        times = g.dec.step_times(wl.T) if timed else None
        g.dec.time_steps(0)
        return rec, times

    plain, _ = run(False)
    timed, (ms, n) = run(True)
    assert n == wl.T and len(ms) == wl.T and all(m > 0.0 for m in ms), (ms, n)
    for x, y in zip(plain, timed):
        assert np.array_equal(np.ascontiguousarray(x).view(np.uint8), np.ascontiguousarray(y).view(np.uint8))
