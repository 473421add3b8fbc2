"""Requests are independent: decoding a batch as G groups of R / G requests, one decoder
and one stream per group (the schedule bench.py times), selects what one decoder over
the whole batch selects.  Parents and tokens are compared exactly, scores within 1e-6
(the groups may take another code grouping of the log-sum-exp, so the last bits of a
score may differ).
"""
import numpy as np
import pytest
import torch

import synth
from synth import device as sdev
from synth import gen
from linear_attention_beam_amd.decoder import BeamDecoder, prefill
from gpu_harness import say

pytestmark = pytest.mark.gpu


def _decode(wl, G, S_ctx, Wout, inputs, forced):
    dev = S_ctx.device
    Rg = wl.R // G
    decs = [BeamDecoder(Rg, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, wl.io, wl.wout, H_K=wl.H_K)
            for _ in range(G)]
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(G - 1)]
    out = []
    for t in range(wl.T):
        out.append({n: torch.full((wl.R, wl.width(t + 1)), -7, dtype=dt, device=dev) for n, dt in
                    (("parent", torch.int32), ("token", torch.int32), ("score", torch.float32))})
    o = [torch.empty((wl.R, wl.H, wl.width(t), wl.d_v), dtype=torch.float32, device=dev) for t in range(wl.T)]
    for g in range(G):
        decs[g].init(S_ctx[g * Rg:(g + 1) * Rg], wl.width(0), streams[g])
    for t in range(wl.T):
        x = inputs[t]
        for g in range(G):
            q = slice(g * Rg, (g + 1) * Rg)
            decs[g].step(t, x["q"][q], x["k"][q], x["v"][q], x["alpha"][q], x["beta"][q], o[t][q], streams[g])
            fp = forced[t][0][q] if forced[t][0] is not None else None
            ft = forced[t][1][q] if forced[t][1] is not None else None
            decs[g].select(t, o[t][q], Wout, wl.V, wl.width(t + 1), out[t]["parent"][q], out[t]["token"][q],
                           out[t]["score"][q], fp, ft, streams[g])
    torch.cuda.synchronize()
    return [{k: v.cpu().numpy() for k, v in d.items()} for d in out]


@pytest.mark.parametrize("name,G", [("batch", 2), ("batch", 4), ("stress", 2)])
def test_request_groups_select_what_one_decoder_selects(name, G):
    wl = synth.get(name)
    dev = torch.device("cuda")
    p = sdev.prompts(wl, dev)
    S_ctx = torch.empty((wl.R, wl.H, wl.d_v, wl.d_k), dtype=torch.float32, device=dev)
    prefill(S_ctx, p["k"], p["v"], p["alpha"], p["beta"], p["offsets"])
    del p
    Wout = sdev.wout(wl, dev)
    inputs = [sdev.step_inputs(wl, t, dev) for t in range(wl.T)]
    forced = [(None, None)] * wl.T
    if wl.parents == "heavy":
        forced = [(torch.from_numpy(np.stack([gen.forced_parents(wl, r, t) for r in range(wl.R)])).to(dev),
                   torch.from_numpy(np.stack([gen.forced_tokens(wl, r, t) for r in range(wl.R)])).to(dev))
                  for t in range(wl.T)]
    say(f"{name}: one decoder of {wl.R} requests, then {G} groups of {wl.R // G} on {G} streams")
    one = _decode(wl, 1, S_ctx, Wout, inputs, forced)
    grp = _decode(wl, G, S_ctx, Wout, inputs, forced)
    for t in range(wl.T):
        assert np.array_equal(one[t]["parent"], grp[t]["parent"]), t
        assert np.array_equal(one[t]["token"], grp[t]["token"]), t
        a, b = one[t]["score"].astype(np.float64), grp[t]["score"].astype(np.float64)
        assert np.all(np.abs(a - b) <= 1e-6 * np.maximum(1.0, np.abs(a))), t
