"""Oracle drivers over the synthetic workloads (float64 FullState).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.

Inputs come from synth.gen (the shared seeded generators); values stored in
bf16 by a workload are taken at their bf16 value and upcast to float64.
"""
from __future__ import annotations

import numpy as np

from synth import gen
from .gdn import prefill
from .beam import FullStateDecoder


def prefill_request(wl, r, heads=None):
    """S_ctx of request r: eq. (3) over its prompt in float64, then rounded to fp32.
    heads: the value heads to compute (all by default), in that order."""
    p = gen.prompt_tokens(wl, r)
    # grouped value heads: value head h reads the keys of key head h // group
    k = np.repeat(p["k"].astype(np.float64), wl.group, axis=1)
    v, a, b = p["v"].astype(np.float64), p["alpha"].astype(np.float64), p["beta"].astype(np.float64)
    if heads is not None:
        hs = list(heads)
        k, v, a, b = k[:, hs], v[:, hs], a[:, hs], b[:, hs]
    return prefill(k, v, a, b).astype(np.float32)


def step_arrays(wl, r, t):
    """float64 views of the step-t inputs of request r."""
    x = gen.step_inputs(wl, r, t)
    # grouped value heads: value head h reads q, k of key head h // group
    g = wl.group
    return (np.repeat(x["q"].value.astype(np.float64), g, axis=0),
            np.repeat(x["k"].value.astype(np.float64), g, axis=0),
            x["v"].value.astype(np.float64), x["alpha"].astype(np.float64),
            x["beta"].astype(np.float64))


def decode_request(wl, r, S_ctx, mode="select", Wout=None, keep_scores=False):
    """Decode request r from the fp32 state S_ctx [H, d_v, d_k] over all T steps.

    mode "select": the global top-W drives the beams; "forced": the seed-fixed
    parent/token maps of synth.gen drive them (the top-W is still computed).
    Returns a list with one dict per step.
    """
    if Wout is None:
        Wout = gen.wout(wl).value
    Wout = np.asarray(Wout, dtype=np.float64)
    dec = FullStateDecoder(np.asarray(S_ctx, dtype=np.float64), wl.width(0))
    out = []
    for t in range(wl.T):
        o, delta = dec.step(t, *step_arrays(wl, r, t))
        fp = ft = None
        if mode == "forced":
            fp, ft = gen.forced_parents(wl, r, t), gen.forced_tokens(wl, r, t)
        sel = dec.select(t, o, Wout, wl.width(t + 1), fp, ft)
        rec = {"o": o, "delta": delta, "parent": sel["parent"], "token": sel["token"],
               "top_score": sel["top_score"], "cum": dec.cum.copy(),
               "anc": dec.anc.copy(), "tokens": dec.tokens.copy()}
        if keep_scores:
            rec["score"] = sel["score"]
        out.append(rec)
    return out
