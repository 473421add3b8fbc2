"""Pins of the oracle's beam bookkeeping and head grouping (no GPU).

Three parts of the oracle that the GDN pins do not reach:
  * the SID prefix each beam carries (eq. (1) of the OneLA reading note,
    section 1.1: a candidate is a token sequence s^1 .. s^t built one step at a
    time, each child extending its parent's prefix by one token);
  * the cumulative score each beam carries, in select and in forced mode (the log
    of eq. (1)'s product: the sum over the steps of the chosen token's
    log-softmax);
  * grouped value heads (the operator sweep of the reading note, section 3, has
    head geometries with fewer key heads than value heads): value head h reads
    the q, k of key head h // (H / H_K).

Each is checked against a reconstruction written only here, that shares nothing
with the oracle but the seeded inputs: prefixes and scores by walking the parent
pointers back from each final beam and re-running eq. (3) (section 1.2) token by
token along that chain, scores by scipy's log_softmax; head grouping by an
explicit loop over value heads.
"""
import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax

import synth
from synth import gen
from oracle import FullStateDecoder, prefill_request
from oracle.run import step_arrays


def _wl(name, **kw):
    return synth.get(name).scaled(name=f"{name}_pin", **kw)


def _run(wl, mode, r=0):
    """Oracle decode of request r; returns the decoder and the per-step (parent,
    token) maps the beams actually followed."""
    S = prefill_request(wl, r).astype(np.float64)
    Wout = gen.wout(wl).value.astype(np.float64)
    dec = FullStateDecoder(S, wl.width(0))
    followed = []
    for t in range(wl.T):
        o, _ = dec.step(t, *step_arrays(wl, r, t))
        if mode == "forced":
            fp, ft = gen.forced_parents(wl, r, t), gen.forced_tokens(wl, r, t)
            dec.select(t, o, Wout, wl.width(t + 1), fp, ft)
            followed.append((np.asarray(fp), np.asarray(ft)))
        else:
            sel = dec.select(t, o, Wout, wl.width(t + 1))
            followed.append((sel["parent"], sel["token"]))
    return dec, followed, S, Wout


def _chain(followed, b):
    """Beam indices b_0 .. b_{T-1} and tokens c_0 .. c_{T-1} of final beam b, by
    following the parent pointers backwards from the last step."""
    beams, toks = [], []
    cur = b
    for parent, token in reversed(followed):
        toks.append(int(token[cur]))
        cur = int(parent[cur])
        beams.append(cur)
    return beams[::-1], toks[::-1]


def _replay_outputs(wl, r, S_ctx, beams):
    """o_j [H, d_v] of the beam whose index at step j is beams[j]: eq. (3) rerun token
    by token from S_ctx with the beam's own inputs, one value head at a time (value
    head h reads key head h // (H / H_K) of the raw draws)."""
    g = wl.H // wl.hk
    outs = []
    S = [S_ctx[h].copy() for h in range(wl.H)]
    for j, bj in enumerate(beams):
        x = gen.step_inputs(wl, r, j)
        o_j = np.zeros((wl.H, wl.d_v))
        for h in range(wl.H):
            kh = h // g
            q = x["q"].value[kh, bj].astype(np.float64)
            k = x["k"].value[kh, bj].astype(np.float64)
            v = x["v"].value[h, bj].astype(np.float64)
            a = float(x["alpha"][h, bj])
            be = float(x["beta"][h, bj])
            St = S[h]
            St = a * St + be * np.outer(v - a * (St @ k), k)     # eq. (3)
            S[h] = St
            o_j[h] = St @ q                                       # o = S_t q_t
        outs.append(o_j)
    return outs


@pytest.mark.parametrize("mode", ["forced", "select"])
@pytest.mark.parametrize("name,kw", [("tiny", {}), ("tiny", dict(T=5, widths=(4, 9, 6, 11, 7), V=37)),
                                     ("tiny", dict(H=4, H_K=2, widths=(6, 10, 5)))])
def test_sid_prefixes_follow_parent_pointers(name, kw, mode):
    """Every live beam's SID prefix equals the tokens met walking its parents back."""
    wl = _wl(name, **kw)
    dec, followed, _, _ = _run(wl, mode)
    assert dec.tokens.shape == (wl.width(wl.T), wl.T)
    for b in range(wl.width(wl.T)):
        _, toks = _chain(followed, b)
        assert dec.tokens[b].tolist() == toks, (mode, b)


@pytest.mark.parametrize("mode", ["forced", "select"])
@pytest.mark.parametrize("name,kw", [("tiny", {}), ("tiny", dict(T=4, widths=(5, 8, 3, 6), V=40)),
                                     ("tiny", dict(H=4, H_K=2, widths=(6, 10, 5)))])
def test_cumulative_scores_rescored_along_chains(name, kw, mode):
    """A beam's cumulative score is the sum over its steps of log_softmax((sum over
    heads of o_j) . Wout)[c_j], with o_j from eq. (3) rerun along its own chain."""
    wl = _wl(name, **kw)
    r = 0
    dec, followed, S_ctx, Wout = _run(wl, mode, r)
    for b in range(wl.width(wl.T)):
        beams, toks = _chain(followed, b)
        outs = _replay_outputs(wl, r, S_ctx, beams)
        total = 0.0
        for j in range(wl.T):
            z = outs[j].sum(axis=0)
            total += sp_log_softmax(z @ Wout)[toks[j]]
        assert abs(dec.cum[b] - total) <= 1e-10 * max(1.0, abs(total)), (mode, b, dec.cum[b], total)
    if mode == "select":
        # the top-W keeps the beams in score order
        assert np.all(np.diff(dec.cum) <= 0)


def test_grouped_heads_share_key_heads():
    """H = 4 value heads on H_K = 2 key heads.  Value heads 0 and 1 are given the same
    prefill state, v, alpha and beta: with q, k of key head 0 for both, their outputs
    must be identical; value head 2 reads key head 1 and must differ.  Every head's
    output must equal the explicit per-value-head loop."""
    wl = _wl("tiny", H=4, H_K=2, widths=(6, 6, 6))
    r = 0
    S = prefill_request(wl, r).astype(np.float64)
    S[1] = S[0]
    S[3] = S[2]
    dec = FullStateDecoder(S, wl.width(0))
    # per value head, the parent state of every beam of the coming step
    Sref = [np.broadcast_to(S[h], (wl.width(0),) + S[h].shape) for h in range(wl.H)]
    for t in range(wl.T):
        q, k, v, al, be = step_arrays(wl, r, t)
        v, al, be = v.copy(), al.copy(), be.copy()
        v[1], al[1], be[1] = v[0], al[0], be[0]
        v[3], al[3], be[3] = v[2], al[2], be[2]
        o, _ = dec.step(t, q, k, v, al, be)
        np.testing.assert_array_equal(o[0], o[1])
        np.testing.assert_array_equal(o[2], o[3])
        assert np.max(np.abs(o[0] - o[2])) > 1e-3
        # explicit loop over value heads on the raw key-head draws (parents are the
        # identity here, so beam b's parent state is beam b's state of the last step)
        x = gen.step_inputs(wl, r, t)
        for h in range(wl.H):
            kh = h // (wl.H // wl.hk)
            nxt = np.empty((wl.width(t),) + S[h].shape)
            for b in range(wl.width(t)):
                qq = x["q"].value[kh, b].astype(np.float64)
                kk = x["k"].value[kh, b].astype(np.float64)
                P = Sref[h][b]
                nxt[b] = al[h, b] * P + be[h, b] * np.outer(v[h, b] - al[h, b] * (P @ kk), kk)
                np.testing.assert_allclose(o[h, b], nxt[b] @ qq, rtol=1e-12, atol=1e-12)
            Sref[h] = nxt
        ident = np.arange(wl.width(t + 1))
        dec.advance(t, ident, np.zeros_like(ident), np.zeros(len(ident)))


def test_grouped_prefill_reads_its_key_head():
    """The prefill state of value head h runs eq. (3) over the prompt keys of key head
    h // (H / H_K), then is rounded to fp32."""
    wl = _wl("tiny", H=4, H_K=2, L_prompt=(24, 24))
    r = 0
    got = prefill_request(wl, r)
    p = gen.prompt_tokens(wl, r)
    assert p["k"].shape[1] == 2
    for h in range(wl.H):
        kh = h // 2
        S = np.zeros((wl.d_v, wl.d_k))
        for i in range(p["k"].shape[0]):
            k = p["k"][i, kh].astype(np.float64)
            v = p["v"][i, h].astype(np.float64)
            a, b = float(p["alpha"][i, h]), float(p["beta"][i, h])
            S = a * S + b * np.outer(v - a * (S @ k), k)
        # fp32 rounding of the same float64 value (the two sides may round the last
        # float64 bit differently)
        np.testing.assert_allclose(got[h], S, rtol=1e-6, atol=1e-7)
    # the two value heads of a key-head pair differ (their v and gates differ)
    assert np.max(np.abs(got[0] - got[1])) > 1e-3
