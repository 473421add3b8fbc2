"""Pins of the CPU oracle in exact rational arithmetic (no GPU).

The oracle's FullState decode (eq. 4 of the OneLA reading note, section 2.2)
is checked for EQUALITY against two implementations written only here:
  * brute force: walk each beam's parents back and rerun eq. (3) (section 1.2)
    token by token from S_ctx with that beam's own inputs;
  * projection replay: eqs. (6)-(8) (section 2.3) over append-only transition
    records located through the ancestry index of eq. (9) (section 2.4).
The reading note states the replay is an exact reordering, not an
approximation, so in rational arithmetic all three must agree exactly.
"""
from fractions import Fraction as F

import numpy as np
import pytest

from oracle.beam import FullStateDecoder, ancestry_update
from oracle.gdn import prefill


def _rat(rng, shape, lo=-3, hi=3, den=4):
    """Small random rationals as an object array."""
    num = rng.integers(lo * den, hi * den + 1, size=shape)
    out = np.empty(shape, dtype=object)
    for i, n in np.ndenumerate(num):
        out[i] = F(int(n), den)
    return out


def _gate(rng, shape):
    """Rational gates in (0, 1]."""
    num = rng.integers(1, 9, size=shape)
    out = np.empty(shape, dtype=object)
    for i, n in np.ndenumerate(num):
        out[i] = F(int(n), 8)
    return out


def _problem(seed, H=2, d_k=3, d_v=3, widths=(3, 3, 3), L=4):
    rng = np.random.default_rng(seed)
    pk, pv = _rat(rng, (L, H, d_k)), _rat(rng, (L, H, d_v))
    pa, pb = _gate(rng, (L, H)), _gate(rng, (L, H))
    S_ctx = prefill(pk, pv, pa, pb)
    steps, parents = [], []
    for t, W in enumerate(widths):
        steps.append(dict(q=_rat(rng, (H, W, d_k)), k=_rat(rng, (H, W, d_k)),
                          v=_rat(rng, (H, W, d_v)), alpha=_gate(rng, (H, W)),
                          beta=_gate(rng, (H, W))))
        W_next = widths[t + 1] if t + 1 < len(widths) else W
        parents.append(rng.integers(0, W, W_next))
    return S_ctx, steps, parents


def _brute_force(S_ctx, steps, parents, t, b):
    """Eq. (3) rerun along beam b's own history; returns o_t per head."""
    chain = [b]                       # beam index at steps t, t-1, ..., 0
    for j in range(t, 0, -1):
        chain.append(int(parents[j - 1][chain[-1]]))
    chain.reverse()
    H = S_ctx.shape[0]
    outs = []
    for h in range(H):
        S = S_ctx[h].copy()
        for j in range(t + 1):
            x = steps[j]
            bj = chain[j]
            k, v, q = x["k"][h, bj], x["v"][h, bj], x["q"][h, bj]
            a, be = x["alpha"][h, bj], x["beta"][h, bj]
            S = a * S + be * np.outer(v - a * S.dot(k), k)   # eq. (3), S_t
            o = S.dot(q)                                        # o_t = S_t q_t
        outs.append(o)
    return outs


def _replay(S_ctx, steps, parents):
    """Eqs. (6)-(8) with GTRs in fixed slots (j, b) and the ancestry of eq. (9)."""
    H = S_ctx.shape[0]
    pool = {}                    # (h, j, slot) -> (alpha_j, delta_j, k_j)
    anc = {b: [] for b in range(steps[0]["q"].shape[1])}
    results = []
    for t, x in enumerate(steps):
        W = x["q"].shape[1]
        o_t, d_t = {}, {}
        for h in range(H):
            for b in range(W):
                q, k, v = x["q"][h, b], x["k"][h, b], x["v"][h, b]
                a, be = x["alpha"][h, b], x["beta"][h, b]
                uq, uk = S_ctx[h].dot(q), S_ctx[h].dot(k)        # u^(-1)
                for j, slot in enumerate(anc[b]):                # 0 <= j < t
                    aj, dj, kj = pool[(h, j, slot)]
                    uq = aj * uq + dj * kj.dot(q)                # eq. (6)
                    uk = aj * uk + dj * kj.dot(k)                # eq. (7)
                delta = be * (v - a * uk)                        # eq. (8)
                o = a * uq + delta * k.dot(q)
                pool[(h, t, b)] = (a, delta, k)                  # append r_t at slot (t, b)
                o_t[(h, b)], d_t[(h, b)] = o, delta
        results.append((o_t, d_t))
        anc = {c: anc[int(p)] + [int(p)] for c, p in enumerate(parents[t])}   # eq. (9)
    return results


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fullstate_equals_brute_force_and_replay_exactly(seed):
    S_ctx, steps, parents = _problem(seed)
    H = S_ctx.shape[0]
    dec = FullStateDecoder(S_ctx, steps[0]["q"].shape[1])
    replay = _replay(S_ctx, steps, parents)
    for t, x in enumerate(steps):
        o, delta = dec.step(t, x["q"], x["k"], x["v"], x["alpha"], x["beta"])
        assert o.dtype == object and isinstance(o[0, 0, 0], F)
        W = x["q"].shape[1]
        for b in range(W):
            bf = _brute_force(S_ctx, steps, parents, t, b)
            for h in range(H):
                assert list(o[h, b]) == list(bf[h]), (t, b, h)
                assert list(o[h, b]) == list(replay[t][0][(h, b)]), (t, b, h)
                assert list(delta[h, b]) == list(replay[t][1][(h, b)]), (t, b, h)
        dec.advance(t, parents[t], np.zeros(len(parents[t]), dtype=np.int32),
                    np.zeros(len(parents[t])))


def test_growing_widths_exact():
    """Fan-out 2 -> 4 -> 5 beams: eq. (9) and the replay stay exact."""
    S_ctx, steps, parents = _problem(7, H=1, d_k=2, d_v=4, widths=(2, 4, 5), L=3)
    dec = FullStateDecoder(S_ctx, 2)
    replay = _replay(S_ctx, steps, parents)
    for t, x in enumerate(steps):
        o, delta = dec.step(t, x["q"], x["k"], x["v"], x["alpha"], x["beta"])
        for b in range(x["q"].shape[1]):
            assert list(o[0, b]) == list(replay[t][0][(0, b)])
            assert list(o[0, b]) == list(_brute_force(S_ctx, steps, parents, t, b)[0])
        dec.advance(t, parents[t], np.zeros(len(parents[t]), dtype=np.int32),
                    np.zeros(len(parents[t])))


def test_ancestry_matches_pointer_chasing():
    """Eq. (9) equals following the parent pointers back, and slots are in range."""
    rng = np.random.default_rng(3)
    widths = [5, 7, 3, 6, 6]
    anc = np.zeros((widths[0], 0), dtype=np.int32)
    maps = []
    for t in range(len(widths) - 1):
        p = rng.integers(0, widths[t], widths[t + 1])
        maps.append(p)
        anc = ancestry_update(anc, p, t)
        for b in range(widths[t + 1]):
            cur = b
            for j in range(t, -1, -1):
                cur = int(maps[j][cur])
                assert anc[b, j] == cur
                assert 0 <= cur < widths[j]
