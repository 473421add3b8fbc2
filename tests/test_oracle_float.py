"""Pins of the CPU oracle in float64: closed forms, brute force, library routines.

Closed forms are derived from eq. (3) (OneLA reading note, section 1.2) and
eq. (4) (section 2.2); scoring is pinned against scipy's log-softmax and the
selection against a full Python sort and RecoGEM's two-stage precut
(section 4.3).  Values printed on the pages are in tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import log_softmax as sp_log_softmax

import synth
from synth import gen
from oracle import (FullStateDecoder, capacity_elements, decode_request, prefill,
                    prefill_request, step_scores, top_w)
from oracle.run import step_arrays

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_state(rng, H, d_v, d_k):
    return rng.standard_normal((H, d_v, d_k))


def _rand_inputs(rng, H, W, d_k, d_v):
    return dict(q=_unit(rng, (H, W, d_k)), k=_unit(rng, (H, W, d_k)),
                v=rng.standard_normal((H, W, d_v)),
                alpha=rng.uniform(0.9, 1.0, (H, W)), beta=rng.uniform(0, 1, (H, W)))


def test_no_gate_no_write_reads_context():
    """alpha = 1, beta = 0 for every step: o_t = S_ctx q_t whatever the parents."""
    rng = np.random.default_rng(0)
    H, d_k, d_v, W = 2, 8, 6, 5
    S_ctx = _rand_state(rng, H, d_v, d_k)
    dec = FullStateDecoder(S_ctx, W)
    for t in range(3):
        x = _rand_inputs(rng, H, W, d_k, d_v)
        x["alpha"][:] = 1.0
        x["beta"][:] = 0.0
        o, delta = dec.step(t, **x)
        ref = np.einsum("hvk,hbk->hbv", S_ctx, x["q"])
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
        assert np.all(delta == 0)
        dec.advance(t, rng.integers(0, W, W), np.zeros(W, np.int32), np.zeros(W))


def test_first_step_query_equals_key():
    """t = 0, |k| = 1, q = k: o = (1 - beta) alpha S_ctx k + beta v (from eq. 3)."""
    rng = np.random.default_rng(1)
    H, d, W = 3, 16, 7
    S_ctx = _rand_state(rng, H, d, d)
    x = _rand_inputs(rng, H, W, d, d)
    x["q"] = x["k"].copy()
    o, _ = FullStateDecoder(S_ctx, W).step(0, **x)
    Sk = np.einsum("hvk,hbk->hbv", S_ctx, x["k"])
    ref = (1 - x["beta"])[..., None] * x["alpha"][..., None] * Sk + x["beta"][..., None] * x["v"]
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_delta_rule_writes_value():
    """alpha = beta = 1 and |k| = 1: the child state maps k_t exactly to v_t."""
    rng = np.random.default_rng(2)
    H, d, W = 2, 12, 4
    dec = FullStateDecoder(_rand_state(rng, H, d, d), W)
    for t in range(3):
        x = _rand_inputs(rng, H, W, d, d)
        x["alpha"][:] = 1.0
        x["beta"][:] = 1.0
        x["q"] = x["k"].copy()
        o, _ = dec.step(t, **x)
        np.testing.assert_allclose(o, x["v"], rtol=1e-12, atol=1e-12)
        dec.advance(t, rng.integers(0, W, W), np.zeros(W, np.int32), np.zeros(W))


def test_single_beam_is_sequential_decode():
    """W = 1 with identity parents: the decode is eq. (3) continued from S_ctx."""
    rng = np.random.default_rng(3)
    H, d_k, d_v, T = 2, 10, 7, 5
    S_ctx = _rand_state(rng, H, d_v, d_k)
    xs = [_rand_inputs(rng, H, 1, d_k, d_v) for _ in range(T)]
    dec = FullStateDecoder(S_ctx, 1)
    for t in range(T):
        o, _ = dec.step(t, **xs[t])
        dec.advance(t, [0], [0], [0.0])
        # eq. (3) over the same tokens with the prompt routine, from S_ctx
        S = prefill(np.stack([x["k"][:, 0] for x in xs[:t + 1]]),
                    np.stack([x["v"][:, 0] for x in xs[:t + 1]]),
                    np.stack([x["alpha"][:, 0] for x in xs[:t + 1]]),
                    np.stack([x["beta"][:, 0] for x in xs[:t + 1]]), S0=S_ctx)
        ref = np.einsum("hvk,hk->hv", S, xs[t]["q"][:, 0])
        np.testing.assert_allclose(o[:, 0], ref, rtol=1e-11, atol=1e-11)


def test_prefill_orthonormal_keys_closed_form():
    """alpha = beta = 1 with orthonormal keys from S = 0: S_L = sum_i v_i k_i^T."""
    rng = np.random.default_rng(4)
    d_k, d_v, L = 8, 5, 6
    Q, _ = np.linalg.qr(rng.standard_normal((d_k, d_k)))
    k = Q[:L][:, None, :]                       # [L, 1, d_k], orthonormal rows
    v = rng.standard_normal((L, 1, d_v))
    ones = np.ones((L, 1))
    S = prefill(k, v, ones, ones)
    np.testing.assert_allclose(S[0], v[:, 0].T @ k[:, 0], rtol=1e-12, atol=1e-12)


def test_prefill_decay_only():
    """beta = 0: the state only decays, S_L = (prod alpha) S_0."""
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((2, 4, 3))
    L = 9
    a = rng.uniform(0.5, 1.0, (L, 2))
    S = prefill(_unit(rng, (L, 2, 3)), rng.standard_normal((L, 2, 4)), a, np.zeros((L, 2)), S0=S0)
    np.testing.assert_allclose(S, np.prod(a, axis=0)[:, None, None] * S0, rtol=1e-12)


def _brute_force_eq3(S_ctx, xs, parent_maps, t, b):
    """Eq. (3) rerun along beam b's history (float64), one head at a time."""
    chain = [b]
    for j in range(t, 0, -1):
        chain.append(int(parent_maps[j - 1][chain[-1]]))
    chain.reverse()
    outs = []
    for h in range(S_ctx.shape[0]):
        S = S_ctx[h].copy()
        for j in range(t + 1):
            q, k, v, a, be = (xs[j][n][h, chain[j]] for n in range(5))
            S = a * S + be * np.outer(v - a * (S @ k), k)
        outs.append(S @ q)
    return np.array(outs)


def test_tiny_workload_matches_brute_force():
    """The tiny workload in forced mode: FullState equals eq. (3) rerun per beam."""
    wl = synth.get("tiny")
    S_ctx = prefill_request(wl, 0).astype(np.float64)
    recs = decode_request(wl, 0, S_ctx, mode="forced")
    xs = [step_arrays(wl, 0, t) for t in range(wl.T)]
    maps = [gen.forced_parents(wl, 0, t) for t in range(wl.T)]
    for t in range(wl.T):
        for b in range(wl.width(t)):
            ref = _brute_force_eq3(S_ctx, xs, maps, t, b)
            got = recs[t]["o"][:, b]
            assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        np.testing.assert_array_equal(recs[t]["token"].shape, (wl.width(t + 1),))


def test_scores_match_library_log_softmax():
    rng = np.random.default_rng(6)
    H, W, d_v, V = 3, 6, 5, 11
    o = rng.standard_normal((H, W, d_v))
    Wout = rng.standard_normal((d_v, V))
    cum = rng.standard_normal(W)
    s = step_scores(o, Wout, cum)
    ref = cum[:, None] + sp_log_softmax(o.sum(0) @ Wout, axis=1)
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)


def test_scores_zero_codebook():
    """Wout = 0: every candidate scores cum_b - log V."""
    s = step_scores(np.ones((2, 3, 4)), np.zeros((4, 7)), np.array([0.0, -1.0, 2.5]))
    np.testing.assert_allclose(s, np.array([0.0, -1.0, 2.5])[:, None] - math.log(7) + np.zeros((3, 7)),
                               rtol=0, atol=1e-15)


def _two_stage(score, K):
    """RecoGEM section 4.3: per-row precut to the row's top K, then a request-level top-K."""
    W, V = score.shape
    keep = []
    for b in range(W):
        row = sorted(range(V), key=lambda c: (-score[b, c], c))[:K]
        keep += [(score[b, c], b * V + c) for c in row]
    keep.sort(key=lambda p: (-p[0], p[1]))
    return [i for _, i in keep[:K]]


@pytest.mark.parametrize("kind", ["random", "ties", "all_equal"])
@pytest.mark.parametrize("W,V,K", [(4, 9, 4), (8, 32, 8), (5, 6, 30), (3, 7, 1)])
def test_top_w_exact_and_ordered(kind, W, V, K):
    rng = np.random.default_rng(W * 100 + V + K)
    if kind == "random":
        score = rng.standard_normal((W, V))
    elif kind == "ties":
        score = rng.integers(-3, 3, (W, V)).astype(np.float64)
    else:
        score = np.full((W, V), -1.5)
    p, c, s = top_w(score, K)
    flat = [p_ * V + c_ for p_, c_ in zip(p, c)]
    full = sorted(range(W * V), key=lambda i: (-score.reshape(-1)[i], i))[:K]
    assert flat == full
    assert flat == _two_stage(score, K)
    np.testing.assert_array_equal(s, score[p, c])


def test_golden_page_counts():
    """Sizes the pages print: 257-element records, ~64x per record, ~30x capacity."""
    g = json.load(open(os.path.join(GOLDEN, "pages_counts.json")))
    c = capacity_elements(128, 128, W=1, T=1)
    assert c["record"] == g["gtr_record_elements_d128"]["value"]
    assert c["state"] == g["full_state_elements_d128"]["value"]
    assert abs(c["state"] / c["record"] - g["record_saving_ratio_approx"]["value"]) <= \
        g["record_saving_ratio_approx"]["tolerance"]
    e = g["capacity_ratio_W512_T2_approx"]
    c2 = capacity_elements(e["d_k"], e["d_v"], W=e["W"], T=e["T"])
    assert abs(c2["fullstate"] / c2["gtr"] - e["value"]) <= e["tolerance"]
    f = g["flat_candidates_C8192_W512"]
    assert 512 * 8192 == f["value"] and 2 * f["value"] == f["bytes_fp16"]


def test_generator_is_request_keyed_and_rounds_bf16():
    """Regenerating one request alone gives the same draws; bf16 values are exact bf16."""
    wl = synth.get("batch")
    a = gen.step_inputs(wl, 3, 1)
    b = gen.step_inputs(wl, 3, 1)
    np.testing.assert_array_equal(a["q"].bits, b["q"].bits)
    assert a["q"].bits.dtype == np.uint16
    v = a["q"].value
    assert np.all((v.view(np.uint32) & 0xFFFF) == 0)
    # round-to-nearest-even on a few hand cases: 1 + 2^-8 ties to 1, 1 + 3*2^-8 ties up
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.0 ** -9], dtype=np.float32)
    np.testing.assert_array_equal(gen.bf16_value(gen.bf16_bits(x)),
                                  np.array([1.0, 1.0, 1 + 2.0 ** -6, -2.0 ** -9], np.float32))


def test_heavy_fanout_parent_law():
    wl = synth.get("stress")
    p = gen.forced_parents(wl, 0, 0)
    assert p.shape == (1024,)
    top = -(-1024 // 10)
    assert np.sum(p < top) == (8 * 1024) // 10
    assert p.min() >= 0 and p.max() < 1024
