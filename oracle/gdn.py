"""Oracle: the Gated DeltaNet recurrence, written out plainly (float64 or exact).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP
path and imports nothing from it.

Sources (OneLA reading note, paper-archivist.com):
  section 1.2 eq. (3): S_t = a_t S_{t-1} + b_t (v_t - a_t S_{t-1} k_t) k_t^T,  o_t = S_t q_t
  section 2.2 eq. (4): the same update as a rank-1 step S_t = a_t S_{t-1} + delta_t k_t^T
                       with delta_t = b_t (v_t - a_t S_{t-1} k_t); the parent state of a
                       beam's first decode step is the shared prefill state S_ctx.
Every function works on numpy float64 arrays and equally on numpy object arrays
of fractions.Fraction (only +, -, * and matmul are used), which is how the
exact-arithmetic checks run it.
"""
from __future__ import annotations

import numpy as np


def gdn_token(S, k, v, alpha, beta):
    """One token of eq. (3) for a batch of independent states.

    S [..., d_v, d_k], k [..., d_k], v [..., d_v], alpha/beta [...].
    Returns the new state S_t (the output o_t = S_t q_t is left to the caller).
    """
    Sk = (S @ k[..., None])[..., 0]                          # S_{t-1} k_t
    corr = beta[..., None] * (v - alpha[..., None] * Sk)     # b_t (v_t - a_t S_{t-1} k_t)
    return alpha[..., None, None] * S + corr[..., :, None] * k[..., None, :]


def prefill(k, v, alpha, beta, S0=None):
    """Shared prefill state from a prompt by eq. (3), token by token.

    k [L, H, d_k], v [L, H, d_v], alpha/beta [L, H]  ->  S_ctx [H, d_v, d_k].
    The state before the first prompt token is zero (the pages do not say;
    zero is the plain reading for a fresh recurrence).
    """
    L, H, d_k = k.shape
    d_v = v.shape[2]
    if S0 is None:
        S = np.zeros((H, d_v, d_k), dtype=np.result_type(k, v, np.float64))
    else:
        S = S0.copy()
    for i in range(L):
        S = gdn_token(S, k[i], v[i], alpha[i], beta[i])
    return S


def rank1_transition(P, q, k, v, alpha, beta):
    """One decode step of eq. (4) from explicit parent states (FullState form).

    P [..., d_v, d_k] parent states; q, k [..., d_k]; v [..., d_v]; alpha, beta [...].
    Returns (S, delta, o): the child states, the update vectors delta_t and
    the outputs o_t = S_t q_t (eq. 3's output rule).
    """
    Pk = (P @ k[..., None])[..., 0]
    delta = beta[..., None] * (v - alpha[..., None] * Pk)
    S = alpha[..., None, None] * P + delta[..., :, None] * k[..., None, :]
    o = (S @ q[..., None])[..., 0]
    return S, delta, o
