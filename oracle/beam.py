"""Oracle: large-beam FullState decoding, scoring, global top-W and ancestry.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP
path and imports nothing from it.

Sources:
  OneLA reading note (paper-archivist.com)
    section 1.1 eq. (1): the SID sequence probability is a product of per-step
        conditionals; large-beam decoding expands every live beam over the
        codebook and keeps a global top-k, so parents change every step.
    section 1.3, Fig. 2: FullState keeps one d_v x d_k state per beam and copies
        states when beams are reordered (copy-on-reorder).
    section 2.2 eq. (4): rank-1 transition (oracle.gdn.rank1_transition).
    section 2.4 eq. (9): ancestry index h_t(b, j) = h_{t-1}(pi_t(b), j) for
        j < t-1, and h_t(b, t-1) = pi_t(b).
  RecoGEM (conceptio mirror), section 4.3: the selection is an exact top-K
        over the W x C candidate matrix of a request.

Readings where the pages are silent:
  * Scoring: z_b = sum over heads of o_b; logits = z_b^T Wout; the step score of
    candidate (b, c) is cum_b + (logit_bc - logsumexp_c(logit_b)), natural log
    (the log of eq. 1's product, one log-softmax per step).
  * Ranking: score descending, then flat index b*V + c ascending.  New beam b'
    is the rank; its parent is b, its token c and its cumulative score the score.
  * t = 0: all W_0 beams are children of S_ctx with cumulative score 0.
"""
from __future__ import annotations

import numpy as np

from .gdn import rank1_transition


def log_softmax_rows(logits):
    """Row-wise natural log-softmax in float64: l - (m + log sum exp(l - m))."""
    m = np.max(logits, axis=1, keepdims=True)
    lse = m + np.log(np.sum(np.exp(logits - m), axis=1, keepdims=True))
    return logits - lse


def step_scores(o, Wout, cum):
    """Candidate scores of one request at one step.

    o [H, W, d_v] outputs of all heads; Wout [d_v, V]; cum [W].
    Returns score [W, V] = cum_b + log_softmax(z_b^T Wout) with z_b = sum_h o_b.
    """
    z = np.sum(o, axis=0)
    logits = z @ Wout
    return cum[:, None] + log_softmax_rows(logits)


def top_w(score, K):
    """Exact global top-K of a [W, V] score matrix by a full sort.

    Order: score descending, then flat index b*V + c ascending.
    Returns (parent [K], token [K], score [K]) in rank order.
    """
    W, V = score.shape
    flat = score.reshape(-1)
    idx = np.arange(W * V, dtype=np.int64)
    order = np.lexsort((idx, -flat))[:K]
    return (order // V).astype(np.int32), (order % V).astype(np.int32), flat[order]


def ancestry_update(anc, parent, t):
    """Eq. (9): ancestry of the children chosen after step t.

    anc [W_t, t] holds h_t(b, j) for the beams of step t (slot = beam index at
    step j).  Returns [W_{t+1}, t+1]: row b' copies its parent's row and
    appends the parent itself as the step-t slot.
    """
    parent = np.asarray(parent, dtype=np.int64)
    out = np.empty((parent.shape[0], t + 1), dtype=np.int32)
    out[:, :t] = anc[parent, :t]
    out[:, t] = parent
    return out


class FullStateDecoder:
    """FullState decode of one request: every beam owns its d_v x d_k state per head.

    Use: step(t, ...) -> (o, delta); then select(t, ...) or advance(t, ...).
    Works in float64, or on object arrays of Fractions when only step() and
    advance() are used.
    """

    def __init__(self, S_ctx, W0):
        S_ctx = np.asarray(S_ctx)
        self.H, self.d_v, self.d_k = S_ctx.shape
        self.S_ctx = S_ctx
        # parent state of every beam of the coming step; at t = 0 it is S_ctx
        self.parent_states = np.broadcast_to(S_ctx[:, None], (self.H, W0, self.d_v, self.d_k))
        self.W = W0
        self.t = 0
        self.cum = np.zeros(W0, dtype=np.float64)
        self.anc = np.zeros((W0, 0), dtype=np.int32)      # h_t(b, j), j < t
        self.tokens = np.zeros((W0, 0), dtype=np.int32)   # SID prefix of each beam
        self.child_states = None

    def step(self, t, q, k, v, alpha, beta):
        """Eq. (4) for every (head, beam): q, k [H, W, d_k]; v [H, W, d_v]; alpha, beta [H, W]."""
        assert t == self.t and q.shape[1] == self.W
        S, delta, o = rank1_transition(self.parent_states, q, k, v, alpha, beta)
        self.child_states = S
        return o, delta

    def advance(self, t, parent, token, cum_next):
        """Re-parent after step t: copy-on-reorder of FullState, ancestry by eq. (9)."""
        parent = np.asarray(parent, dtype=np.int64)
        self.parent_states = self.child_states[:, parent]
        self.anc = ancestry_update(self.anc, parent, t)
        tok = np.empty((parent.shape[0], t + 1), dtype=np.int32)
        tok[:, :t] = self.tokens[parent, :t]
        tok[:, t] = token
        self.tokens = tok
        self.cum = np.asarray(cum_next, dtype=np.float64)
        self.W = parent.shape[0]
        self.t = t + 1
        self.child_states = None

    def select(self, t, o, Wout, W_next, forced_parent=None, forced_token=None):
        """Score, take the global top-W_next, and advance.

        With forced maps the top-W is still computed and returned, but the
        beams follow the forced (parent, token) and their cumulative score is
        the score of that candidate.
        Returns dict(score=[W,V], parent, token, top_score (the top-W result),
        cum (the cumulative scores the beams carry on)).
        """
        score = step_scores(o, Wout, self.cum)
        parent, token, top = top_w(score, W_next)
        if forced_parent is not None:
            fp = np.asarray(forced_parent, dtype=np.int64)
            ft = np.asarray(forced_token, dtype=np.int64)
            cum_next = score[fp, ft]
            self.advance(t, fp, ft, cum_next)
        else:
            cum_next = top
            self.advance(t, parent, token, cum_next)
        return {"score": score, "parent": parent, "token": token,
                "top_score": top, "cum": cum_next}


def capacity_elements(d_k, d_v, W, T):
    """Persistent state elements per (request, head).

    GTR form: one shared S_ctx plus W*T records of (alpha, delta, k), i.e.
    d_v*d_k + W*T*(d_v + d_k + 1) (OneLA reading note, section 2.2 eq. 5 and
    the capacity check in section 4.3).  FullState: W*d_v*d_k.
    """
    return {"gtr": d_v * d_k + W * T * (d_v + d_k + 1), "fullstate": W * d_v * d_k,
            "record": 1 + d_v + d_k, "state": d_v * d_k}
