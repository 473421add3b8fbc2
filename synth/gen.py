"""Seeded synthetic inputs for large-beam GDN decoding (numpy, host side).

This module serves both the GPU path and the CPU oracle.  It only draws
random numbers and casts them to the storage dtype of a workload; it holds
none of the decoding arithmetic.

Distributions (OneLA reading note, section 1.2 eq. 3 symbols; the pages do
not fix them, so the plainest choice is taken):
  q, k ~ N(0, I) then L2-normalised in fp32; v ~ N(0, I);
  alpha ~ U[0.9, 1.0]; beta ~ U[0, 1]  (fp32, one per request/head/step/beam);
  codebook projection Wout[d_v, V] ~ N(0, 1/d_v);
  prompt tokens use the same k, v, alpha, beta laws (fp32).
Values the workload stores in bf16 are rounded to nearest-even here, so every
consumer sees identical bits.

Every stream is keyed by (seed, tag, request, step): a single request can be
regenerated on its own, which is how sampled requests of large workloads are
checked.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload

# stream tags
_PLEN, _PROMPT, _STEP, _WOUT, _PARENT, _TOKEN = 1, 2, 3, 4, 5, 6


def _rng(wl: Workload, tag: int, r: int = 0, t: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.seed, tag, r, t]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """float32 value of bfloat16 bit patterns."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """A synthetic array: the float32 value every consumer uses, plus the stored bits."""

    __slots__ = ("value", "bits", "dtype")

    def __init__(self, value: np.ndarray, dtype: str):
        value = np.ascontiguousarray(value, dtype=np.float32)
        if dtype == "bf16":
            self.bits = bf16_bits(value)
            self.value = bf16_value(self.bits)
        elif dtype == "f32":
            self.bits = value
            self.value = value
        else:
            raise ValueError(dtype)
        self.dtype = dtype

    @property
    def shape(self):
        return self.value.shape


def _unit(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def prompt_length(wl: Workload, r: int) -> int:
    lo, hi = wl.L_prompt
    if lo == hi:
        return lo
    return int(_rng(wl, _PLEN, r).integers(lo, hi + 1))


def prompt_tokens(wl: Workload, r: int) -> dict:
    """Prompt tokens of request r: k [L,H,d_k], v [L,H,d_v], alpha/beta [L,H], all fp32."""
    L = prompt_length(wl, r)
    g = _rng(wl, _PROMPT, r)
    k = _unit(g, (L, wl.hk, wl.d_k))
    v = g.standard_normal((L, wl.H, wl.d_v), dtype=np.float32)
    alpha = g.uniform(0.9, 1.0, (L, wl.H)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (L, wl.H)).astype(np.float32)
    return {"k": k, "v": v, "alpha": alpha, "beta": beta}


def step_inputs(wl: Workload, r: int, t: int) -> dict:
    """Per-beam inputs of request r at SID step t (arrays [H, W_t, .])."""
    W = wl.width(t)
    g = _rng(wl, _STEP, r, t)
    q = _unit(g, (wl.hk, W, wl.d_k))
    k = _unit(g, (wl.hk, W, wl.d_k))
    v = g.standard_normal((wl.H, W, wl.d_v), dtype=np.float32)
    alpha = g.uniform(0.9, 1.0, (wl.H, W)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (wl.H, W)).astype(np.float32)
    return {"q": Tensor(q, wl.io), "k": Tensor(k, wl.io), "v": Tensor(v, wl.io),
            "alpha": alpha, "beta": beta}


def wout(wl: Workload) -> Tensor:
    """Codebook projection [d_v, V], shared by all heads, requests and steps."""
    g = _rng(wl, _WOUT)
    w = g.standard_normal((wl.d_v, wl.V), dtype=np.float32) / np.float32(np.sqrt(wl.d_v))
    return Tensor(w.astype(np.float32), wl.wout)


def wout_step(wl: Workload, t: int, V: int) -> Tensor:
    """A step's own codebook projection [d_v, V] (per-step vocabularies), same law as
    wout(); step t draws its own stream."""
    g = _rng(wl, _WOUT, 0, t + 1)
    w = g.standard_normal((wl.d_v, V), dtype=np.float32) / np.float32(np.sqrt(wl.d_v))
    return Tensor(w.astype(np.float32), wl.wout)


def forced_parents(wl: Workload, r: int, t: int) -> np.ndarray:
    """Seed-fixed parent map for the selection after step t: W_{t+1} children of W_t parents.

    "uniform": i.i.d. uniform parents.  "heavy": exactly floor(0.8 W_{t+1})
    children draw from the lowest ceil(0.1 W_t) parent indices (beams are kept
    in score order, so low index = top), the rest from the remaining parents,
    then the child order is shuffled.
    """
    Wp, Wc = wl.width(t), wl.width(t + 1)
    g = _rng(wl, _PARENT, r, t)
    if wl.parents == "uniform":
        return g.integers(0, Wp, Wc).astype(np.int32)
    if wl.parents == "heavy":
        top = max(1, -(-Wp // 10))
        n_top = (8 * Wc) // 10
        if top >= Wp:
            p = g.integers(0, Wp, Wc)
        else:
            p = np.concatenate([g.integers(0, top, n_top), g.integers(top, Wp, Wc - n_top)])
            g.shuffle(p)
        return p.astype(np.int32)
    raise ValueError(wl.parents)


def forced_tokens(wl: Workload, r: int, t: int) -> np.ndarray:
    """Seed-fixed codebook tokens for the W_{t+1} children chosen after step t."""
    return _rng(wl, _TOKEN, r, t).integers(0, wl.V, wl.width(t + 1)).astype(np.int32)
