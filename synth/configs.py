"""Workload table for large-beam Gated DeltaNet decoding.

Each workload is one synthetic decode job: R requests, H GDN heads of shape
d_v x d_k, a shared prefill state per (request, head) seeded from L_prompt
random tokens, then T SID steps with W_t live beams and a codebook of V
tokens.  Sizes follow the operator sweep and selection shapes of the OneLA
reading note (section 3, experimental setup) and RecoGEM (section 4.3, fast
candidate selection).

Nothing here computes anything: it only names sizes and seeds.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    R: int                      # requests
    H: int                      # GDN heads
    d_k: int
    d_v: int
    io: str                     # dtype of q, k, v ("f32" | "bf16"); GTR keys stored in it
    wout: str                   # dtype of the codebook projection ("f32" | "bf16")
    L_prompt: Tuple[int, int]   # prompt length range [lo, hi] (lo == hi: fixed)
    T: int                      # SID decode steps
    widths: Tuple[int, ...]     # W_0 .. W_{T-1}; the last select keeps W_T = W_{T-1}
    V: int                      # codebook size per step
    parents: str                # forced parent draw: "uniform" | "heavy"
    seed: int
    H_K: int = 0                # key heads (0: one per value head); value head h uses
                                # key head h // (H / H_K), grouped value heads
    summary: str = field(default="", compare=False)

    @property
    def hk(self) -> int:
        """Key heads: q, k and the records' keys are per key head."""
        return self.H_K or self.H

    @property
    def group(self) -> int:
        """Value heads per key head."""
        return self.H // self.hk

    @property
    def W_max(self) -> int:
        return max(self.widths)

    def width(self, t: int) -> int:
        """Live beams at step t (t == T gives the width kept by the last select)."""
        return self.widths[min(t, self.T - 1)]

    def transitions(self) -> int:
        """GDN beam transitions of one decode: sum over steps of R*H*W_t."""
        return sum(self.R * self.H * self.width(t) for t in range(self.T))

    def scaled(self, **kw) -> "Workload":
        d = {k: getattr(self, k) for k in self.__dataclass_fields__}
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", R=1, H=1, d_k=16, d_v=16, io="f32", wout="f32",
        L_prompt=(64, 64), T=3, widths=(8, 8, 8), V=32, parents="uniform",
        seed=1001,
        summary="1 request, 1 head, d=16, fp32, W=8, V=32, T=3, L_prompt=64"),
    "single": Workload(
        name="single", R=1, H=4, d_k=128, d_v=128, io="f32", wout="f32",
        L_prompt=(1024, 1024), T=3, widths=(128, 128, 128), V=256,
        parents="uniform", seed=1002,
        summary="1 request, 4 heads, d=128, fp32, W=128, V=256, T=3, L_prompt=1024"),
    "batch": Workload(
        name="batch", R=32, H=16, d_k=128, d_v=128, io="bf16", wout="bf16",
        L_prompt=(1024, 1024), T=4, widths=(256, 256, 256, 256), V=1024,
        parents="uniform", seed=1003,
        summary="32 requests, 16 heads, d=128, bf16 io / fp32 state, W=256, V=1024, T=4"),
    "stress": Workload(
        name="stress", R=64, H=16, d_k=128, d_v=128, io="bf16", wout="bf16",
        L_prompt=(1024, 1024), T=4, widths=(1024, 1024, 1024, 1024), V=8192,
        parents="heavy", seed=1004,
        summary="64 requests, 16 heads, d=128, bf16 io, W=1024, V=8192, T=4, heavy fan-out"),
    "growing": Workload(
        name="growing", R=128, H=16, d_k=128, d_v=256, io="bf16", wout="bf16",
        L_prompt=(512, 8192), T=4, widths=(64, 256, 512, 1024), V=4096,
        parents="uniform", seed=1005,
        summary="128 requests, 16 heads, d_k=128, d_v=256, bf16 io, W 64->256->512->1024, V=4096, T=4"),
    # geometry variants of the operator sweep at the batch shape
    "wide": Workload(
        name="wide", R=32, H=16, d_k=256, d_v=256, io="bf16", wout="bf16",
        L_prompt=(1024, 1024), T=4, widths=(256, 256, 256, 256), V=1024,
        parents="uniform", seed=1006,
        summary="32 requests, 16 heads, d_k=d_v=256, bf16 io, W=256, V=1024, T=4"),
    "grouped": Workload(
        name="grouped", R=32, H=32, H_K=16, d_k=128, d_v=128, io="bf16", wout="bf16",
        L_prompt=(1024, 1024), T=4, widths=(256, 256, 256, 256), V=1024,
        parents="uniform", seed=1007,
        summary="32 requests, 32 value heads on 16 key heads, d=128, bf16 io, W=256, V=1024, T=4"),
    "wide_v": Workload(
        name="wide_v", R=32, H=16, d_k=128, d_v=512, io="bf16", wout="bf16",
        L_prompt=(1024, 1024), T=4, widths=(256, 256, 256, 256), V=1024,
        parents="uniform", seed=1008,
        summary="32 requests, 16 heads, d_k=128, d_v=512, bf16 io, W=256, V=1024, T=4"),
}


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None
