"""Large synthetic inputs drawn directly on the device (torch RNG).

Same laws as synth.gen, different random streams: used where the host
generator would be too slow (all requests of the large workloads).  Requests
that are checked against the oracle are overwritten with synth.gen's draws
(upload_request / upload_prompt), so both sides see identical bits for them.
Holds only random draws and dtype casts.
"""
from __future__ import annotations

import numpy as np
import torch

from . import gen
from .configs import Workload

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(wl: Workload, tag: int, t: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((wl.seed * 1000003 + tag * 9176 + t) & 0x7FFFFFFF)
    return g


def _unit(shape, g, device):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x / x.norm(dim=-1, keepdim=True)


def step_inputs(wl: Workload, t: int, device, R=None) -> dict:
    """q, k [R,H,W_t,d_k], v [R,H,W_t,d_v] in the io dtype; alpha, beta [R,H,W_t] fp32."""
    R = wl.R if R is None else R
    W = wl.width(t)
    g = _gen(wl, 3, t, device)
    dt = TDT[wl.io]
    q = _unit((R, wl.hk, W, wl.d_k), g, device).to(dt)
    k = _unit((R, wl.hk, W, wl.d_k), g, device).to(dt)
    v = torch.randn((R, wl.H, W, wl.d_v), generator=g, device=device).to(dt)
    alpha = torch.rand((R, wl.H, W), generator=g, device=device) * 0.1 + 0.9
    beta = torch.rand((R, wl.H, W), generator=g, device=device)
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "alpha": alpha.contiguous(), "beta": beta.contiguous()}


def _to_dev(x: gen.Tensor, device) -> torch.Tensor:
    if x.dtype == "bf16":
        return torch.from_numpy(x.bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x.value).to(device)


def upload_request(dst: dict, wl: Workload, r: int, t: int, slot=None):
    """Overwrite request r's slice (at index `slot`, default r) with synth.gen's draws."""
    x = gen.step_inputs(wl, r, t)
    i = r if slot is None else slot
    dev = dst["q"].device
    for name in ("q", "k", "v"):
        dst[name][i].copy_(_to_dev(x[name], dev))
    dst["alpha"][i].copy_(torch.from_numpy(x["alpha"]).to(dev))
    dst["beta"][i].copy_(torch.from_numpy(x["beta"]).to(dev))


def wout(wl: Workload, device) -> torch.Tensor:
    return _to_dev(gen.wout(wl), device).contiguous()


def wout_step(wl: Workload, t: int, V: int, device) -> torch.Tensor:
    return _to_dev(gen.wout_step(wl, t, V), device).contiguous()


def prompts(wl: Workload, device, R=None, lengths=None) -> dict:
    """Stacked prompt tokens of R requests: k [N,H,d_k], v [N,H,d_v], alpha, beta [N,H], offsets [R+1]."""
    R = wl.R if R is None else R
    if lengths is None:
        lengths = [gen.prompt_length(wl, r) for r in range(R)]
    offs = np.zeros(R + 1, dtype=np.int32)
    offs[1:] = np.cumsum(lengths)
    N = int(offs[-1])
    g = _gen(wl, 2, 0, device)
    k = _unit((N, wl.hk, wl.d_k), g, device)
    v = torch.randn((N, wl.H, wl.d_v), generator=g, device=device)
    alpha = torch.rand((N, wl.H), generator=g, device=device) * 0.1 + 0.9
    beta = torch.rand((N, wl.H), generator=g, device=device)
    return {"k": k, "v": v, "alpha": alpha, "beta": beta,
            "offsets": torch.from_numpy(offs).to(device), "N": N, "lengths": list(lengths)}


def upload_prompt(dst: dict, wl: Workload, r: int, slot=None):
    """Overwrite request r's prompt rows with synth.gen's draws (lengths must match)."""
    p = gen.prompt_tokens(wl, r)
    i = r if slot is None else slot
    lo, hi = int(dst["offsets"][i]), int(dst["offsets"][i + 1])
    assert hi - lo == p["k"].shape[0]
    dev = dst["k"].device
    for name in ("k", "v", "alpha", "beta"):
        dst[name][lo:hi].copy_(torch.from_numpy(p[name]).to(dev))
