"""gdn_beam_select_static, the selection that allocates nothing (its per-call scratch
in a static device array), against gdn_beam_select through the C ABI.

Two decoders run the same inputs side by side, one selecting with each entry point;
every selection and the final ancestry, SID prefixes and cumulative scores must have
the same bits (same kernels on the same operands).  Two workloads run one after the
other, the second smaller, so the second reads the array the first left behind.  A
configuration whose selection scratch exceeds the array is refused before any launch.
"""
import numpy as np
import pytest
import torch

import synth
from linear_attention_beam_amd import binding as B
from linear_attention_beam_amd.decoder import BeamDecoder
from gpu_harness import GpuDecode, same_bits, say, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # bounded tile selection from t = 1 (W x ceil(V/32) > 8192), partial chunks
    ("tiny", dict(R=3, widths=(300, 512, 512), V=1024, io="bf16", wout="bf16")),
    # smaller: fewer requests, beams and codes, partial tiles, an fp32 codebook
    ("tiny", dict(R=2, widths=(40, 72, 40), V=200)),
]


def _run_pair(base, kw):
    wl = synth.get(base).scaled(name=f"{base}_static", **kw)
    g = GpuDecode(wl, R=wl.R, exact=())
    other = BeamDecoder(wl.R, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, wl.io, wl.wout, H_K=wl.H_K)
    g.init()
    other.init(g.S_ctx, wl.width(0))
    stream = torch.cuda.current_stream()
    for t in range(wl.T):
        x = g.inputs[t]
        o_a = g.step(t)
        o_b = torch.empty_like(o_a)
        other.step(t, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o_b)
        sel_a = g.select(t)
        K = wl.width(t + 1)
        s_b = {n: torch.empty((wl.R, K), dtype=dt, device=g.dev) for n, dt in
               (("parent", torch.int32), ("token", torch.int32), ("score", torch.float32))}
        say(f"gdn_beam_select_static t={t} R={wl.R} W={wl.width(t)} V={wl.V} W_next={K}")
        B.gdn_beam_select_static(other.ctx, t, o_b, g.Wout, wl.V, K, None, None, s_b["parent"],
                                 s_b["token"], s_b["score"], stream)
        torch.cuda.synchronize()
        assert same_bits(to_np(o_a), to_np(o_b)), f"t={t}: o differs"
        for n in ("parent", "token", "score"):
            assert same_bits(sel_a[n], to_np(s_b[n])), f"t={t}: {n} differs"
    assert other.query() == g.dec.query()
    for what in (B.GDN_EXPORT_ANCESTRY, B.GDN_EXPORT_TOKENS, B.GDN_EXPORT_CUM, B.GDN_EXPORT_STATUS):
        a = g.export(what)
        b = to_np(other.export(what))
        torch.cuda.synchronize()
        assert same_bits(a, b), f"export {what} differs"
    other.close()


def test_static_select_matches_workspace_select_twice():
    for base, kw in CASES:
        _run_pair(base, kw)


def test_static_select_refuses_a_large_configuration():
    """A configuration whose selection scratch exceeds the array is refused with
    GDN_ERR_CAPACITY, and the context can still select from its workspace."""
    wl = synth.get("tiny").scaled(name="tiny_static_big", R=32, T=2, widths=(1024, 1024), V=8192)
    g = GpuDecode(wl, R=wl.R, exact=())
    g.init()
    g.step(0)
    s = g.sel[0]
    K = wl.width(1)
    st = B.raw_status("gdn_beam_select_static", g.dec.ctx, 0, g.o[0].data_ptr(), g.Wout.data_ptr(),
                      wl.V, K, None, None, s["parent"].data_ptr(), s["token"].data_ptr(),
                      s["score"].data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == B.GDN_ERR_CAPACITY
    assert "static array holds" in B.gdn_beam_last_error()
    assert g.dec.query() == (0, wl.width(0))
    sel = g.select(0)                       # the workspace selection still runs
    assert np.all((sel["parent"] >= 0) & (sel["parent"] < wl.width(0)))
