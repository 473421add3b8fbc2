"""A logits block that takes several code groups in turn computes, for each group, the
tile maxima and the log-sum-exp part that a block of its own would, in the same order:
a decode is the same bit for bit whatever the number of groups per block
(GDN_BEAM_LOGITS_GPB sets it: 1, 2, 4, 8).  The cases have several code groups, a
partial last group and last tile, blocks holding chunks of several requests, the
bounded and the every-tile tile selection, and both forms of the bf16 codebook's
logits (three bf16 terms, and two fp16 terms where GDN_BEAM_F16_MIN_MACS = 0).
"""
import pytest

import synth
from linear_attention_beam_amd import binding as B
from gpu_harness import GpuDecode, same_bits, say, to_np

pytestmark = pytest.mark.gpu

CASES = {
    # three requests of 300 beams, 1024 codes: bounded selection, blocks over requests
    "multi_bounded": ("tiny", dict(R=3, widths=(300, 300, 300), V=1024, io="bf16", wout="bf16")),
    # 777 codes: seven groups of 128, the last one partial, ending in a partial tile
    "mixed_c": ("single", dict(widths=(64, 700, 700), V=777, io="bf16", wout="bf16")),
    # 512 beams x 1000 codes: the bounded pass over a partial last group
    "bounded_v1000": ("tiny", dict(widths=(512, 512, 512), V=1000, io="bf16", wout="bf16")),
    # d_v = 256 (one tile per stage), 777 codes
    "dv256_v777": ("single", dict(d_k=256, d_v=256, widths=(64, 300, 300), V=777, io="bf16", wout="bf16")),
}


def _record(wl):
    g = GpuDecode(wl, R=wl.R, exact=())
    g.init()
    rec = []
    for t in range(wl.T):
        rec.append(to_np(g.step(t)).copy())
        sel = g.select(t)
        rec += [sel["parent"].copy(), sel["token"].copy(), sel["score"].copy()]
    for what in (B.GDN_EXPORT_ANCESTRY, B.GDN_EXPORT_TOKENS, B.GDN_EXPORT_CUM, B.GDN_EXPORT_STATUS):
        rec.append(g.export(what).copy())
    return rec


@pytest.mark.parametrize("f16", [False, True], ids=["three_bf16_terms", "two_fp16_terms"])
@pytest.mark.parametrize("name", list(CASES))
def test_logits_blocks_of_several_code_groups_decode_the_same_bits(name, f16, monkeypatch):
    base, kw = CASES[name]
    wl = synth.get(base).scaled(name=name, **kw)
    if f16:
        monkeypatch.setenv("GDN_BEAM_F16_MIN_MACS", "0")
    recs = {}
    for gpb in (1, 2, 4, 8):
        monkeypatch.setenv("GDN_BEAM_LOGITS_GPB", str(gpb))
        recs[gpb] = _record(wl)
    say(f"{name} ({'fp16' if f16 else 'bf16'} terms): {wl.R} requests, widths "
        f"{[wl.width(t) for t in range(wl.T + 1)]}, V = {wl.V}, code groups per block 1, 2, 4, 8")
    for gpb in (2, 4, 8):
        for i, (x, y) in enumerate(zip(recs[1], recs[gpb])):
            assert same_bits(x, y), (name, f16, gpb, i)
