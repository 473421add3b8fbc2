"""GPU parity of the prefill (eq. 3 of the OneLA reading note, section 1.2) against the
oracle's token-by-token fp64 recurrence, for both forms of gdn_beam_prefill: the chunked
form (with a workspace) and the token-sequential form (without).

Bar: 1e-4 max per-row relative error of S_ctx (the fp32-io bar of the workloads).
The chunked form cuts the stacked prompt array into 32-token blocks, so the cases
include prompts shorter than a block, prompts that start and end inside blocks, empty
prompts, several prompts inside one block and, at the full growing size, requests of
512..8192 tokens sampled over the batch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import device as sdev
from linear_attention_beam_amd import binding as B
from linear_attention_beam_amd.decoder import prefill
from gpu_harness import rel_err, say, to_np
from test_gpu_parity import _wl

pytestmark = pytest.mark.gpu

TOL = 1e-4
FORMS = ("chunked", "token")


def _run(p, wl, R, form):
    S = torch.full((R, wl.H, wl.d_v, wl.d_k), float("nan"), dtype=torch.float32, device="cuda")
    say(f"gdn_beam_prefill {wl.name} R={R} N={p['N']} form={form}")
    prefill(S, p["k"], p["v"], p["alpha"], p["beta"], p["offsets"], chunked=form == "chunked")
    torch.cuda.synchronize()
    return to_np(S)


def _oracle_from_device(p, wl, r, heads=None):
    """oracle.prefill over request r's rows of the device-drawn prompt arrays."""
    lo, hi = int(p["offsets"][r]), int(p["offsets"][r + 1])
    k = np.repeat(to_np(p["k"][lo:hi]).astype(np.float64), wl.group, axis=1)
    v, a, b = (to_np(p[n][lo:hi]).astype(np.float64) for n in ("v", "alpha", "beta"))
    if heads is not None:
        hs = list(heads)
        k, v, a, b = k[:, hs], v[:, hs], a[:, hs], b[:, hs]
    return oracle.prefill(k, v, a, b)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("name,R", [("tiny", 1), ("single", 1), ("batch", 2), ("single_gqa", 1),
                                    ("single_dk256", 1), ("single_dk256_dv512", 1),
                                    ("single_dv512", 1)])
def test_prefill_matches_oracle(name, R, form):
    wl = _wl(name)
    p = sdev.prompts(wl, torch.device("cuda"), R=R)
    for r in range(R):
        sdev.upload_prompt(p, wl, r)
    S = _run(p, wl, R, form)
    for r in range(R):
        e = rel_err(S[r], oracle.prefill_request(wl, r))
        say(f"prefill r={r} rel err {e:.3e}")
        assert e <= TOL


# prompt lengths that put request boundaries everywhere inside 32-token blocks
RAGGED = [1, 5, 0, 33, 64, 31, 100, 0, 7, 26, 3, 90]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("name", ["single", "single_gqa", "single_dk256_dv512"])
def test_prefill_ragged_prompts(name, form):
    wl = _wl(name)
    R = len(RAGGED)
    p = sdev.prompts(wl, torch.device("cuda"), R=R, lengths=RAGGED)
    S = _run(p, wl, R, form)
    for r in range(R):
        ref = _oracle_from_device(p, wl, r)
        if RAGGED[r] == 0:
            assert np.all(S[r] == 0.0), "an empty prompt leaves the zero state"
            continue
        e = rel_err(S[r], ref)
        say(f"r={r} L={RAGGED[r]} rel err {e:.3e}")
        assert e <= TOL


def test_prefill_nan_prompt_stays_in_its_request():
    """A NaN key of one prompt reaches none of the prompts that share its 32-token
    blocks (the chunked form's in-block products stay inside each request)."""
    wl = _wl("single")
    lengths = [40, 20, 50]                       # request 1 lies inside blocks 1 and 2
    p = sdev.prompts(wl, torch.device("cuda"), R=3, lengths=lengths)
    p["k"][45, 0, 3] = float("nan")
    p["alpha"][50, 1] = float("nan")
    S = _run(p, wl, 3, "chunked")
    for r in (0, 2):
        e = rel_err(S[r], _oracle_from_device(p, wl, r))
        say(f"r={r} rel err {e:.3e}")
        assert e <= TOL
    assert np.isnan(S[1]).any()


def test_prefill_growing_full_size():
    """The growing workload's prefill at full size (128 requests of 512..8192 tokens,
    16 heads, d_k = 128, d_v = 256) in the chunked form the decode benchmark runs:
    requests spread over the batch checked against the oracle on three heads, and every
    state against the token-sequential form."""
    wl = synth.get("growing")
    dev = torch.device("cuda")
    p = sdev.prompts(wl, dev)
    sample = [0, 37, 64, 101, 127]
    for r in sample:
        sdev.upload_prompt(p, wl, r)
    heads = [0, wl.H // 2, wl.H - 1]
    S = _run(p, wl, wl.R, "chunked")
    for r in sample:
        e = rel_err(S[r][heads], oracle.prefill_request(wl, r, heads=heads))
        say(f"r={r} L={p['lengths'][r]} rel err {e:.3e}")
        assert e <= TOL
    T = _run(p, wl, wl.R, "token")
    assert np.isfinite(S).all()
    e = rel_err(S, T)
    say(f"chunked vs token-sequential, all requests and heads: {e:.3e}")
    assert e <= 2 * TOL


def test_prefill_workspace_reuse_and_short_workspace():
    """One workspace serves consecutive calls of different sizes; a short one is refused."""
    wl = _wl("single")
    dev = torch.device("cuda")
    big = B.gdn_beam_prefill_workspace_bytes(wl.H, wl.d_k, wl.d_v, 400)
    ws = torch.empty(big, dtype=torch.uint8, device=dev)
    for lengths in ([100, 300], [7, 70, 9]):
        R = len(lengths)
        p = sdev.prompts(wl, dev, R=R, lengths=lengths)
        S = torch.empty((R, wl.H, wl.d_v, wl.d_k), dtype=torch.float32, device=dev)
        prefill(S, p["k"], p["v"], p["alpha"], p["beta"], p["offsets"], workspace=ws)
        torch.cuda.synchronize()
        S = to_np(S)
        for r in range(R):
            assert rel_err(S[r], _oracle_from_device(p, wl, r)) <= TOL
    p = sdev.prompts(wl, dev, R=1, lengths=[500])
    S = torch.empty((1, wl.H, wl.d_v, wl.d_k), dtype=torch.float32, device=dev)
    with pytest.raises(B.GdnBeamError) as ei:
        prefill(S, p["k"], p["v"], p["alpha"], p["beta"], p["offsets"], workspace=ws)
    assert ei.value.status == B.GDN_ERR_WORKSPACE


def test_prefill_zero_and_tiny_decay():
    """Decay gates of 0 (the state restarts from that token) and of 1e-20 (whose products
    underflow in fp32), inside a chunk, at a chunk's last and first tokens and over a
    run: both forms agree with the oracle and stay finite.  The chunked form takes its
    in-chunk decay ratios as direct products over the tokens between, never as quotients,
    so no 0/0 or inf can arise."""
    wl = _wl("single")
    lengths = [100, 70]                          # request 1 starts inside block 3
    p = sdev.prompts(wl, torch.device("cuda"), R=2, lengths=lengths)
    a = p["alpha"]
    a[5, :] = 0.0
    a[31, :] = 0.0                               # last token of block 0
    a[32, :] = 1e-20                             # first token of block 1
    a[77, :] = 0.0
    a[120, :2] = 1e-20                           # two heads only
    a[150:153, :] = 0.0                          # a run, in request 1
    for form in FORMS:
        S = _run(p, wl, 2, form)
        for r in range(2):
            assert np.isfinite(S[r]).all(), (form, r)
            e = rel_err(S[r], _oracle_from_device(p, wl, r))
            say(f"{form} r={r} rel err {e:.3e}")
            assert e <= TOL
