"""Host-side checks of the C ABI (no GPU): exported symbols, workspace formula,
and every argument error that is decided before a launch.

Device pointers passed here are never dereferenced: each call below is
rejected by the host checks before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

import synth
from linear_attention_beam_amd import binding as B
from oracle import capacity_elements

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gdn_beam.h")
FAKE = 0x7F0000000000            # 256-aligned, never dereferenced


def header_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:gdn_status|void|size_t|const char\*)\s+(gdn_\w+)\s*\(", txt, re.M)))


def test_header_symbols_exported():
    names = header_functions()
    assert set(names) == set(B.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (gdn_\w+)$", out, re.M))
    missing = set(names) - exported
    assert not missing, missing
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert getattr(lib, n)


def _cfg(**kw):
    d = dict(R=2, H=3, d_k=128, d_v=128, T_max=4, W_max=256, V_max=1024, io="bf16", wout="bf16")
    d.update(kw)
    return B.make_config(**d)


def _a(x):
    return (x + 255) & ~255


def expected_bytes(R, H, d_k, d_v, T, W, V, e, ew, HK=None):
    """Workspace regions as documented in include/gdn_beam.h, each 256-aligned."""
    HK = H if not HK else HK
    dvp = max(d_v, 32)
    nvg = -(-V // 128)
    Vt = -(-V // 32)                      # 32-code tiles
    nch = -(-W // 32)                     # 32-beam MFMA columns
    groups = nch + 1 + min(Vt, W)
    regions = [R * H * 4 * dvp * d_k, R * H * T * W * 4, R * H * T * W * d_v * 4,
               R * HK * T * W * d_k * e, R * W * T * 4, R * W * T * 4, R * W * T * 4, R * W * T * 4,
               R * W * 4, R * W * 4, R * W * 4, R * W * 4, R * W * 4, R * W * 4, R * W * d_v * 4, R * nch * 32 * d_v * 6, V * d_v * ew,
               R * Vt * W * 4, R * W * nvg * 16, R * W * 4, R * 16, R * Vt * W * 4, R * W * 4,
               R * groups * 4, R * groups * 32 * 4, R * W * 32 * 4, R * W * 4, 128, Vt * 4, V * d_v * 2, R * W * 4,
               64 * 4]
    return sum(_a(x) for x in regions)


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_workspace_formula(name):
    wl = synth.get(name)
    e = 2 if wl.io == "bf16" else 4
    ew = 2 if wl.wout == "bf16" else 4
    got = B.gdn_beam_workspace_bytes(B.make_config(wl.R, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V,
                                                   wl.io, wl.wout))
    assert got == expected_bytes(wl.R, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, e, ew)
    # grouped value heads: the records' keys are per key head
    g = B.gdn_beam_workspace_bytes(B.make_config(wl.R, 4 * wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V,
                                                 wl.io, wl.wout, H_K=wl.H))
    assert g == expected_bytes(wl.R, 4 * wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, e, ew, HK=wl.H)


def test_persistent_state_is_gtr_capacity_and_beats_fullstate():
    """S_ctx + GTR pool per (request, head) is the capacity form d_v d_k + W T (d_v + d_k + 1)
    in elements (OneLA reading note, section 4.3 b), and the whole workspace per request
    stays far below FullState's W d_v d_k fp32 at the stress shape."""
    wl = synth.get("stress")
    e = 2
    cap = capacity_elements(wl.d_k, wl.d_v, W=wl.W_max, T=wl.T)
    gtr_bytes = 4 * wl.d_v * wl.d_k + wl.T * wl.W_max * (4 + 4 * wl.d_v + e * wl.d_k)
    assert gtr_bytes == 4 * cap["state"] + wl.T * wl.W_max * (4 * (1 + wl.d_v) + e * wl.d_k)
    ws = B.gdn_beam_workspace_bytes(B.make_config(1, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V))
    fullstate = wl.H * wl.W_max * wl.d_v * wl.d_k * 4
    # the GDN state alone is about 20x smaller; the selection scratch (W x V / 32 tile
    # maxima) is extra
    assert wl.H * gtr_bytes * 18 < fullstate
    assert ws < fullstate


def test_workspace_does_not_grow_with_dv_dk_w():
    """Doubling W adds a term linear in W (records, scores), never W*d_v*d_k."""
    b1 = B.gdn_beam_workspace_bytes(_cfg(W_max=256))
    b2 = B.gdn_beam_workspace_bytes(_cfg(W_max=512))
    R, H, T, d, V = 2, 3, 4, 128, 1024
    records = H * T * (4 + 4 * d + 2 * d)              # GTR slots of every head
    beam_state = 4 * T * 4 + 2 * 4 + 4 * 4             # ancestry + SID prefixes, scores, order
    # z (fp32 and operand), tile maxima, lse parts, lse, kept tiles, chosen tiles,
    # groups and their tiles, refined keys
    scoring = 4 * d + 6 * d + 4 * (V // 32) + 16 * (V // 128) + 4 + 4 * (V // 32) + 4 + 4 + 128 + 128
    per_w = R * (records + beam_state + scoring)
    assert b2 - b1 <= 256 * per_w + 20 * 256
    assert b2 - b1 < 256 * 128 * 128 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(d_k=64), B.GDN_ERR_UNSUPPORTED),
    (dict(d_k=128, d_v=64), B.GDN_ERR_UNSUPPORTED),
    (dict(W_max=2048), B.GDN_ERR_CAPACITY),
    (dict(T_max=9), B.GDN_ERR_CAPACITY),
    (dict(V_max=70000), B.GDN_ERR_CAPACITY),
    (dict(R=0), B.GDN_ERR_INVALID_ARG),
    (dict(H=-1), B.GDN_ERR_INVALID_ARG),
    (dict(H=4, H_K=3), B.GDN_ERR_INVALID_ARG),
    (dict(d_k=256, d_v=256, io="f32"), B.GDN_ERR_UNSUPPORTED),
    (dict(d_k=256, d_v=128), B.GDN_ERR_UNSUPPORTED),
    (dict(d_v=512, wout="f32"), B.GDN_ERR_UNSUPPORTED),
    (dict(d_v=384), B.GDN_ERR_UNSUPPORTED),
    (dict(H_K=-2), B.GDN_ERR_INVALID_ARG),
])
def test_config_errors(kw, status):
    cfg = _cfg(**kw)
    n = ctypes.c_size_t(0)
    assert B.raw_status("gdn_beam_workspace_bytes", ctypes.byref(cfg), ctypes.byref(n)) == status
    ctx = ctypes.c_void_p()
    assert B.raw_status("gdn_beam_init", ctypes.byref(cfg), FAKE, 4, FAKE, 1 << 40, None,
                        ctypes.byref(ctx)) == status
    assert ctx.value is None


def test_bad_dtype():
    cfg = _cfg()
    cfg.io_dtype = 7
    n = ctypes.c_size_t(0)
    assert B.raw_status("gdn_beam_workspace_bytes", ctypes.byref(cfg), ctypes.byref(n)) == B.GDN_ERR_INVALID_ARG


def test_init_argument_errors():
    cfg = _cfg()
    need = B.gdn_beam_workspace_bytes(cfg)
    ctx = ctypes.c_void_p()
    st = lambda *a: B.raw_status("gdn_beam_init", ctypes.byref(cfg), *a, ctypes.byref(ctx))
    assert st(None, 4, FAKE, need, None) == B.GDN_ERR_INVALID_ARG           # null S_ctx
    assert st(FAKE + 4, 4, FAKE, need, None) == B.GDN_ERR_INVALID_ARG       # misaligned S_ctx
    assert st(FAKE, 4, FAKE + 16, need, None) == B.GDN_ERR_INVALID_ARG      # workspace not 256-aligned
    assert st(FAKE, 0, FAKE, need, None) == B.GDN_ERR_INVALID_ARG           # no beams
    assert st(FAKE, 257, FAKE, need, None) == B.GDN_ERR_CAPACITY            # W0 > W_max
    assert st(FAKE, 4, FAKE, need - 1, None) == B.GDN_ERR_WORKSPACE         # too small
    assert B.raw_status("gdn_beam_init", ctypes.byref(cfg), FAKE, 4, FAKE, need, None, None) == \
        B.GDN_ERR_INVALID_ARG                                                # no out pointer
    assert ctx.value is None


def test_null_context_calls():
    assert B.raw_status("gdn_beam_step", None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.GDN_ERR_INVALID_ARG
    assert B.raw_status("gdn_beam_select", None, 0, FAKE, FAKE, 8, 8, None, None, FAKE, FAKE, FAKE,
                        None) == B.GDN_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert B.raw_status("gdn_beam_export_bytes", None, 0, ctypes.byref(n)) == B.GDN_ERR_INVALID_ARG
    assert B.raw_status("gdn_beam_export", None, 0, FAKE, 16, None) == B.GDN_ERR_INVALID_ARG
    t, w = ctypes.c_int32(), ctypes.c_int32()
    assert B.raw_status("gdn_beam_query", None, ctypes.byref(t), ctypes.byref(w)) == B.GDN_ERR_INVALID_ARG
    B.gdn_beam_destroy(None)   # no-op


def test_step_timing_argument_errors():
    """The step-launch timer refuses a capacity out of range and missing outputs before
    any HIP call; with no timer set, reading gives nothing and releasing is a no-op."""
    f = B.raw_status
    assert f("gdn_beam_time_steps", -1) == B.GDN_ERR_INVALID_ARG
    assert f("gdn_beam_time_steps", 65537) == B.GDN_ERR_INVALID_ARG
    n = ctypes.c_int32(7)
    ms = (ctypes.c_float * 4)()
    assert f("gdn_beam_step_times", None, 4, ctypes.byref(n)) == B.GDN_ERR_INVALID_ARG   # no ms
    assert f("gdn_beam_step_times", ms, -1, ctypes.byref(n)) == B.GDN_ERR_INVALID_ARG    # cap < 0
    assert f("gdn_beam_step_times", ms, 4, None) == B.GDN_ERR_INVALID_ARG                # no n
    assert f("gdn_beam_time_steps", 0) == B.GDN_OK
    assert f("gdn_beam_step_times", None, 0, ctypes.byref(n)) == B.GDN_OK and n.value == 0


def test_stream_probe_argument_errors():
    """The streaming probe refuses null or misaligned pointers, sizes that are not whole
    16-byte units and unknown modes before any HIP call; nothing to move is a no-op."""
    f = lambda *a: B.raw_status("gdn_beam_stream_probe", *a)
    A = 1 << 20                                    # aligned host-side stand-ins, never used
    assert f(None, A, 64, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(A, None, 64, 1, None) == B.GDN_ERR_INVALID_ARG
    assert f(A + 4, A, 64, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(A, A + 8, 64, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(A, A, 60, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(A, A, 64, 3, None) == B.GDN_ERR_INVALID_ARG
    assert f(A, A, 64, -1, None) == B.GDN_ERR_INVALID_ARG
    assert f(None, None, 64, 2, None) == B.GDN_ERR_INVALID_ARG      # the write needs dst
    assert f(A + 4, None, 64, 2, None) == B.GDN_ERR_INVALID_ARG
    assert f(A, A, 0, 0, None) == B.GDN_OK


def test_prefill_argument_errors():
    f = lambda *a: B.raw_status("gdn_beam_prefill", *a)
    F6 = (FAKE,) * 6
    assert f(2, 3, 0, 64, 64, 10, *F6, None, 0, None) == B.GDN_ERR_UNSUPPORTED
    assert f(0, 3, 0, 128, 128, 10, *F6, None, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(2, 3, 0, 128, 128, 10, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(2, 3, 0, 128, 128, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(2, 3, 0, 128, 128, 10, FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(2, 3, 0, 128, 128, 1 << 31, *F6, None, 0, None) == B.GDN_ERR_CAPACITY
    # grouped value heads: H a multiple of H_K
    assert f(2, 4, 3, 128, 128, 10, *F6, None, 0, None) == B.GDN_ERR_INVALID_ARG
    assert f(2, 4, -1, 128, 128, 10, *F6, None, 0, None) == B.GDN_ERR_INVALID_ARG
    # chunked form: workspace 256-byte aligned and at least the stated size
    need = B.gdn_beam_prefill_workspace_bytes(3, 128, 128, 10)
    assert f(2, 3, 0, 128, 128, 10, *F6, FAKE + 16, need, None) == B.GDN_ERR_INVALID_ARG
    assert f(2, 3, 0, 128, 128, 10, *F6, FAKE, need - 1, None) == B.GDN_ERR_WORKSPACE


@pytest.mark.parametrize("H,d_k,d_v,N", [(3, 128, 128, 10), (16, 128, 256, 559622),
                                         (4, 256, 512, 64), (1, 128, 128, 0)])
def test_prefill_workspace_bytes(H, d_k, d_v, N):
    """One 32 x 32 chunk matrix and two 32-entry decay products (fp32) per 32-token
    block of the stacked prompts and value head."""
    blocks = -(-N // 32)
    assert B.gdn_beam_prefill_workspace_bytes(H, d_k, d_v, N) == blocks * H * (32 * 32 + 64) * 4


def test_prefill_workspace_bytes_token_form():
    """d_k = 16 has only the token-sequential form; unsupported dims need nothing."""
    assert B.gdn_beam_prefill_workspace_bytes(1, 16, 16, 64) == 0
    assert B.gdn_beam_prefill_workspace_bytes(1, 64, 64, 64) == 0


def test_status_strings():
    for s in range(7):
        assert B.gdn_beam_status_str(s)
    assert B.gdn_beam_status_str(99) == "unknown status"
    assert B.gdn_beam_last_error() == ""


def test_single_hip_runtime():
    """The library shares PyTorch's HIP runtime: exactly one libamdhip64 is mapped."""
    assert len(B._hip_runtimes()) == 1


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_fullstate_bytes_formula(name):
    """Two generations of one fp32 d_v x d_k state per (request, head, beam): the
    FullState capacity of the OneLA reading note (section 1.3, Fig. 2)."""
    wl = synth.get(name)
    cfg = B.make_config(wl.R, wl.H, wl.d_k, wl.d_v, wl.T, wl.W_max, wl.V, wl.io, wl.wout)
    assert B.gdn_fullstate_bytes(cfg) == 2 * wl.R * wl.H * wl.W_max * wl.d_v * wl.d_k * 4


def test_fullstate_argument_errors():
    n = ctypes.c_size_t(0)
    assert B.raw_status("gdn_fullstate_bytes", None, ctypes.byref(n)) == B.GDN_ERR_INVALID_ARG
    cfg = _cfg(d_k=64)
    assert B.raw_status("gdn_fullstate_bytes", ctypes.byref(cfg), ctypes.byref(n)) == B.GDN_ERR_UNSUPPORTED
    cfg = _cfg()
    assert B.raw_status("gdn_fullstate_bytes", ctypes.byref(cfg), None) == B.GDN_ERR_INVALID_ARG
    # a null context is rejected before anything touches the device
    assert B.raw_status("gdn_fullstate_step", None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, 1 << 30, None) == B.GDN_ERR_INVALID_ARG
