"""Resources of built kernels, read from the gfx950 device object's kernel descriptors.

The chunk kernel of the chunked prefill keeps the next blocks' operands in register
arrays that its staging lambdas capture by reference.  When one of those lambdas was
left out of line the arrays went to scratch memory: every load of the pipeline then
passed through a scratch store and a full wait, and the d_v = 128 form took twice as
long with unchanged results.  These tests catch that from the build alone.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_beam_amd")
DEV_OBJ = os.path.join(PKG, "_build", "gdn_prefill.gfx950.o")


def _resources():
    if not os.path.exists(DEV_OBJ):
        pytest.skip("gdn_prefill.gfx950.o is not built (run the package build first)")
    sys.path.insert(0, PKG)
    try:
        import build
    finally:
        sys.path.remove(PKG)
    return build.kernel_resources(DEV_OBJ)


def _chunk(res, d_k, d_v):
    name = f"_ZN3gdn12chunk_kernelILi{d_k}ELi{d_v}EEEvNS_11PrefillArgsE"
    assert name in res, sorted(res)
    return res[name]


def test_chunk_kernel_d_k_128_keeps_its_pipeline_out_of_scratch():
    res = _resources()
    # eight waves (d_v >= 256): no scratch at all
    for d_v in (256, 512):
        assert _chunk(res, 128, d_v)[1] == 0, (d_v, _chunk(res, 128, d_v))
    # four waves (d_v = 128): a few spilled words outside the main loop; the scratch
    # staging of the load registers took 192 bytes per lane
    assert _chunk(res, 128, 128)[1] <= 32, _chunk(res, 128, 128)


def test_prefill_kernels_use_no_static_lds_beyond_the_preparation():
    res = _resources()
    # the chunk kernel's LDS is dynamic (two buffers sized at launch); the preparation
    # kernel's is static: alpha, beta and the columns of L
    for d_k, d_v in ((128, 128), (128, 256)):
        assert _chunk(res, d_k, d_v)[0] == 0
    prep = res["_ZN3gdn17chunk_prep_kernelILi128EEEvNS_11PrefillArgsE"]
    assert prep[0] == 4 * (32 + 32 + 32 * 2 * 20), prep


STEP_OBJ = os.path.join(PKG, "_build", "gdn_step.gfx950.o")
SELECT_OBJ = os.path.join(PKG, "_build", "gdn_select.gfx950.o")


def _resources_of(path):
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} is not built (run the package build first)")
    sys.path.insert(0, PKG)
    try:
        import build
    finally:
        sys.path.remove(PKG)
    return build.kernel_resources(path)


def _step(res, d_k, d_v, bf16, tt):
    name = f"_ZN3gdn11step_kernelILi{d_k}ELi{d_v}ELb{int(bf16)}ELi{tt}EEEvNS_5StepKE"
    assert name in res, name
    return res[name][1]


def test_step_kernels_use_no_scratch_where_the_workloads_run():
    res = _resources_of(STEP_OBJ)
    dims = [(16, 16), (128, 128), (128, 256), (128, 512), (256, 256), (256, 512)]
    # bf16 io up to t = 3 (the measured workloads replay at most three records)
    for d_k, d_v in dims:
        for tt in range(4):
            assert _step(res, d_k, d_v, True, tt) == 0, (d_k, d_v, tt)
    # d_k = 256 runs 128 state rows per workgroup from t = 1 on: no scratch up to t = 6
    for d_v in (256, 512):
        for tt in range(7):
            assert _step(res, 256, d_v, True, tt) == 0, (256, d_v, tt)
    # fp32 io (d_k <= 128) up to t = 2
    for d_k, d_v in dims[:4]:
        for tt in range(3):
            assert _step(res, d_k, d_v, False, tt) == 0, (d_k, d_v, tt)


def test_selection_kernels_keep_their_loops_out_of_scratch():
    res = _resources_of(SELECT_OBJ)
    scratch = {name: v[1] for name, v in res.items()}
    for name, s in scratch.items():
        if "logits_kernelILi512ELb0" in name:
            continue                      # an fp32 codebook is refused above d_v = 256
        if "logits_kernelILi256ELb1" in name:
            assert s <= 40, (name, s)     # setup values, stored and reloaded outside the stage loop
        elif "tile_select_kernelILb1" in name:
            assert s <= 64, (name, s)     # a few uniform values of the bounded pass
        else:
            assert s == 0, (name, s)
    assert any("logits_kernelILi128ELb1" in n for n in scratch)
