"""The C-ABI library on the host: it loads, exports every function that
include/moe.h declares, and rejects bad layer descriptors before touching a
device (no compute calls here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    import mixture_experts_layer_f32_amd as m
    names = declared_functions()
    assert {"moe_plan", "moe_forward", "moe_workspace_size", "moe_plan_free", "moe_status_str",
            "moe_plan_info"} <= set(names)
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings():
    import mixture_experts_layer_f32_amd as m
    assert m.moe_status_str(0) == "MOE_OK"
    assert m.moe_status_str(m.MOE_ERR_WORKSPACE) == "MOE_ERR_WORKSPACE"
    assert m.moe_status_str(99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("fields,status", [
    (dict(d_model=0), 2), (dict(top_k=9), 2), (dict(max_tokens=0), 2), (dict(renorm=2), 2),
    (dict(path=5), 2), (dict(n_experts=2048, top_k=2), 3), (dict(top_k=17, n_experts=64), 3),
    (dict(d_model=200), 3), (dict(d_ff=96), 3), (dict(wfmt=7), 3),
    (dict(wfmt=1, d_model=48), 3), (dict(wfmt=1, d_ff=80), 3),
    (dict(wfmt=2, d_model=48), 3), (dict(wfmt=2, d_ff=80), 3), (dict(wfmt=3), 3),
    # the activation-quantised variant: unknown act_fmt; NVFP4 weights; e2m1
    # dims that are multiples of 32 but not of 64
    (dict(act_fmt=2), 2), (dict(act_fmt=-1), 2), (dict(act_fmt=1, wfmt=2), 3),
    (dict(act_fmt=1, wfmt=1, d_model=160), 3), (dict(act_fmt=1, wfmt=1, d_ff=96), 3),
])
def test_descriptor_validation_before_device(fields, status):
    import mixture_experts_layer_f32_amd as m
    base = dict(d_model=256, d_ff=256, n_experts=8, top_k=2, max_tokens=4, wfmt=0, renorm=1,
                path=0, act_fmt=0)
    base.update(fields)
    assert m.moe_plan_status(m.moe_desc(**base)) == status


def test_plan_needs_gfx950_device():
    import torch
    import mixture_experts_layer_f32_amd as m
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present; covered by the GPU tests")
    d = m.moe_desc(256, 256, 8, 2, 4, 0, 1, 0)
    assert m.moe_plan_status(d) == m.MOE_ERR_DEVICE


def test_null_plan_queries():
    import mixture_experts_layer_f32_amd as m
    assert m.lib.moe_workspace_size(None, 4) == 0
    assert m.lib.moe_workspace_h_offset(None, 4) == -1
    assert m.lib.moe_plan_path(None, 4) == -1
    assert m.lib.moe_plan_info(None) == b""
    m.lib.moe_plan_free(None)


def test_block_step_argument_errors_before_launch():
    """moe_rmsnorm / moe_residual_add check every argument before launching
    (these calls never reach a launch, so they need no device)."""
    import mixture_experts_layer_f32_amd as m
    L = m.lib
    A = 1 << 20  # a 16-byte-aligned address that is never dereferenced
    assert L.moe_rmsnorm(0, 2048, None, None, 1e-6, None, None) == m.MOE_OK
    assert L.moe_rmsnorm(-1, 2048, A, A, 1e-6, A, None) == m.MOE_ERR_BAD_SHAPE
    assert L.moe_rmsnorm(4, 0, A, A, 1e-6, A, None) == m.MOE_ERR_BAD_SHAPE
    assert L.moe_rmsnorm(4, 12, A, A, 1e-6, A, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_rmsnorm(4, 16, A, A, -1.0, A, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_rmsnorm(4, 16, None, A, 1e-6, A, None) == m.MOE_ERR_NULL_ARG
    assert L.moe_rmsnorm(4, 16, A + 2, A, 1e-6, A, None) == m.MOE_ERR_ALIGNMENT
    assert L.moe_residual_add(0, 64, None, None, None, None, None) == m.MOE_OK
    assert L.moe_residual_add(4, 6, A, A, None, A, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_residual_add(4, 64, A, None, None, A, None) == m.MOE_ERR_NULL_ARG
    assert L.moe_residual_add(4, 64, A, A + 8, None, A, None) == m.MOE_ERR_ALIGNMENT
    assert L.moe_residual_add(4, 64, A, A, A + 4, A, None) == m.MOE_ERR_ALIGNMENT


def test_act_quant_argument_errors_before_launch():
    """moe_act_quant checks its arguments before launching (no device here:
    only calls that must fail, or return early, are made)."""
    import mixture_experts_layer_f32_amd as m
    L = m.lib
    A = 1 << 20   # a 16-byte aligned host-side stand-in; never dereferenced
    assert L.moe_act_quant(-1, 128, A, A, A, None) == m.MOE_ERR_BAD_SHAPE
    assert L.moe_act_quant(4, 0, A, A, A, None) == m.MOE_ERR_BAD_SHAPE
    assert L.moe_act_quant(4, 100, A, A, A, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_act_quant(0, 128, None, None, None, None) == m.MOE_OK
    assert L.moe_act_quant(4, 128, None, A, A, None) == m.MOE_ERR_NULL_ARG
    assert L.moe_act_quant(4, 128, A, A, None, None) == m.MOE_ERR_NULL_ARG
    assert L.moe_act_quant(4, 128, A + 8, A, A, None) == m.MOE_ERR_ALIGNMENT
    assert L.moe_act_quant(4, 128, A, A + 4, A, None) == m.MOE_ERR_ALIGNMENT
