"""GPU parity of the expert-stage kernels that the default dispatch does not
pick for these shapes but that a plan can be switched to (MOE_GEMM and
MOE_BIG_CFG for the grouped path, MOE_DEC_KERNEL / MOE_DEC_MFMA_MIN_T for the
decode path): each
one against the CPU oracle with the same bars as the default path.  The
shapes carry the tails the kernels guard: K = 160 (an fp4 k-tail of 32
inputs against 64-input stages), N = 96 and 384 (partial 128- and 256-row
column blocks), 37 and 70 tokens (partial 64-token tiles), and one expert
holding every slot (several 64-token tiles of one expert)."""
import os

import numpy as np
import pytest

import synth
from gpu_util import check_h, check_out, check_routing, device_weights, gpu_run, oracle_run

pytestmark = pytest.mark.gpu

DECODE, GROUPED = 1, 2

WLS = {
    "e4m3": synth.Workload("var-e4m3", 256, 384, 6, 2, "e4m3", False, (37,), False, 5001),
    "e2m1": synth.Workload("var-e2m1", 160, 96, 8, 3, "e2m1", True, (70,), False, 5002),
    "nvfp4": synth.Workload("var-nvfp4", 160, 96, 8, 3, "nvfp4", True, (70,), False, 5003),
}
_cache = {}


def get(fmt):
    if fmt not in _cache:
        wl = WLS[fmt]
        layer = synth.make_layer(wl)
        _cache[fmt] = (wl, layer, device_weights(layer))
    return _cache[fmt]


def run_with_env(env, wl, W, batch, path):
    """Plan, forward and outputs with the given tuning switches set while the
    plan is made (moe_plan reads them)."""
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        g, run = gpu_run(wl, W, batch, path)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return g


def check_all(g, ref):
    check_routing(g, ref)
    check_h(g["h"], ref.h)
    check_out(g["out"], ref.out)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
@pytest.mark.parametrize("gemm", ["0", "1", "2", "3"])
def test_grouped_kernels(fmt, gemm):
    wl, layer, W = get(fmt)
    T = wl.batches[0]
    batch = synth.make_batch(wl, layer, T)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_env({"MOE_GEMM": gemm}, wl, W, batch, GROUPED), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
@pytest.mark.parametrize("gemm", ["0", "1", "2", "3"])
def test_grouped_kernels_one_expert_many_tiles(fmt, gemm):
    """A large bias on expert 1 sends all 150 tokens there: that expert spans
    three 64-token tiles (the last one partial), the others share the rest."""
    wl, layer, W = get(fmt)
    T = 150
    batch = synth.make_batch(wl, layer, T)
    bias = np.zeros((T, wl.E), np.float32)
    bias[:, 1] = 100.0
    batch = synth.Batch(batch.x, bias)
    ref = oracle_run(wl, layer, batch)
    assert ref.counts[1] == T
    check_all(run_with_env({"MOE_GEMM": gemm}, wl, W, batch, GROUPED), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
@pytest.mark.parametrize("T", [2, 37])
def test_decode_matvec_kernel(fmt, T):
    """The wavefront matvec (default only for one token) on several tokens."""
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, T)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_env({"MOE_DEC_KERNEL": "0"}, wl, W, batch, DECODE), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
def test_decode_mfma_one_token(fmt):
    """The MFMA decode tiles (default from two tokens) on a single token."""
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, 1)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_env({"MOE_DEC_MFMA_MIN_T": "1"}, wl, W, batch, DECODE), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
@pytest.mark.parametrize("cfg", ["11", "12", "22", "23", "24"])
def test_big_tile_shapes(fmt, cfg):
    """Every tile shape of the default grouped kernel (MOE_GEMM=3): 32 x 256,
    64 x 256, 128 x 128, 192 x 128 and 256 x 128 tokens x rows per matrix, on
    the one-expert batch (one expert spans several tiles of the small shapes)."""
    wl, layer, W = get(fmt)
    T = 150
    batch = synth.make_batch(wl, layer, T)
    bias = np.zeros((T, wl.E), np.float32)
    bias[:, 1] = 100.0
    batch = synth.Batch(batch.x, bias)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_env({"MOE_GEMM": "3", "MOE_BIG_CFG": cfg}, wl, W, batch, GROUPED), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("T,path", [(17, DECODE), (37, DECODE), (64, GROUPED)])
def test_one_workgroup_routing_up_to_64_tokens(fmt, T, path):
    """Top-k and permute in one workgroup (MOE_SMALL_ROUTE_T) for 17..64 tokens:
    several row-group tiles per expert in the tile list, against the oracle."""
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, T)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_env({"MOE_SMALL_ROUTE_T": "64"}, wl, W, batch, path), ref)


def test_one_workgroup_routing_olmoe_shape():
    """64 experts, top-8, 64 tokens (512 slots) routed in one workgroup."""
    wl = synth.WORKLOADS["olmoe-decode"]
    layer = synth.make_layer(wl)
    W = device_weights(layer)
    batch = synth.make_batch(wl, layer, 64)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_env({"MOE_SMALL_ROUTE_T": "64"}, wl, W, batch, DECODE), ref)
