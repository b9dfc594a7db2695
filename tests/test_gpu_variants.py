"""GPU parity of the expert-stage and routing variants that the default
dispatch does not pick for these shapes but that a plan can be switched to
with moe_plan_set (MOE_OPT_GROUPED_TILE for the grouped path,
MOE_OPT_DEC_KERNEL / MOE_OPT_DEC_MFMA_MIN_T for the decode path,
MOE_OPT_SMALL_ROUTE_T for the routing stage): each one against the CPU
oracle with the same bars as the default path.  The shapes carry the tails
the kernels guard: K = 160 (an fp4 k-tail of 32 inputs against 64-input
stages), N = 96 and 384 (partial 128- and 256-row column blocks), 37, 70 and
150 tokens (partial tiles), and one expert holding every slot (several tiles
of one expert)."""
import numpy as np
import pytest

import synth
import mixture_experts_layer_f32_amd as moe
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


def run_with_options(opts, wl, W, batch, path):
    """Plan with the given options set (moe_plan_set), forward, outputs."""
    g, run = gpu_run(wl, W, batch, path, options=opts)
    return g


def check_all(g, ref):
    check_routing(g, ref)
    check_h(g["h"], ref.h)
    check_out(g["out"], ref.out)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
@pytest.mark.parametrize("tile", [13, 14, 15, 22, 23, 24])
def test_grouped_tiles(fmt, tile):
    """Every tile height of the grouped kernel on a batch of a few tokens per
    expert (partial tiles, chunks past the rows)."""
    wl, layer, W = get(fmt)
    T = wl.batches[0]
    batch = synth.make_batch(wl, layer, T)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_options({moe.MOE_OPT_GROUPED_TILE: tile}, wl, W, batch, GROUPED), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
@pytest.mark.parametrize("T", [2, 37])
def test_decode_matvec_kernel(fmt, T):
    """The wavefront matvec (default only for one token) on several tokens."""
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, T)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_options({moe.MOE_OPT_DEC_KERNEL: 0}, wl, W, batch, DECODE), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
def test_decode_mfma_one_token(fmt):
    """The MFMA decode tiles (default from two tokens) on a single token."""
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, 1)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_options({moe.MOE_OPT_DEC_MFMA_MIN_T: 1}, wl, W, batch, DECODE), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
@pytest.mark.parametrize("tile", [13, 14, 15, 22, 23, 24])
def test_grouped_tiles_one_expert_many_tiles(fmt, tile):
    """A large bias on expert 1 sends all 150 tokens there: at 96- and
    128-token tiles that expert spans two tiles (the last one partial), at 160
    to 256 one partial tile; the chunks of a tile are shared out between the
    wavefront rows, so many counts of active chunks per wavefront occur."""
    wl, layer, W = get(fmt)
    T = 150
    batch = synth.make_batch(wl, layer, T)
    bias = np.zeros((T, wl.E), np.float32)
    bias[:, 1] = 100.0
    batch = synth.Batch(batch.x, bias)
    ref = oracle_run(wl, layer, batch)
    assert ref.counts[1] == T
    check_all(run_with_options({moe.MOE_OPT_GROUPED_TILE: tile}, wl, W, batch, GROUPED), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "nvfp4"])
@pytest.mark.parametrize("T,tile", [(33, 24), (65, 24), (97, 24), (129, 24), (161, 24), (193, 24),
                                    (225, 24), (256, 24), (1, 15), (40, 15), (70, 15), (100, 15),
                                    (130, 15), (160, 15)])
def test_grouped_chunk_counts(fmt, T, tile):
    """One expert holding T slots in one tile: at 256-token tiles 2..8 active
    32-row chunks, so each wavefront row takes every count from 1 to 4 (and
    odd splits, where the two rows differ by one chunk); at 160-token tiles of
    one wavefront row every count from 1 to 5."""
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, T)
    bias = np.zeros((T, wl.E), np.float32)
    bias[:, 1] = 100.0
    batch = synth.Batch(batch.x, bias)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_options({moe.MOE_OPT_GROUPED_TILE: tile}, wl, W, batch, GROUPED), ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("T,path", [(17, DECODE), (37, DECODE), (64, GROUPED)])
def test_one_workgroup_routing_up_to_64_tokens(fmt, T, path):
    """Top-k and permute in one workgroup (MOE_OPT_SMALL_ROUTE_T) for 17..64 tokens:
    several row-group tiles per expert in the tile list, against the oracle."""
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, T)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_options({moe.MOE_OPT_SMALL_ROUTE_T: 64}, wl, W, batch, path), ref)


def test_one_workgroup_routing_olmoe_shape():
    """64 experts, top-8, 64 tokens (512 slots) routed in one workgroup."""
    wl = synth.WORKLOADS["olmoe-decode"]
    layer = synth.make_layer(wl)
    W = device_weights(layer)
    batch = synth.make_batch(wl, layer, 64)
    ref = oracle_run(wl, layer, batch)
    check_all(run_with_options({moe.MOE_OPT_SMALL_ROUTE_T: 64}, wl, W, batch, DECODE), ref)
