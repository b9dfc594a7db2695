"""Full-size parity, NVFP4 expert layer: the FP4 layer's shape (d=4096,
f=2880, 384 experts, top-6 renormalised) with e2m1 codes and one e4m3 scale
per 16 inputs (19.9 MB per expert), at 1, 16 and 1024 tokens.  Routing (ids,
counts, offsets, permutation) is compared bit for bit over every token; the
outputs of a seeded sample of tokens are compared with the oracle, which
evaluates those tokens one by one."""
import numpy as np
import pytest

import synth
from gpu_util import check_out, check_routing, device_weights, gpu_run, log, oracle_run

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["fp4-nvfp4"]


@pytest.fixture(scope="module")
def layer():
    log("generating fp4-nvfp4 layer (7.6 GB)")
    L = synth.make_layer(WL)
    log("uploading")
    W = device_weights(L)
    yield L, W
    del W


def sample_tokens(T, n=6):
    if T <= n:
        return list(range(T))
    rng = np.random.default_rng(T)
    return sorted({0, T - 1, *rng.choice(T, n - 2, replace=False).tolist()})


@pytest.mark.parametrize("T,path", [(1, 0), (16, 0), (1024, 0), (16, 2), (1024, 2)])
def test_fp4_nvfp4(layer, T, path):
    L, W = layer
    batch = synth.make_batch(WL, L, T)
    toks = sample_tokens(T)
    log(f"fp4-nvfp4 T={T} path={path}: oracle on tokens {toks}")
    ref = oracle_run(WL, L, batch, tokens=toks)
    log("gpu")
    g, run = gpu_run(WL, W, batch, path)
    check_routing(g, ref)
    mx, rms, mrel = check_out(g["out"][toks], ref.out)
    log(f"max|err| {mx:.3e} rms {rms:.3e} mean rel {mrel:.3e}")
