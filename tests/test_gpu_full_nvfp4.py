"""Full-size parity, NVFP4 expert layer (the Qwen-Flash-Next post's expert
shape): d=2560, f=640, 512 experts, top-10 renormalised, e2m1 codes with one
e4m3 scale per 16 inputs (2.64 MiB per expert), at 1, 16 and 256 tokens.
Routing (ids, counts, offsets, permutation) is compared bit for bit over
every token; the outputs of a seeded sample of tokens are compared with the
oracle, which evaluates those tokens one by one."""
import numpy as np
import pytest

import synth
from gpu_util import check_out, check_routing, device_weights, gpu_run, log, oracle_run

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["nvfp4-qwen"]


@pytest.fixture(scope="module")
def layer():
    log("generating nvfp4-qwen layer (1.4 GB)")
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


@pytest.mark.parametrize("T,path", [(1, 0), (16, 0), (256, 0), (16, 2), (256, 2)])
def test_nvfp4_qwen(layer, T, path):
    L, W = layer
    batch = synth.make_batch(WL, L, T)
    toks = sample_tokens(T)
    log(f"nvfp4-qwen T={T} path={path}: oracle on tokens {toks}")
    ref = oracle_run(WL, L, batch, tokens=toks)
    log("gpu")
    g, run = gpu_run(WL, W, batch, path)
    check_routing(g, ref)
    mx, rms, mrel = check_out(g["out"][toks], ref.out)
    log(f"max|err| {mx:.3e} rms {rms:.3e} mean rel {mrel:.3e}")
