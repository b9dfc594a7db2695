"""Full-size parity, FP4 expert layer (DeepSeek-V4.1-Flash sizes): d=4096,
f=2880, 384 experts, top-6 renormalised, e2m1 with UE8M0 scales per 32
(17.93 MiB per expert), at 1, 16 and 1024 tokens.  Routing (ids,
counts, offsets, permutation) is compared bit for bit over every token; the
outputs of a seeded sample of tokens are compared with the oracle, which
evaluates those tokens one by one."""
import numpy as np
import pytest

import synth
from gpu_util import check_out, check_routing, device_weights, gpu_run, log, oracle_run

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["fp4-e2m1"]


@pytest.fixture(scope="module")
def layer():
    log("generating fp4-e2m1 layer (7.2 GB)")
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


@pytest.mark.parametrize("T,path", [(1, 0), (16, 0), (1024, 0), (1, 2), (16, 2)])
def test_fp4_e2m1(layer, T, path):
    L, W = layer
    batch = synth.make_batch(WL, L, T)
    toks = sample_tokens(T)
    log(f"fp4-e2m1 T={T} path={path}: oracle on tokens {toks}")
    ref = oracle_run(WL, L, batch, tokens=toks)
    log("gpu")
    g, run = gpu_run(WL, W, batch, path)
    check_routing(g, ref)
    mx, rms, mrel = check_out(g["out"][toks], ref.out)
    log(f"max|err| {mx:.3e} rms {rms:.3e} mean rel {mrel:.3e}")


@pytest.mark.parametrize("T", [16, 1024])
def test_fp4_e2m1_act_quant(layer, T):
    """The activation-quantised variant (x and h as e4m3 per 128-input group)
    at full size: routing bit-exact, sampled outputs against the oracle's own
    quantised layer."""
    import oracle
    from gpu_util import omat
    from test_gpu_actquant import check_h_q8, q8_reference, run_q8
    L, W = layer
    batch = synth.make_batch(WL, L, T)
    toks = sample_tokens(T)
    log(f"{WL.name} act-quant T={T}: routing by the oracle")
    ref = oracle.moe_forward(batch.x, L.w_router, batch.bias, omat(L.gate), omat(L.up), omat(L.down),
                             WL.k, WL.renorm, WL.fmt, tokens=[], act_quant=True)
    log("gpu")
    g = run_q8(WL, W, batch)
    check_routing(g, ref)
    log(f"oracle steps for tokens {toks}")
    h_ref, out_ref = q8_reference(WL, L, batch, ref, g["h"], toks)
    pos = ref.inv_perm.reshape(T, WL.k)[toks]
    check_h_q8(g["h"][pos.reshape(-1)], h_ref.reshape(-1, WL.f))
    mx, rms, mrel = check_out(g["out"][toks], out_ref)
    log(f"max|err| {mx:.3e} rms {rms:.3e} mean rel {mrel:.3e}")
