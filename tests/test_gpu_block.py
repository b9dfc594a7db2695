"""GPU parity of the steps either side of the layer in a transformer block:
the RMS normalisation feeding the router and experts, the dense (shared)
branch as a one-expert top-1 plan, and the add of routed + dense into the
bf16 residual stream; each against the CPU oracle (B1-B3)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_out, device_weights

pytestmark = pytest.mark.gpu


def bf16_bits(v):
    import torch
    return torch.tensor(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_vals(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_bf16(got, ref, min_equal=0.999):
    """GPU bf16 (f32 arithmetic) vs the float64 oracle rounded once: equal but
    for rare ties of the two roundings, never more than one bf16 step apart."""
    g, r = bf16_vals(got), bf16_vals(ref)
    step = np.maximum(np.abs(r), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(g - r) <= step), f"max diff {np.max(np.abs(g - r) / step):.2f} steps"
    assert np.mean(got == ref) >= min_equal, f"only {np.mean(got == ref):.5f} equal"


def to_dev(a):
    from mixture_experts_layer_f32_amd.device import to_dev as td
    return td(a)


@pytest.mark.parametrize("T,d", [(1, 2048), (7, 7168), (33, 4096), (3, 136), (2, 8)])
def test_rmsnorm(T, d):
    import torch
    import mixture_experts_layer_f32_amd as m
    rng = np.random.default_rng(100 + T + d)
    x = bf16_bits(rng.standard_normal((T, d)) * rng.uniform(0.1, 10.0, (T, 1)))
    gamma = bf16_bits(rng.uniform(0.5, 1.5, d))
    xn = torch.empty((T, d), dtype=torch.int16, device="cuda")
    m.moe_rmsnorm(to_dev(x), to_dev(gamma), 1e-6, xn)
    torch.cuda.synchronize()
    check_bf16(xn.cpu().numpy().view(np.uint16), oracle.rmsnorm(x, gamma, 1e-6))


def test_rmsnorm_zero_row_and_eps():
    import torch
    import mixture_experts_layer_f32_amd as m
    x = np.zeros((2, 64), np.uint16)
    x[1] = bf16_bits(np.full(64, 2.0))
    gamma = bf16_bits(np.ones(64))
    xn = torch.empty((2, 64), dtype=torch.int16, device="cuda")
    m.moe_rmsnorm(to_dev(x), to_dev(gamma), 4.0, xn)
    torch.cuda.synchronize()
    got = xn.cpu().numpy().view(np.uint16)
    assert np.all(got[0] == 0)
    assert np.array_equal(got, oracle.rmsnorm(x, gamma, 4.0))


@pytest.mark.parametrize("dense", [False, True])
def test_residual_add(dense):
    import torch
    import mixture_experts_layer_f32_amd as m
    rng = np.random.default_rng(7 if dense else 8)
    T, d = 5, 2048
    res = bf16_bits(rng.standard_normal((T, d)) * 4.0)
    a = rng.standard_normal((T, d)).astype(np.float32)
    b = rng.standard_normal((T, d)).astype(np.float32) if dense else None
    out = torch.empty((T, d), dtype=torch.int16, device="cuda")
    m.moe_residual_add(to_dev(res), to_dev(a), to_dev(b) if dense else None, out)
    torch.cuda.synchronize()
    check_bf16(out.cpu().numpy().view(np.uint16), oracle.residual_add(res, a, b))


def test_residual_add_in_place():
    """out may be the residual buffer itself."""
    import torch
    import mixture_experts_layer_f32_amd as m
    rng = np.random.default_rng(9)
    res = bf16_bits(rng.standard_normal((3, 256)))
    a = rng.standard_normal((3, 256)).astype(np.float32)
    buf = to_dev(res)
    m.moe_residual_add(buf, to_dev(a), None, buf)
    torch.cuda.synchronize()
    check_bf16(buf.cpu().numpy().view(np.uint16), oracle.residual_add(res, a))


ROUTED = synth.WORKLOADS["olmoe-decode"]
DENSE = synth.Workload("olmoe-dense", 2048, 1024, 1, 1, "e4m3", True, (), False, 1101)
_cache = {}


def layers():
    if not _cache:
        for wl in (ROUTED, DENSE):
            L = synth.make_layer(wl)
            _cache[wl.name] = (L, device_weights(L))
    return _cache[ROUTED.name], _cache[DENSE.name]


@pytest.mark.parametrize("T", [1, 8, 100, 300])
def test_block_forward(T):
    """x -> RMSNorm -> routed layer + dense branch (a one-expert top-1 plan) ->
    add into the residual stream, every step against the oracle.  1 and 8
    tokens take the decode path, 100 and 300 the grouped one (the dense
    branch's 300 rows span several tiles)."""
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import Runner
    (L, W), (LD, WD) = layers()
    x = synth.make_batch(ROUTED, L, T).x
    rng = np.random.default_rng(T)
    gamma = bf16_bits(rng.uniform(0.5, 1.5, ROUTED.d))
    eps = 1e-6
    xn = torch.empty((T, ROUTED.d), dtype=torch.int16, device="cuda")
    m.moe_rmsnorm(to_dev(x), to_dev(gamma), eps, xn)
    routed = Runner(ROUTED.d, ROUTED.f, ROUTED.E, ROUTED.k, ROUTED.fmt, ROUTED.renorm, T)
    r_out = routed.outputs(T)
    routed.forward(W, xn, None, r_out)
    dense = Runner(DENSE.d, DENSE.f, 1, 1, DENSE.fmt, True, T)
    d_out = dense.outputs(T)
    dense.forward(WD, xn, None, d_out)
    blk = torch.empty((T, ROUTED.d), dtype=torch.int16, device="cuda")
    m.moe_residual_add(to_dev(x), r_out["out"], d_out["out"], blk)
    torch.cuda.synchronize()

    xn_g = xn.cpu().numpy().view(np.uint16)
    check_bf16(xn_g, oracle.rmsnorm(x, gamma, eps), min_equal=0.998)
    # the layers on the GPU's normed input (routing must see the same bits)
    M = lambda q: oracle.Mat(q.q, q.s, q.K)  # noqa: E731
    ref_r = oracle.moe_forward(xn_g, L.w_router, None, M(L.gate), M(L.up), M(L.down), ROUTED.k,
                               ROUTED.renorm, ROUTED.fmt)
    assert np.array_equal(r_out["topk_ids"].cpu().numpy(), ref_r.ids)
    check_out(r_out["out"].cpu().numpy(), ref_r.out)
    ref_d = oracle.moe_forward(xn_g, LD.w_router, None, M(LD.gate), M(LD.up), M(LD.down), 1, True,
                               DENSE.fmt)
    # one expert, top-1: identity routing with weight exactly 1, no router or combine
    assert np.all(d_out["topk_w"].cpu().numpy() == 1.0)
    assert np.all(d_out["topk_ids"].cpu().numpy() == 0)
    assert np.array_equal(d_out["perm"].cpu().numpy(), np.arange(T))
    assert np.array_equal(d_out["counts"].cpu().numpy(), [T])
    assert np.array_equal(d_out["offsets"].cpu().numpy(), [0, T])
    check_out(d_out["out"].cpu().numpy(), ref_d.out)
    # the add: the oracle's sum of its own layer outputs, so the bound is the
    # layers' tolerance plus one bf16 step
    ref_b = oracle.residual_add(x, ref_r.out, ref_d.out)
    g, r = bf16_vals(blk.cpu().numpy().view(np.uint16)), bf16_vals(ref_b)
    s = ref_r.out.astype(np.float64) + ref_d.out
    tol = 2e-2 * np.sqrt(np.mean(s * s)) + np.abs(r) * 2.0 ** -7
    assert np.all(np.abs(g - r) <= tol)
