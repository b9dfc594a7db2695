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


# ---------------------------------------------------------------- fused block
# moe_forward_block: the shared expert's rows ride in the routed experts'
# launches and the combine adds them and the residual.  Shared-expert weights
# are a one-expert layer of the routed experts' shape and format.

FUSED = {
    "e4m3": (ROUTED, DENSE),
    "e2m1": (synth.Workload("blk-e2m1", 192, 320, 8, 3, "e2m1", True, (), False, 1102),
             synth.Workload("blk-e2m1-sh", 192, 320, 1, 1, "e2m1", True, (), False, 1103)),
    "nvfp4": (synth.Workload("blk-nvfp4", 512, 288, 8, 2, "nvfp4", False, (), False, 1104),
              synth.Workload("blk-nvfp4-sh", 512, 288, 1, 1, "nvfp4", True, (), False, 1105)),
}
_fcache = {}


def fused_layers(fmt):
    if fmt not in _fcache:
        wl, swl = FUSED[fmt]
        if fmt == "e4m3":
            (L, W), (LS, WS) = layers()
        else:
            L, LS = synth.make_layer(wl), synth.make_layer(swl)
            W, WS = device_weights(L), device_weights(LS)
        _fcache[fmt] = (wl, L, W, LS, WS)
    return _fcache[fmt]


def run_fused(fmt, T, path, act_fmt=0, in_place=False, keep_f32=True):
    """x -> moe_forward_block(shared expert, residual = x) on the GPU, and the
    oracle's routed layer and shared expert on the same input."""
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import Runner
    wl, L, W, LS, WS = fused_layers(fmt)
    x = synth.make_batch(wl, L, T).x
    rng = np.random.default_rng(1000 + T)
    res = bf16_bits(rng.standard_normal((T, wl.d)) * 2.0)
    runner = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T, path, act_fmt=act_fmt,
                    shared_expert=True)
    outs = runner.outputs(T)
    if not keep_f32:
        del outs["out"]
    xd, rd = to_dev(x), to_dev(res)
    ob = rd if in_place else torch.empty((T, wl.d), dtype=torch.int16, device="cuda")
    runner.forward_block(W, WS, xd, None, rd, ob, outs)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in outs.items()}
    got["out_bf16"] = ob.cpu().numpy().view(np.uint16)
    got["path"] = m.moe_plan_path(runner.plan, T)
    aq = act_fmt != 0
    M = lambda q: oracle.Mat(q.q, q.s, q.K)  # noqa: E731
    ref_r = oracle.moe_forward(x, L.w_router, None, M(L.gate), M(L.up), M(L.down), wl.k,
                               wl.renorm, wl.fmt, act_quant=aq)
    # the shared expert alone: a one-expert top-1 layer (weight exactly 1)
    ref_s = oracle.moe_forward(x, LS.w_router, None, M(LS.gate), M(LS.up), M(LS.down), 1, True,
                               wl.fmt, act_quant=aq)
    return got, ref_r, ref_s, res


def check_fused(got, ref_r, ref_s, res, aq=False):
    from gpu_util import check_out_actq
    assert np.array_equal(got["topk_ids"], ref_r.ids)
    s = ref_r.out.astype(np.float64) + ref_s.out
    if "out" in got:
        (check_out_actq if aq else check_out)(got["out"], s)
    # the bf16 sum: the layers' tolerance plus one bf16 step of the result
    ref_b = oracle.residual_add(res, ref_r.out, ref_s.out)
    g, r = bf16_vals(got["out_bf16"]), bf16_vals(ref_b)
    bar = (1e-1 if aq else 2e-2) * np.sqrt(np.mean(s * s))
    assert np.all(np.abs(g - r) <= bar + np.abs(r) * 2.0 ** -7)
    assert np.all(np.isfinite(g))


@pytest.mark.parametrize("fmt,T,path", [
    ("e4m3", 1, 0), ("e4m3", 8, 0), ("e4m3", 33, 1), ("e4m3", 33, 2), ("e4m3", 100, 0),
    ("e4m3", 300, 0), ("e2m1", 5, 1), ("e2m1", 70, 2), ("nvfp4", 9, 1), ("nvfp4", 130, 2)])
def test_fused_block(fmt, T, path):
    """The shared expert inside the routed launches and the residual add in
    the combine, against the oracle's routed layer plus shared expert; both
    expert paths and every weight format."""
    got, ref_r, ref_s, res = run_fused(fmt, T, path)
    if path:
        assert got["path"] == path
    check_fused(got, ref_r, ref_s, res)


def test_fused_block_matches_unfused():
    """The routed part of the fused forward equals the routed-only plan's
    (same tiles and kernels for the routed rows): out - routed is the shared
    expert's output, within the layer bars."""
    import torch
    from mixture_experts_layer_f32_amd.device import Runner
    wl, L, W, LS, WS = fused_layers("e4m3")
    T = 40
    got, ref_r, ref_s, res = run_fused("e4m3", T, 2)
    r = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T, 2)
    o = r.outputs(T)
    r.forward(W, to_dev(synth.make_batch(wl, L, T).x), None, o)
    torch.cuda.synchronize()
    assert np.array_equal(o["topk_ids"].cpu().numpy(), got["topk_ids"])
    assert np.array_equal(o["perm"].cpu().numpy(), got["perm"])
    check_out(got["out"] - o["out"].cpu().numpy(), ref_s.out)


def test_fused_block_in_place_and_bf16_only():
    """out_bf16 may be the residual buffer itself, and the f32 out may be left out."""
    got, ref_r, ref_s, res = run_fused("e4m3", 8, 0, in_place=True, keep_f32=False)
    assert "out" not in got
    check_fused(got, ref_r, ref_s, res)


@pytest.mark.parametrize("T,path", [(8, 1), (100, 2)])
def test_fused_block_act_quant(T, path):
    """The activation-quantised layer with a shared expert: x and h quantised
    as for the routed experts, against the oracle's own quantised layer."""
    got, ref_r, ref_s, res = run_fused("e4m3", T, path, act_fmt=1)
    check_fused(got, ref_r, ref_s, res, aq=True)


def test_fused_block_argument_errors():
    """The shared matrices exactly when the plan has a shared expert; residual
    and out_bf16 together; a plan without a shared expert still takes the
    residual add."""
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import Runner
    wl, L, W, LS, WS = fused_layers("e4m3")
    T = 4
    x = to_dev(synth.make_batch(wl, L, T).x)
    res = to_dev(bf16_bits(np.ones((T, wl.d))))
    ob = torch.empty((T, wl.d), dtype=torch.int16, device="cuda")
    sh = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T, shared_expert=True)
    outs = sh.outputs(T)
    g, u, dn = W.mats()
    with pytest.raises(m.MoeError) as e:  # the plan has a shared expert, no matrices given
        m.moe_forward_block(sh.plan, T, x, W.w_router, None, g, u, dn, None, res, ob,
                            outs["out"], workspace=sh.workspace)
    assert e.value.status == m.MOE_ERR_NULL_ARG
    with pytest.raises(m.MoeError) as e:  # moe_forward has no place for them
        m.moe_forward(sh.plan, T, x, W.w_router, None, g, u, dn, outs["out"],
                      workspace=sh.workspace)
    assert e.value.status == m.MOE_ERR_NULL_ARG
    with pytest.raises(m.MoeError) as e:  # residual without out_bf16
        m.moe_forward_block(sh.plan, T, x, W.w_router, None, g, u, dn, WS.mats(), res, None,
                            outs["out"], workspace=sh.workspace)
    assert e.value.status == m.MOE_ERR_NULL_ARG
    # no shared expert: the residual add alone, against the routed layer
    plain = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T)
    po = plain.outputs(T)
    with pytest.raises(m.MoeError) as e:
        m.moe_forward_block(plain.plan, T, x, W.w_router, None, g, u, dn, WS.mats(), res, ob,
                            po["out"], workspace=plain.workspace)
    assert e.value.status == m.MOE_ERR_NULL_ARG
    m.moe_forward_block(plain.plan, T, x, W.w_router, None, g, u, dn, None, res, ob, po["out"],
                        workspace=plain.workspace)
    torch.cuda.synchronize()
    want = oracle.residual_add(bf16_bits(np.ones((T, wl.d))), po["out"].cpu().numpy())
    check_bf16(ob.cpu().numpy().view(np.uint16), want)
    with pytest.raises(m.MoeError) as e:  # a shared expert on a one-expert top-1 plan
        m.moe_plan(wl.d, wl.f, 1, 1, T, wl.fmt, True, shared_expert=True)
    assert e.value.status == m.MOE_ERR_UNSUPPORTED
