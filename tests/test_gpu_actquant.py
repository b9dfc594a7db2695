"""GPU parity of the activation-quantised variant (MOE_ACT_E4M3_G128) against
the oracle's Q1-Q2: the quantiser bit for bit (codes and scale bytes, over
zero groups, values far below their group's maximum, negative zeros and rows
whose length is not a multiple of 128), and the whole layer with x and h
quantised, on e4m3 and e2m1 weights, every tile height of the block-scaled
GEMM, with k-tails (e2m1: K = 192 and 320, a 64-input last group), partial
column blocks and one expert spanning several tiles.  Routing is bit-exact.
out is checked twice: end to end against the oracle's own quantised layer
(on the decode route, whose bf16 MFMA sums the exact quantised values, at the
default bars; on the grouped path, whose fp8 MFMA rounds inside, at the
variant's own bars, derived in gpu_util), and step by step against the
oracle's down projection fed the GPU's own h at the default bars."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (check_h, check_out, check_out_actq, check_routing, device_weights, log,
                      omat)

pytestmark = pytest.mark.gpu

DECODE, GROUPED = 1, 2

WLS = {
    "e4m3": synth.Workload("aq-e4m3", 256, 384, 6, 2, "e4m3", False, (37,), False, 5101),
    "e2m1": synth.Workload("aq-e2m1", 192, 320, 8, 3, "e2m1", True, (70,), False, 5102),
}
_cache = {}


def get(fmt):
    if fmt not in _cache:
        wl = WLS[fmt]
        layer = synth.make_layer(wl)
        _cache[fmt] = (wl, layer, device_weights(layer))
    return _cache[fmt]


def bf16_bits(v):
    import torch
    return torch.tensor(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("R,K", [(37, 320), (5, 2880), (3, 7168), (64, 8), (1, 128)])
def test_act_quant_bit_exact(R, K):
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import to_dev
    rng = np.random.default_rng(R * 1000 + K)
    x = rng.standard_normal((R, K)) * np.ldexp(1.0, rng.integers(-40, 40, (R, 1)))
    x[0, : min(K, 128)] = 0.0                        # an all-zero group
    x[-1, ::5] *= 1e-5                               # far below the group maximum
    x[R // 2, 1::7] = -0.0
    bits = bf16_bits(x)
    ng = (K + 127) // 128
    q = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((R, ng), dtype=torch.uint8, device="cuda")
    m.moe_act_quant(to_dev(bits), q, s)
    torch.cuda.synchronize()
    rq, rs = oracle.act_quant_e4m3(bits)
    assert np.array_equal(s.cpu().numpy(), rs), "scale bytes differ"
    assert np.array_equal(q.cpu().numpy(), rq), "codes differ"


def run_q8(wl, W, batch, tm=None, path=None):
    """The activation-quantised plan; a tile height (tm) selects the grouped
    path, else `path` (default AUTO: decode sizes run the decode kernels on
    the quantised values as bf16)."""
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import Runner, to_dev
    T = batch.x.shape[0]
    if path is None:
        path = GROUPED if tm is not None else 0
    opts = {m.MOE_OPT_Q8_TILE: 64 * tm} if tm is not None else None
    run = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T, path, act_fmt=1, options=opts)
    outs = run.outputs(T)
    run.forward(W, to_dev(batch.x), to_dev(batch.bias) if batch.bias is not None else None, outs)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in outs.items()}
    res["h"] = run.h(T).cpu().numpy().view(np.uint16)
    res["path"] = "decode" if m.moe_plan_path(run.plan, T) == DECODE else "grouped"
    return res


def check_out_q8_e2e(g, ref_out, rows=None):
    """out against the oracle's own quantised layer: the decode route's h
    equals the oracle's bit for bit, so it is held to the default bars; the
    grouped path's to the variant's own."""
    got = g["out"] if rows is None else g["out"][rows]
    return check_out(got, ref_out) if g["path"] == "decode" else check_out_actq(got, ref_out)


def q8_reference(wl, layer, batch, ref, g_h, tokens):
    """The oracle's steps for the listed tokens with the down projection fed
    by the GPU's own h: h quantises to codes by a rounding decision, so an h
    that differs by one bf16 step (the sums behind it are taken in another
    order) can move its code by a whole e4m3 step; feeding both sides the
    same h keeps that decision common.  Returns (h the oracle computes for
    the tokens' slots [n, k, f], out [n, d] from the GPU's h)."""
    T, k = ref.ids.shape
    tokens = np.asarray(tokens, np.int64)
    pos = ref.inv_perm.reshape(T, k)[tokens]
    xq = oracle.act_dequant(*oracle.act_quant_e4m3(batch.x[tokens]))
    deq = {}

    def mats(e):
        if e not in deq:
            deq[e] = tuple(oracle.dequant(m.q[e], m.s[e], wl.fmt, m.K)
                           for m in (layer.gate, layer.up, layer.down))
        return deq[e]

    h_ref = np.zeros((len(tokens), k, wl.f), np.uint16)
    out = np.zeros((len(tokens), wl.d))
    for j in range(k):
        hq = oracle.act_dequant(*oracle.act_quant_e4m3(g_h[pos[:, j]]))
        for r in range(len(tokens)):
            Wg, Wu, Wd = mats(int(ref.ids[tokens[r], j]))
            g, u = xq[r] @ Wg.T, xq[r] @ Wu.T
            h_ref[r, j] = oracle.bf16_rne(oracle.silu(g) * u)
            out[r] += ref.w[tokens[r], j] * (hq[r] @ Wd.T)
    return h_ref, out.astype(np.float32)


def check_h_q8(h_gpu, h_ref, min_equal=0.9):
    """h of the block-scaled path against the oracle's: within one bf16 step
    of the larger magnitude plus 2^-10 of h's RMS.  The fp8 x fp8 MFMA rounds
    its 64-product sums inside the instruction at about 2^-14 of the largest
    product, so h that comes out of cancelling sums (near zero) carries an
    absolute error on that scale, and h's bf16 rounding lands on the other
    neighbour for a few percent of values.  Returns the equal fraction."""
    g = oracle.bf16_to_f64(h_gpu)
    r = oracle.bf16_to_f64(h_ref)
    rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 0.0
    err = np.abs(g - r)
    tol = 2.0 ** -7 * np.maximum(np.abs(g), np.abs(r)) + 2.0 ** -10 * rms
    assert np.all(err <= tol), f"h off by {float(np.max(err - tol)):.3e} beyond the bound (rms {rms:.3e})"
    eq = float((h_gpu == h_ref).mean()) if h_ref.size else 1.0
    assert eq >= min_equal, f"only {eq:.4f} of h values equal"
    return eq


def oracle_q8(wl, layer, batch, tokens=None):
    return oracle.moe_forward(batch.x, layer.w_router, batch.bias, omat(layer.gate), omat(layer.up),
                              omat(layer.down), wl.k, wl.renorm, wl.fmt, tokens=tokens,
                              act_quant=True)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("T,tm", [(1, None), (37, 1), (37, 2), (37, 3), (150, 1), (150, 3)])
def test_act_quant_layer(fmt, T, tm):
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, T)
    if T == 150:
        # every token on expert 1 (+ the next k-1): one expert spans several tiles
        bias = np.zeros((T, wl.E), np.float32)
        bias[:, 1] = 100.0
        batch = synth.Batch(batch.x, bias)
    ref = oracle_q8(wl, layer, batch)
    g = run_q8(wl, W, batch, tm)
    check_routing(g, ref)
    eq = check_h_q8(g["h"], ref.h)
    _, out_ref = q8_reference(wl, layer, batch, ref, g["h"], np.arange(T))
    mx, rms, mrel = check_out(g["out"], out_ref)
    mx_o, _, mrel_o = check_out_q8_e2e(g, ref.out)
    log(f"act-quant {fmt} T={T} tm={tm} ({g['path']}): h equal {eq:.4f}; against the oracle's "
        f"down fed this h: max|err| {mx:.3e} rms {rms:.3e} mean rel {mrel:.3e}; end to end: "
        f"max|err| {mx_o:.3e} mean rel {mrel_o:.3e}")


def test_act_quant_differs_from_bf16_layer():
    """The variant is opt-in because it changes results: its out differs from
    the default path's by about the e4m3 quantisation step (2^-4 relative per
    input), far beyond the default path's own tolerance."""
    from gpu_util import gpu_run, oracle_run
    wl, layer, W = get("e4m3")
    batch = synth.make_batch(wl, layer, 37)
    q8 = run_q8(wl, W, batch)["out"]
    ref = oracle_run(wl, layer, batch).out
    rel = float(np.abs(q8 - ref).sum() / np.abs(ref).sum())
    assert 1e-3 < rel < 0.1, rel
    g, _ = gpu_run(wl, W, batch, 2)
    check_out(g["out"], ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_act_quant_dense_branch(fmt):
    """A one-expert top-1 plan with quantised activations (the dense branch of
    the block): identity routing with weight 1, the down projection writing
    out directly, against the oracle's quantised layer with E = 1, k = 1."""
    base = WLS[fmt]
    wl = synth.Workload(f"aq-dense-{fmt}", base.d, base.f, 1, 1, fmt, True, (100,), False, 5111)
    layer = synth.make_layer(wl)
    W = device_weights(layer)
    batch = synth.make_batch(wl, layer, 100)
    ref = oracle_q8(wl, layer, batch)
    g = run_q8(wl, W, batch)
    assert np.all(g["topk_ids"] == 0) and np.all(g["topk_w"] == 1.0)
    check_h_q8(g["h"], ref.h)
    _, out_ref = q8_reference(wl, layer, batch, ref, g["h"], np.arange(100))
    check_out(g["out"], out_ref)
    check_out_q8_e2e(g, ref.out)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("T,path", [(1, DECODE), (8, DECODE), (37, DECODE), (37, GROUPED)])
def test_act_quant_decode_route(fmt, T, path):
    """The decode path of the activation-quantised plan: x and h replaced by
    their quantised values as bf16 (exact: code * 2^E has at most 5
    significant bits), then the decode kernels (matvec at one token, MFMA
    tiles above); the grouped path at the same size for comparison.  Both
    against the oracle's quantised layer."""
    wl, layer, W = get(fmt)
    batch = synth.make_batch(wl, layer, T)
    ref = oracle_q8(wl, layer, batch)
    g = run_q8(wl, W, batch, path=path)
    check_routing(g, ref)
    eq = check_h_q8(g["h"], ref.h)
    _, out_ref = q8_reference(wl, layer, batch, ref, g["h"], np.arange(T))
    mx, rms, mrel = check_out(g["out"], out_ref)
    mx_o, _, mrel_o = check_out_q8_e2e(g, ref.out)
    if path == DECODE:  # the bf16 MFMA on exact quantised values: the default path's h bars
        check_h(g["h"], ref.h)
    log(f"act-quant {fmt} T={T} path={path}: h equal {eq:.4f}, max|err| {mx:.3e} mean rel "
        f"{mrel:.3e}; end to end max|err| {mx_o:.3e} mean rel {mrel_o:.3e}")

