"""Pins of the CPU oracle.  Each pin takes the oracle module as an argument so
that the planted-mistake tests can run the same pins on a mutated copy; a pin
raises AssertionError (or any exception) when the oracle is wrong."""
import math

import numpy as np
import torch

import bruteforce as bf
import synth

# Small workloads: non-square blocks (d != f) so that transposed operands or
# transposed scale indices cannot go unnoticed.
SMALL = {
    "tiny": synth.WORKLOADS["tiny"],
    "e4m3-nonsquare": synth.Workload("e4m3-nonsquare", 256, 384, 6, 2, "e4m3", False, (5,), False,
                                     2001),
    "e2m1-small": synth.Workload("e2m1-small", 128, 96, 8, 3, "e2m1", True, (5,), False, 2002),
    "nvfp4-small": synth.Workload("nvfp4-small", 128, 96, 8, 3, "nvfp4", True, (5,), False, 2003),
}

_CACHE = {}


def case(name, T=None, biased=False):
    key = (name, T, biased)
    if key not in _CACHE:
        wl = SMALL[name]
        layer = synth.make_layer(wl)
        T = wl.batches[0] if T is None else T
        batch = synth.make_batch(wl, layer, T)
        if biased:
            rng = np.random.default_rng(7)
            batch.bias = (rng.standard_normal((T, wl.E)) * 0.5).astype(np.float32)
            batch = synth.Batch(batch.x, batch.bias)
        _CACHE[key] = (wl, layer, batch)
    return _CACHE[key]


def mats(om, layer):
    return (om.Mat(layer.gate.q, layer.gate.s, layer.gate.K),
            om.Mat(layer.up.q, layer.up.s, layer.up.K),
            om.Mat(layer.down.q, layer.down.s, layer.down.K))


def run(om, wl, layer, batch, **kw):
    g, u, d = mats(om, layer)
    return om.moe_forward(batch.x, layer.w_router, batch.bias, g, u, d, wl.k, wl.renorm, wl.fmt, **kw)


def assert_out_close(got, ref, ulps=2.0):
    """f32 result vs float64 reference: within a couple of f32 ulps."""
    ref = np.asarray(ref, np.float64)
    err = np.abs(got.astype(np.float64) - ref)
    tol = ulps * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-37
    assert np.all(err <= tol), f"max err {err.max():.3e}"


# ---------------------------------------------------------------- brute force


def pin_bruteforce(om, name, T=None, biased=False):
    wl, layer, batch = case(name, T, biased)
    r = run(om, wl, layer, batch)
    ids, w, out = bf.forward(batch.x, layer.w_router, batch.bias,
                             (layer.gate.q, layer.gate.s, layer.up.q, layer.up.s, layer.down.q,
                              layer.down.s), wl.k, wl.renorm, wl.fmt)
    assert np.array_equal(r.ids, ids), "expert ids differ from brute force"
    np.testing.assert_allclose(r.w, w, rtol=1e-12, atol=0)
    assert_out_close(r.out, out)


# ---------------------------------------------------------------- hand-built closed form


def onehot_layer(om):
    """d=256, f=384, E=3, k=1 (renorm).  Token 0 -> expert 1, token 1 -> expert 2.
    Each expert has a single non-zero weight per matrix, so the output has one
    non-zero element whose value is written out by hand below."""
    d, f, E = 256, 384, 3
    w_router = np.zeros((E, d), np.float32)
    w_router[1, 5] = 1.0      # token 0 (x[5] = 2) -> logits (0, 2, 0)
    w_router[2, 17] = 1.0     # token 1 (x[17] = 2) -> logits (0, 0, 2)
    x = np.zeros((2, d), np.uint16)
    x[0, 5] = 0x4000          # bf16 2.0
    x[1, 17] = 0x4000
    gq = np.zeros((E, f, d), np.uint8)
    uq = np.zeros((E, f, d), np.uint8)
    dq = np.zeros((E, d, f), np.uint8)
    # distinct scale in every block: a wrong block index picks a wrong value
    gs = (1.0 + np.arange(E * 3 * 2, dtype=np.float32)).reshape(E, 3, 2)
    us = (100.0 + np.arange(E * 3 * 2, dtype=np.float32)).reshape(E, 3, 2)
    ds = (1000.0 + np.arange(E * 2 * 3, dtype=np.float32)).reshape(E, 2, 3)
    # expert 1: Wg[300,5] = 1.5*0.5, Wu[300,5] = 2.0*0.25, Wd[200,300] = 3.0*2.0
    gq[1, 300, 5], gs[1, 2, 0] = 0x3C, 0.5
    uq[1, 300, 5], us[1, 2, 0] = 0x40, 0.25
    dq[1, 200, 300], ds[1, 1, 2] = 0x44, 2.0
    # expert 2: Wg[10,17] = -1.25*1, Wu[10,17] = 1.75*0.5, Wd[140,10] = -0.5*4
    gq[2, 10, 17], gs[2, 0, 0] = 0xBA, 1.0
    uq[2, 10, 17], us[2, 0, 0] = 0x3E, 0.5
    dq[2, 140, 10], ds[2, 1, 0] = 0xB0, 4.0
    return x, w_router, (gq, gs, uq, us, dq, ds)


def pin_onehot(om):
    x, w_router, (gq, gs, uq, us, dq, ds) = onehot_layer(om)
    G, U, D = om.Mat(gq, gs, 256), om.Mat(uq, us, 256), om.Mat(dq, ds, 384)
    r = om.moe_forward(x, w_router, None, G, U, D, 1, True, "e4m3")
    assert r.ids.tolist() == [[1], [2]]
    assert r.w.tolist() == [[1.0], [1.0]]

    def hval(g, u):
        return float(bf.bf16_round(np.array(g / (1.0 + math.exp(-g)) * u)))

    exp = np.zeros((2, 256))
    # token 0: g = 2*0.75 = 1.5, u = 2*0.5 = 1, y[200] = h * 6
    exp[0, 200] = hval(1.5, 1.0) * 6.0
    # token 1: g = 2*(-1.25) = -2.5, u = 2*0.875 = 1.75, y[140] = h * (-2)
    exp[1, 140] = hval(-2.5, 1.75) * -2.0
    assert_out_close(r.out, exp)


# ---------------------------------------------------------------- routing


def pin_routing_closed_form(om):
    """Logits (0, ln2, ln3, ln4): softmax = (1, 2, 3, 4)/10; the top-2 are
    experts 2 and 3 with weights 0.3, 0.4, or 3/7, 4/7 when renormalised."""
    E, d = 4, 8
    w_router = np.zeros((E, d), np.float32)
    w_router[:, 0] = np.log([1.0, 2.0, 3.0, 4.0]).astype(np.float32)
    x = np.zeros((1, d), np.uint16)
    x[0, 0] = 0x3F80  # 1.0
    logits = om.router_logits(x, w_router, None)
    ids = om.select_topk(logits, 2)
    assert ids.tolist() == [[2, 3]]
    w = om.routing_weights(logits, ids, False)
    np.testing.assert_allclose(w, [[0.3, 0.4]], rtol=1e-6)
    w = om.routing_weights(logits, ids, True)
    np.testing.assert_allclose(w, [[3 / 7, 4 / 7]], rtol=1e-6)
    p = om.routing_weights(logits, np.arange(E)[None, :].astype(np.int32), False)
    assert abs(p.sum() - 1.0) < 1e-15


def pin_router_exact(om):
    for name in ("tiny", "e4m3-nonsquare"):
        wl, layer, batch = case(name, biased=True)
        got = om.router_logits(batch.x, layer.w_router, batch.bias)
        ref = bf.exact_logits_f32(batch.x, layer.w_router, batch.bias)
        assert np.array_equal(got, ref)


def pin_topk_ties(om):
    # equal logits everywhere: the lowest k indices win
    l = np.zeros((3, 9), np.float32)
    assert om.select_topk(l, 4).tolist() == [[0, 1, 2, 3]] * 3
    # a tie across the k/k+1 boundary: experts 5 and 6 equal, only one fits
    l = np.array([[0.1, 0.9, 0.2, 0.3, 0.0, 0.5, 0.5, 0.4]], np.float32)
    assert om.select_topk(l, 3).tolist() == [[1, 5, 6]]
    assert om.select_topk(l, 2).tolist() == [[1, 5]]
    rng = np.random.default_rng(11)
    l = rng.integers(0, 4, size=(50, 12)).astype(np.float32)   # many ties
    assert np.array_equal(om.select_topk(l, 5), np.nonzero(bf.topk_mask(l, 5))[1].reshape(50, 5))


def pin_permute(om):
    rng = np.random.default_rng(5)
    for T, k, E in ((1, 1, 1), (7, 2, 8), (64, 8, 64), (300, 6, 384)):
        ids = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), axis=1)
        counts, offsets, perm, inv_perm = om.permute(ids.astype(np.int32), E)
        flat = ids.reshape(-1)
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(np.sort(perm), np.arange(T * k))      # every slot exactly once
        assert np.array_equal(inv_perm[perm], np.arange(T * k))
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(seg) > 0) and np.all(flat[seg] == e)


def pin_silu(om):
    np.testing.assert_allclose(om.silu(np.array([0.0, 1.0, -1.0, 2.0])),
                               [0.0, 0.7310585786300049, -0.2689414213699951, 1.7615941559557649],
                               rtol=1e-15)
    assert om.silu(np.array([-800.0]))[0] == 0.0
    assert om.silu(np.array([800.0]))[0] == 800.0


# ---------------------------------------------------------------- invariants and special cases


def pin_scale_doubling(om):
    """Doubling every down scale (or every up scale) doubles out bit-exactly:
    a power of two commutes with every rounding on the way."""
    for name in ("tiny", "e4m3-nonsquare", "e2m1-small"):
        wl, layer, batch = case(name)
        G, U, D = mats(om, layer)
        base = om.moe_forward(batch.x, layer.w_router, None, G, U, D, wl.k, wl.renorm, wl.fmt).out
        if wl.fmt == "e4m3":
            D2 = om.Mat(D.q, D.s * 2, D.K)
            U2 = om.Mat(U.q, U.s * 2, U.K)
        else:
            D2 = om.Mat(D.q, D.s + 1, D.K)
            U2 = om.Mat(U.q, U.s + 1, U.K)
        o1 = om.moe_forward(batch.x, layer.w_router, None, G, U, D2, wl.k, wl.renorm, wl.fmt).out
        o2 = om.moe_forward(batch.x, layer.w_router, None, G, U2, D, wl.k, wl.renorm, wl.fmt).out
        assert np.array_equal(o1, 2 * base) and np.array_equal(o2, 2 * base)


def pin_identical_experts(om):
    """All experts equal and weights renormalised: out does not depend on routing."""
    wl, layer, batch = case("tiny")
    G, U, D = mats(om, layer)
    rep = lambda M: om.Mat(np.repeat(M.q[:1], wl.E, 0), np.repeat(M.s[:1], wl.E, 0), M.K)
    G1, U1, D1 = rep(G), rep(U), rep(D)
    a = om.moe_forward(batch.x, layer.w_router, None, G1, U1, D1, wl.k, True, wl.fmt)
    b = om.moe_forward(batch.x, layer.w_router[::-1].copy(), None, G1, U1, D1, wl.k, True, wl.fmt)
    assert not np.array_equal(a.ids, b.ids)
    np.testing.assert_allclose(a.out, b.out, rtol=1e-6, atol=1e-7)
    single = om.moe_forward(batch.x, layer.w_router[:1].copy(), None,
                            om.Mat(G1.q[:1], G1.s[:1], G.K), om.Mat(U1.q[:1], U1.s[:1], U.K),
                            om.Mat(D1.q[:1], D1.s[:1], D.K), 1, True, wl.fmt)
    np.testing.assert_allclose(a.out, single.out, rtol=1e-6, atol=1e-7)


def pin_relabel(om):
    """Relabelling the experts (router rows and expert weights together) leaves out unchanged."""
    wl, layer, batch = case("e4m3-nonsquare")
    G, U, D = mats(om, layer)
    a = om.moe_forward(batch.x, layer.w_router, None, G, U, D, wl.k, wl.renorm, wl.fmt)
    p = np.random.default_rng(3).permutation(wl.E)
    P = lambda M: om.Mat(M.q[p].copy(), M.s[p].copy(), M.K)
    b = om.moe_forward(batch.x, layer.w_router[p].copy(), None, P(G), P(U), P(D), wl.k,
                       wl.renorm, wl.fmt)
    np.testing.assert_allclose(a.out, b.out, rtol=1e-6, atol=1e-7)


def pin_zero_input(om):
    wl, layer, batch = case("e4m3-nonsquare")
    G, U, D = mats(om, layer)
    x = np.zeros_like(batch.x)
    r = om.moe_forward(x, layer.w_router, None, G, U, D, wl.k, wl.renorm, wl.fmt)
    assert np.all(r.out == 0)
    assert r.ids.tolist() == [list(range(wl.k))] * x.shape[0]
    np.testing.assert_allclose(r.w, 1.0 / wl.E)


def pin_single_expert(om):
    """E = 1, k = 1: a dense SwiGLU MLP with weight exactly 1 and the identity permutation."""
    wl, layer, batch = case("e2m1-small")
    G, U, D = mats(om, layer)
    one = lambda M: om.Mat(M.q[:1], M.s[:1], M.K)
    r = om.moe_forward(batch.x, layer.w_router[:1].copy(), None, one(G), one(U), one(D), 1, True,
                       wl.fmt)
    assert np.all(r.w == 1.0)
    assert np.array_equal(r.perm, np.arange(batch.x.shape[0]))
    Wg = bf.dequant(G.q[0], G.s[0], "e2m1")
    Wu = bf.dequant(U.q[0], U.s[0], "e2m1")
    Wd = bf.dequant(D.q[0], D.s[0], "e2m1")
    xf = bf.bf16_bits_to_f64(batch.x)
    g, u = xf @ Wg.T, xf @ Wu.T
    out = bf.bf16_round(g / (1 + np.exp(-g)) * u) @ Wd.T
    assert_out_close(r.out, out)


def pin_lossless_grid(om):
    """Weights drawn on the e4m3 grid with power-of-two scales are represented
    exactly: dequantisation must return them unchanged."""
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, size=(256, 384)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                   # no NaN codes
    sc = np.ldexp(1.0, rng.integers(-8, 8, size=(2, 3))).astype(np.float32)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    truth = vals * np.kron(sc.astype(np.float64), np.ones((128, 128)))
    assert np.array_equal(om.dequant(codes, sc, "e4m3", 384), truth)


def pin_token_subset(om):
    """out rows of a token subset equal the full forward's rows."""
    wl, layer, batch = case("e4m3-nonsquare")
    full = run(om, wl, layer, batch)
    sub = run(om, wl, layer, batch, tokens=[3, 0])
    assert np.array_equal(sub.out, full.out[[3, 0]])


# ---------------------------------------------------------------- block steps


def _bf16(vals):
    """bf16 bit patterns of float64 values by torch's RNE cast (a library routine)."""
    t = torch.tensor(np.asarray(vals, np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pin_rmsnorm(om):
    """RMS normalisation: a hand-worked row, the closed forms of a constant row
    and of power-of-two rescaling, the unit mean square of the output, and the
    gain applied per column."""
    # x = [3, 4]: mean square 12.5, so x / sqrt(12.5) = [0.84853, 1.13137],
    # whose bf16 roundings (7 fraction bits) are 217/256 and 145/128
    x = _bf16([[3.0, 4.0]])
    got = om.rmsnorm(x, _bf16([1.0, 1.0]), 0.0)
    assert list(got[0]) == [0x3F59, 0x3F91], [hex(v) for v in got[0]]
    assert np.array_equal(got, _bf16([[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]]))
    # a constant row c with eps = 0 normalises to sign(c) * gamma exactly
    rng = np.random.default_rng(11)
    gam = _bf16(rng.uniform(0.5, 2.0, 64))
    for c in (0.375, -3.0, 1000.0):
        got = om.rmsnorm(_bf16(np.full((1, 64), c)), gam, 0.0)
        want = _bf16(np.sign(c) * torch.tensor(gam.view(np.int16)).view(torch.bfloat16).double().numpy())
        assert np.array_equal(got[0], want), c
    # rescaling a row by 2^j leaves it unchanged (eps = 0), and the gain is
    # applied per column: gamma = 2 on one column doubles that column exactly
    xr = _bf16(rng.standard_normal((3, 96)))
    one = _bf16(np.ones(96))
    base = om.rmsnorm(xr, one, 0.0)
    scaled = _bf16(torch.tensor(xr.view(np.int16)).view(torch.bfloat16).double().numpy() * 8.0)
    assert np.array_equal(om.rmsnorm(scaled, one, 0.0), base)
    g2 = np.ones(96)
    g2[5] = 2.0
    two = om.rmsnorm(xr, _bf16(g2), 0.0)
    dbl = torch.tensor(base.view(np.int16)).view(torch.bfloat16).double().numpy() * 2.0
    assert np.array_equal(two[:, 5], _bf16(dbl[:, 5]))
    assert np.array_equal(np.delete(two, 5, axis=1), np.delete(base, 5, axis=1))
    # unit mean square (gain 1, eps 0) up to the bf16 rounding of each entry
    yv = torch.tensor(base.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.all(np.abs(np.mean(yv * yv, axis=1) - 1.0) < 2.0 ** -7)
    # eps keeps a zero row at zero; with eps = mean square the scale is 1/sqrt(2)
    assert np.all(om.rmsnorm(_bf16(np.zeros((1, 8))), _bf16(np.ones(8)), 1e-6) == 0)
    got = om.rmsnorm(_bf16(np.full((1, 8), 2.0)), _bf16(np.ones(8)), 4.0)
    assert np.array_equal(got[0], _bf16(np.full(8, 2.0 / math.sqrt(8.0))))


def pin_residual_add(om):
    """The add into the residual stream, exact on small dyadic values, one
    rounding at the end (257.5 has no bf16 form and rounds to 258; 257 is a
    tie and goes to the even 256), and the dense term optional."""
    res = _bf16([[1.0, 2.0, -3.0, 256.0]])
    a = np.array([[0.5, 0.25, 1.0, 1.0]], np.float32)
    b = np.array([[0.25, 0.0, -1.0, 0.5]], np.float32)
    assert np.array_equal(om.residual_add(res, a, b), _bf16([[1.75, 2.25, -3.0, 258.0]]))
    assert np.array_equal(om.residual_add(res, a), _bf16([[1.5, 2.25, -2.0, 256.0]]))


# ---------------------------------------------------------------- activation-quantised variant


def pin_act_quant(om):
    """Q1 on hand-worked groups (448 is code 0x7E at scale 1; 1.0625 and
    1.1875 are ties that go to the even mantissas 1.0 and 1.25; -0 and a
    negative that rounds to zero keep the sign bit; the next bf16 above
    448 * 2^j needs 2^(j+1); a short last group has its own scale), then on
    random rows of many magnitudes against an independent route: exact
    rational scale search and torch's float8 cast (a library routine)."""
    row = [448.0, 1.0625, 1.1875, -0.0, -1e-6] + [0.0] * 123 + [7.0] + [0.5] * 63
    codes, sc = om.act_quant_e4m3(_bf16([row]))
    assert [int(c) for c in codes[0, :5]] == [0x7E, 0x38, 0x3A, 0x80, 0x80], codes[0, :5]
    assert sc.shape == (1, 2) and list(sc[0]) == [127, 121], sc      # 7 = 448 * 2^-6
    assert codes[0, 128] == 0x7E and np.all(codes[0, 129:] == 0x60)   # 0.5 * 2^6 = 32 = 2^5
    for j in (-3, 0, 5):
        c, s_ = om.act_quant_e4m3(_bf16([[448.0 * 2.0 ** j] + [1.0] * 127]))
        assert s_[0, 0] == 127 + j and c[0, 0] == 0x7E
        c, s_ = om.act_quant_e4m3(_bf16([[450.0 * 2.0 ** j] + [1.0] * 127]))  # next bf16 up
        assert s_[0, 0] == 128 + j and c[0, 0] == 0x76, (s_, hex(c[0, 0]))  # 225 -> 224
    c, s_ = om.act_quant_e4m3(np.zeros((2, 256), np.uint16))
    assert np.all(c == 0) and np.all(s_ == 127)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, 320)) * np.ldexp(1.0, rng.integers(-30, 30, (6, 1)))
    x[2, 128:256] = 0.0
    x[3, ::7] *= 1e-4                         # values below the e4m3 normal range of their group
    bits = _bf16(x)
    codes, sc = om.act_quant_e4m3(bits)
    deq, c_ref, s_ref = bf.act_quant_values(bf.bf16_bits_to_f64(bits))
    assert np.array_equal(sc, s_ref), "scale bytes differ from the exact route"
    assert np.array_equal(codes, c_ref), "codes differ from torch's float8 cast"
    assert np.array_equal(om.act_dequant(codes, sc), deq)
    # half a quantum at most: 2^-4 relative in the normal range, 2^-10 of the scale below it
    xf = bf.bf16_bits_to_f64(bits)
    scale = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 128, axis=1)[:, :320]
    assert np.all(np.abs(deq - xf) <= np.maximum(np.abs(xf) * 2.0 ** -4, scale * 2.0 ** -10))


def pin_act_quant_forward(om, name):
    """Q2 against the dense brute force with the same quantiser route (exact
    scales, torch's float8 cast) applied to x and to h."""
    wl, layer, batch = case(name)
    r = run(om, wl, layer, batch, act_quant=True)
    ids, w, out = bf.forward(batch.x, layer.w_router, batch.bias,
                             (layer.gate.q, layer.gate.s, layer.up.q, layer.up.s, layer.down.q,
                              layer.down.s), wl.k, wl.renorm, wl.fmt, act_quant=True)
    assert np.array_equal(r.ids, ids)
    assert_out_close(r.out, out)
    # and it is not the unquantised layer
    assert not np.array_equal(r.out, run(om, wl, layer, batch).out)


def _block_case(om, fmt="e4m3"):
    """A routed layer plus a shared expert of the same format (one expert with a
    leading axis of 1), hidden rows of mixed magnitudes and a gain."""
    name = {"e4m3": "e4m3-nonsquare", "e2m1": "e2m1-small"}[fmt]
    wl, layer, batch = case(name)
    dwl = synth.Workload(wl.name + "-shared", wl.d, wl.f, 1, 1, wl.fmt, True, (), False, wl.seed + 50)
    dl = synth.make_layer(dwl)
    rng = np.random.default_rng(wl.seed + 7)
    T = batch.x.shape[0]
    hid = _bf16(rng.standard_normal((T, wl.d)) * np.ldexp(1.0, rng.integers(-3, 4, (T, 1))))
    gamma = _bf16(rng.uniform(0.5, 1.5, wl.d))
    return wl, layer, dl, hid, gamma


def _block(om, wl, layer, dl, hid, gamma, eps, residual=None):
    g, u, d = mats(om, layer)
    dense = mats(om, dl)
    return om.block_forward(hid, gamma, eps, layer.w_router, None, g, u, d, wl.k, wl.renorm, wl.fmt,
                            dense=dense, residual=residual)


def pin_block_forward(om, fmt="e4m3"):
    """The block steps composed (B1 -> layer -> B2 -> B3) against an independent
    dense brute force of the block; invariance of both branches to a
    power-of-two rescale of the hidden rows (eps = 0: they read the normed
    rows only); the residual defaults to the hidden rows themselves (with all
    down codes zero both branches are exactly 0 and the block returns its
    residual unchanged); the shortcut layout's later residual is honoured."""
    wl, layer, dl, hid, gamma = _block_case(om, fmt)
    eps = 1e-6
    xn, routed, dense, out = _block(om, wl, layer, dl, hid, gamma, eps)
    bxn, brouted, bdense, bout = bf.block_forward(
        hid, gamma, eps, layer.w_router, None,
        (layer.gate.q, layer.gate.s, layer.up.q, layer.up.s, layer.down.q, layer.down.s), wl.k,
        wl.renorm, wl.fmt, (dl.gate.q, dl.gate.s, dl.up.q, dl.up.s, dl.down.q, dl.down.s), hid)
    assert np.array_equal(xn, bxn), "normed rows differ from the brute force"
    assert_out_close(routed, brouted)
    assert dense is not None
    assert_out_close(dense, bdense)
    # the add rounds once to bf16; the brute force's f32 terms may differ from
    # the oracle's by an f32 ulp, which can move a rounding at a bf16 boundary
    a, b = om.bf16_to_f64(out), om.bf16_to_f64(bout)
    assert np.all(np.abs(a - b) <= 2.0 ** -8 * np.abs(b) + 1e-30), "block out off by > 1 bf16 ulp"
    assert float(np.mean(out == bout)) >= 0.99
    # rescaling the hidden rows by 2^3 with eps = 0 leaves xn, and so both branches, unchanged
    xn0, r0, d0, _ = _block(om, wl, layer, dl, hid, gamma, 0.0)
    hid8 = _bf16(om.bf16_to_f64(hid) * 8.0)
    xn8, r8, d8, out8 = _block(om, wl, layer, dl, hid8, gamma, 0.0)
    assert np.array_equal(xn0, xn8) and np.array_equal(r0, r8) and np.array_equal(d0, d8)
    # the residual is the hidden rows unless given: out8 = bf16(8 hid + branches)
    assert not np.array_equal(out8, _block(om, wl, layer, dl, hid, gamma, 0.0)[3])
    # zero down codes: both branches vanish and the block returns its residual exactly
    zl = synth.Layer(layer.wl, layer.w_router, layer.gate, layer.up,
                     synth.QMat(np.zeros_like(layer.down.q), layer.down.s, layer.down.N, layer.down.K))
    zd = synth.Layer(dl.wl, dl.w_router, dl.gate, dl.up,
                     synth.QMat(np.zeros_like(dl.down.q), dl.down.s, dl.down.N, dl.down.K))
    xz, rz, dz, oz = _block(om, wl, zl, zd, hid, gamma, eps)
    assert np.all(rz == 0) and np.all(dz == 0)
    assert np.array_equal(oz, hid), "the default residual is not the hidden rows"
    later = _bf16(om.bf16_to_f64(hid) * 0.5 + 1.0)
    assert np.array_equal(_block(om, wl, zl, zd, hid, gamma, eps, residual=later)[3], later)


FAST_PINS = [
    lambda om: pin_bruteforce(om, "tiny"),
    lambda om: pin_bruteforce(om, "e4m3-nonsquare", biased=True),
    lambda om: pin_bruteforce(om, "e2m1-small"),
    lambda om: pin_bruteforce(om, "nvfp4-small"),
    pin_onehot, pin_routing_closed_form, pin_router_exact, pin_topk_ties, pin_permute, pin_silu,
    pin_scale_doubling, pin_identical_experts, pin_relabel, pin_zero_input, pin_single_expert,
    pin_lossless_grid, pin_token_subset, pin_rmsnorm, pin_residual_add, pin_act_quant,
    pin_block_forward, lambda om: pin_block_forward(om, "e2m1"),
    lambda om: pin_act_quant_forward(om, "e4m3-nonsquare"),
    lambda om: pin_act_quant_forward(om, "e2m1-small"),
]
