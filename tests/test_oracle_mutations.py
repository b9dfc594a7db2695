"""Planted mistakes in the oracle (on the CPU): each one must turn at least one
pin red.  This checks that the pins can tell a wrong oracle from a right one
(cf. the NVFP4 post on the dev.to page, "How we know it's right": control
runs that must break, e.g. with the nibbles swapped)."""
import numpy as np
import pytest

import oracle.moe_oracle as om
import oracle_pins as P

_orig = {name: getattr(om, name) for name in (
    "unpack_e2m1", "dequant", "routing_weights", "router_logits", "select_topk", "silu",
    "expert_ffn", "combine", "permute", "bf16_rne", "rmsnorm", "residual_add", "ue8m0_for",
    "act_quant_e4m3", "e4m3_rne", "block_forward")}


def m_nibble_swap(q, K):
    hi, lo = q & 0x0F, q >> 4
    return np.stack([lo, hi], axis=-1).reshape(q.shape[0], K)


def m_scale_transposed(q, s, fmt, K):
    if fmt == "e4m3":
        s2 = s.T
        scale = np.repeat(np.repeat(s2.astype(np.float64), 128, axis=0), 128, axis=1)
        return om.E4M3[q] * scale
    return _orig["dequant"](q, s, fmt, K)


def m_scale_divided(q, s, fmt, K):
    if fmt == "e4m3":
        scale = np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            return om.E4M3[q] / scale
    return _orig["dequant"](q, s, fmt, K)


def m_e2m1_bias(q, s, fmt, K):
    if fmt == "e2m1":
        codes = om.unpack_e2m1(q, K)
        return om.E2M1[codes] * np.repeat(np.ldexp(1.0, s.astype(np.int64) - 126), 32, axis=1)
    return _orig["dequant"](q, s, fmt, K)


def m_nvfp4_group32(q, s, fmt, K):
    if fmt == "nvfp4":
        codes = om.unpack_e2m1(q, K)
        return om.E2M1[codes] * np.repeat(om.E4M3[s[:, ::2]], 32, axis=1)
    return _orig["dequant"](q, s, fmt, K)


def m_nvfp4_scale_as_ue8m0(q, s, fmt, K):
    if fmt == "nvfp4":
        codes = om.unpack_e2m1(q, K)
        return om.E2M1[codes] * np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 16, axis=1)
    return _orig["dequant"](q, s, fmt, K)


def m_no_renorm(logits, ids, renorm):
    return _orig["routing_weights"](logits, ids, False)


def m_softmax_over_selected(logits, ids, renorm):
    return _orig["routing_weights"](logits, ids, True)


def m_bf16_router(x, w_router, bias=None):
    wr = om.bf16_to_f64(om.bf16_rne(w_router.astype(np.float64))).astype(np.float32)
    return _orig["router_logits"](x, wr, bias)


def m_router_unused(x, w_router, bias=None):
    T, E = x.shape[0], w_router.shape[0]
    l = np.zeros((T, E))
    if bias is not None:
        l = l + bias
    return l.astype(np.float32)


def m_router_transposed_bias(x, w_router, bias=None):
    return _orig["router_logits"](x, w_router, None)


def m_off_by_one(logits, k):
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.sort(order[:, 1:k + 1], axis=1).astype(np.int32)


def m_ties_high(logits, k):
    E = logits.shape[1]
    order = np.argsort(-logits[:, ::-1], axis=1, kind="stable")
    return np.sort(E - 1 - order[:, :k], axis=1).astype(np.int32)


def m_silu_sign(g):
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(g))


def m_gate_up_swapped(xf, Wg, Wu, Wd):
    return _orig["expert_ffn"](xf, Wu, Wg, Wd)


def m_h_unrounded(xf, Wg, Wu, Wd):
    g, u = xf @ Wg.T, xf @ Wu.T
    hv = om.silu(g) * u
    return om.bf16_rne(hv), hv @ Wd.T


def m_combine_reversed(y, w, inv_perm):
    return _orig["combine"](y, w[:, ::-1].copy(), inv_perm)


def m_combine_drop_last(y, w, inv_perm):
    w2 = w.copy()
    w2[:, -1] = 0
    return _orig["combine"](y, w2, inv_perm)


def m_unstable_permute(ids, E):
    counts, offsets, perm, inv_perm = _orig["permute"](ids, E)
    perm = perm.copy()
    for e in range(E):
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(perm.size)
    return counts, offsets, perm, inv_perm


def m_bf16_truncate(v):
    v = np.asarray(v, np.float64).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def m_rmsnorm_no_gain(x, gamma, eps):
    return _orig["rmsnorm"](x, np.full_like(gamma, 0x3F80), eps)


def m_rmsnorm_sum_not_mean(x, gamma, eps):
    xf = om.bf16_to_f64(x)
    return om.bf16_rne(xf / np.sqrt(np.sum(xf * xf, axis=1, keepdims=True) + eps) * om.bf16_to_f64(gamma))


def m_rmsnorm_eps_outside(x, gamma, eps):
    xf = om.bf16_to_f64(x)
    ms = np.mean(xf * xf, axis=1, keepdims=True)
    return om.bf16_rne(xf / (np.sqrt(ms) + eps) * om.bf16_to_f64(gamma))


def m_residual_drops_dense(residual, routed, dense=None):
    return _orig["residual_add"](residual, routed)


def m_actq_scale_low(amax):
    b = _orig["ue8m0_for"](amax)
    return b - 1 if amax else b


def m_actq_group64(bits, group=128):
    return _orig["act_quant_e4m3"](bits, 64)


def m_actq_ties_away(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    r = np.where(a == 0, 0.0, np.floor(a / q + 0.5) * q)
    idx = np.searchsorted(om.E4M3[:0x7F], r)
    return (idx | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def m_actq_h_unquantised(xf, Wg, Wu, Wd, act_q=False):
    return _orig["expert_ffn"](xf, Wg, Wu, Wd)


def _block_variant(dense_input, default_residual):
    """block_forward with the dense branch fed `dense_input` ("xn" or "hidden")
    and the residual defaulting to `default_residual` ("hidden" or "xn")."""
    def f(x_hidden, gamma, eps, w_router, bias, gate, up, down, k, renorm, fmt, dense=None,
          residual=None):
        xn = om.rmsnorm(x_hidden, gamma, eps)
        routed = om.moe_forward(xn, w_router, bias, gate, up, down, k, renorm, fmt).out
        dense_out = None
        if dense is not None:
            dg, du, dd = dense
            xf = om.bf16_to_f64(xn if dense_input == "xn" else x_hidden)
            Wg = om.dequant(dg.q[0], dg.s[0], fmt, dg.K)
            Wu = om.dequant(du.q[0], du.s[0], fmt, du.K)
            Wd = om.dequant(dd.q[0], dd.s[0], fmt, dd.K)
            dense_out = om.expert_ffn(xf, Wg, Wu, Wd)[1].astype(np.float32)
        res = (x_hidden if default_residual == "hidden" else xn) if residual is None else residual
        return xn, routed, dense_out, om.residual_add(res, routed, dense_out)
    return f


m_block_dense_unnormed = _block_variant("hidden", "hidden")
m_block_residual_normed = _block_variant("xn", "xn")


MUTATIONS = {
    "act_quant_scale_one_binade_low": ("ue8m0_for", m_actq_scale_low),
    "act_quant_group_64": ("act_quant_e4m3", m_actq_group64),
    "act_quant_ties_away": ("e4m3_rne", m_actq_ties_away),
    "act_quant_h_not_quantised": ("expert_ffn", m_actq_h_unquantised),
    "rmsnorm_gain_dropped": ("rmsnorm", m_rmsnorm_no_gain),
    "rmsnorm_sum_not_mean": ("rmsnorm", m_rmsnorm_sum_not_mean),
    "rmsnorm_eps_outside_sqrt": ("rmsnorm", m_rmsnorm_eps_outside),
    "residual_add_drops_dense": ("residual_add", m_residual_drops_dense),
    "block_dense_branch_unnormed": ("block_forward", m_block_dense_unnormed),
    "block_residual_defaults_to_normed": ("block_forward", m_block_residual_normed),
    "nibble_swap": ("unpack_e2m1", m_nibble_swap),
    "scale_block_transposed": ("dequant", m_scale_transposed),
    "scale_divided": ("dequant", m_scale_divided),
    "e2m1_scale_bias": ("dequant", m_e2m1_bias),
    "nvfp4_scale_group_32": ("dequant", m_nvfp4_group32),
    "nvfp4_scale_read_as_ue8m0": ("dequant", m_nvfp4_scale_as_ue8m0),
    "dropped_renorm": ("routing_weights", m_no_renorm),
    "softmax_over_selected": ("routing_weights", m_softmax_over_selected),
    "bf16_router": ("router_logits", m_bf16_router),
    "router_weight_unused": ("router_logits", m_router_unused),
    "bias_dropped": ("router_logits", m_router_transposed_bias),
    "off_by_one_id": ("select_topk", m_off_by_one),
    "ties_to_higher_index": ("select_topk", m_ties_high),
    "silu_sign": ("silu", m_silu_sign),
    "gate_up_swapped": ("expert_ffn", m_gate_up_swapped),
    "h_not_rounded": ("expert_ffn", m_h_unrounded),
    "combine_weights_reversed": ("combine", m_combine_reversed),
    "combine_drops_last_slot": ("combine", m_combine_drop_last),
    "unstable_permute": ("permute", m_unstable_permute),
    "bf16_truncation": ("bf16_rne", m_bf16_truncate),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(om, attr, fn)
    P._CACHE.clear()
    caught = []
    for pin in P.FAST_PINS:
        try:
            pin(om)
        except AssertionError as e:  # a pin's check failed: caught
            caught.append(type(e).__name__)
            break
    P._CACHE.clear()
    assert caught, f"mutation {name} passed every pin"


def test_unmutated_oracle_passes_all_fast_pins():
    for pin in P.FAST_PINS:
        pin(om)
