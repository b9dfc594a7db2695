"""Brute-force float64 evaluation of the MoE layer, written independently of
the oracle to pin it: every expert is evaluated densely on every token and
the result is masked to the top-k, so there is no permutation, no grouping
and no gather.  Decoding uses torch's float8 cast and a bit-shift nibble
split; bf16 rounding is a nearest-value search over all bf16 values; logits
are exact sums (math.fsum) of exactly-representable products."""
import math
from fractions import Fraction

import numpy as np
import torch

_E2M1_POS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _bf16_grid():
    bits = np.arange(65536, dtype=np.int32).astype(np.int16)
    vals = torch.from_numpy(bits).view(torch.bfloat16).to(torch.float64).numpy()
    ub = bits.astype(np.uint16)
    ok = np.isfinite(vals) & ~((vals == 0) & (ub == 0x8000))
    vals, ub = vals[ok], ub[ok]
    o = np.argsort(vals, kind="stable")
    return vals[o], ub[o]


_GRID = None


def bf16_round(v):
    """float64 -> nearest bf16 value (float64), ties to the even bit pattern."""
    global _GRID
    if _GRID is None:
        _GRID = _bf16_grid()
    vals, bits = _GRID
    v = np.asarray(v, np.float64)
    i = np.clip(np.searchsorted(vals, v), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    pick_hi = ((hi - v) < (v - lo)) | (((hi - v) == (v - lo)) & ((bits[i] & 1) == 0))
    return np.where(pick_hi, hi, lo)


def bf16_bits_to_f64(x):
    return torch.from_numpy(np.ascontiguousarray(x).astype(np.uint16).view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()


def dequant_e4m3(q, s):
    vals = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    return vals * np.kron(s.astype(np.float64), np.ones((128, 128)))


def dequant_e2m1(q, s):
    N, half = q.shape
    nib = (q[:, :, None] >> np.array([0, 4], np.uint8)) & 0xF   # low nibble first
    nib = nib.reshape(N, 2 * half)
    mag = np.array(_E2M1_POS)[nib & 0x7]
    val = np.where(nib & 0x8, -mag, mag)
    return val * np.kron(2.0 ** (s.astype(np.float64) - 127.0), np.ones((1, 32)))


def dequant_nvfp4(q, s):
    N, half = q.shape
    nib = (q[:, :, None] >> np.array([0, 4], np.uint8)) & 0xF   # low nibble first
    nib = nib.reshape(N, 2 * half)
    mag = np.array(_E2M1_POS)[nib & 0x7]
    val = np.where(nib & 0x8, -mag, mag)
    sc = torch.from_numpy(np.ascontiguousarray(s)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return val * np.kron(sc, np.ones((1, 16)))


def dequant(q, s, fmt):
    return {"e4m3": dequant_e4m3, "e2m1": dequant_e2m1, "nvfp4": dequant_nvfp4}[fmt](q, s)


def exact_logits_f32(x_bits, w_router, bias):
    """f32(exact sum_i W[e,i] x[t,i] + bias[t,e]) by math.fsum."""
    xf = bf16_bits_to_f64(x_bits)
    W = w_router.astype(np.float64)
    T, E = xf.shape[0], W.shape[0]
    out = np.empty((T, E), np.float32)
    for t in range(T):
        prods = W * xf[t][None, :]   # exact: 8-bit x 24-bit significands
        for e in range(E):
            terms = list(prods[e])
            if bias is not None:
                terms.append(float(bias[t, e]))
            out[t, e] = np.float32(math.fsum(terms))
    return out


def topk_mask(logits, k):
    """mask[t,e]: e is among the k largest, ties to the lower index (rank counting)."""
    T, E = logits.shape
    mask = np.zeros((T, E), bool)
    for t in range(T):
        l = logits[t]
        for e in range(E):
            beaten_by = sum(1 for e2 in range(E) if l[e2] > l[e] or (l[e2] == l[e] and e2 < e))
            mask[t, e] = beaten_by < k
    return mask


def softmax_row(l):
    m = max(float(v) for v in l)
    z = [math.exp(float(v) - m) for v in l]
    Z = math.fsum(z)
    return np.array([v / Z for v in z])


def scale_byte(a):
    """The biased exponent E + 127 of the smallest power of two 2^E with
    a <= 448 * 2^E, by exact rational arithmetic (at least 0; 127 for a = 0)."""
    if a == 0:
        return 127
    f = Fraction(float(a)) / 448
    E = f.numerator.bit_length() - f.denominator.bit_length()
    while Fraction(2) ** E < f:
        E += 1
    while Fraction(2) ** (E - 1) >= f:
        E -= 1
    return max(E, -127) + 127


def act_quant_values(xf, group=128):
    """Per-row groups of `group` inputs quantised to e4m3 with a power-of-two
    scale by torch's float8 cast (round to nearest even; every value fits),
    returned dequantised (float64) together with codes and scale bytes."""
    R, K = xf.shape
    codes = np.zeros((R, K), np.uint8)
    bytes_ = np.zeros((R, -(-K // group)), np.uint8)
    out = np.zeros((R, K))
    for r in range(R):
        for g0 in range(0, K, group):
            blk = xf[r, g0:g0 + group]
            b = scale_byte(np.max(np.abs(blk)))
            v = torch.from_numpy(blk / 2.0 ** (b - 127)).to(torch.float32).to(torch.float8_e4m3fn)
            codes[r, g0:g0 + group] = v.view(torch.uint8).numpy()
            bytes_[r, g0 // group] = b
            out[r, g0:g0 + group] = v.to(torch.float64).numpy() * 2.0 ** (b - 127)
    return out, codes, bytes_


def forward(x_bits, w_router, bias, mats, k, renorm, fmt, act_quant=False):
    """Dense evaluation.  mats = (gate_q, gate_s, up_q, up_s, down_q, down_s), each
    with a leading expert axis.  Returns (ids [T,k], w [T,k], out f64 [T,d]).
    act_quant: the expert inputs (x, then h) quantised per 128-input group."""
    gq, gs, uq, us, dq, ds = mats
    T = x_bits.shape[0]
    E = w_router.shape[0]
    logits = exact_logits_f32(x_bits, w_router, bias)
    mask = topk_mask(logits, k)
    P = np.stack([softmax_row(logits[t]) for t in range(T)]) if T else np.zeros((0, E))
    xf = bf16_bits_to_f64(x_bits)
    if act_quant:
        xf = act_quant_values(xf)[0]
    d = xf.shape[1]
    out = np.zeros((T, d))
    ids = np.zeros((T, k), np.int64)
    wts = np.zeros((T, k))
    for t in range(T):
        sel = np.nonzero(mask[t])[0]          # ascending expert ids
        ids[t] = sel
        pw = P[t, sel]
        wts[t] = pw / math.fsum(pw) if renorm else pw
    # every expert on every token (dense), then masked combine in ascending
    # expert order, which is ascending j since ids are listed ascending
    Y = np.zeros((E, T, d))
    for e in range(E):
        Wg, Wu, Wd = dequant(gq[e], gs[e], fmt), dequant(uq[e], us[e], fmt), dequant(dq[e], ds[e], fmt)
        g = xf @ Wg.T
        u = xf @ Wu.T
        h = bf16_round(g / (1.0 + np.exp(-g)) * u)
        if act_quant:
            h = act_quant_values(h)[0]
        Y[e] = h @ Wd.T
    for t in range(T):
        acc = np.zeros(d)
        for j, e in enumerate(ids[t]):
            acc = acc + wts[t, j] * Y[int(e), t]
        out[t] = acc
    return ids, wts, out


def bf16_bits_of(v):
    """float64 values already on the bf16 grid -> their bit patterns (torch's cast,
    exact on such values)."""
    t = torch.tensor(np.asarray(v, np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def block_forward(x_bits, gamma_bits, eps, w_router, bias, mats, k, renorm, fmt, dense_mats,
                  residual_bits):
    """Dense evaluation of the transformer-block steps around the layer: RMS
    normalisation of the hidden rows (float64, one nearest-value bf16 rounding),
    the routed layer by forward() on the normed rows, the shared expert as a
    one-expert layer by forward() on the same rows, and the add into the
    residual stream with the two layer outputs taken as f32 values.
    Returns (xn bits, routed f64, dense f64, block out bits)."""
    xf = bf16_bits_to_f64(x_bits)
    g = bf16_bits_to_f64(gamma_bits)
    T, d = xf.shape
    xn_val = np.zeros((T, d))
    for t in range(T):
        ms = math.fsum(float(v) * float(v) for v in xf[t]) / d
        xn_val[t] = bf16_round(xf[t] / math.sqrt(ms + eps) * g)
    xn = bf16_bits_of(xn_val)
    _, _, routed = forward(xn, w_router, bias, mats, k, renorm, fmt)
    _, _, dense = forward(xn, np.zeros((1, d), np.float32), None, dense_mats, 1, True, fmt)
    acc = (routed.astype(np.float32).astype(np.float64)
           + dense.astype(np.float32).astype(np.float64))
    out = bf16_bits_of(bf16_round(bf16_bits_to_f64(residual_bits) + acc))
    return xn, routed, dense, out
