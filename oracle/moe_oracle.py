"""CPU oracle of the MoE FFN layer forward pass.

TEST INFRASTRUCTURE.  This module is the plain, slow, obviously-correct
definition the GPU path is checked against.  Only the test-suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path never does, and this module imports nothing from the product.

What it computes, step by step, with the passage each step follows (the
pages are engineering write-ups of MoE inference engines; none prints this
layer's code, so each step states the plainest reading):

  O1  x arrives as bf16 and is widened exactly: the bf16 bits are the top
      half of an f32 (dragon.c page, section 8 "The speed war", Round 3:
      bf16 -> f32 is a 16-bit left shift).
  O2  Router logits l[t,e] = sum_i W_r[e,i] x[t,i] (+ bias[t,e]), an f32
      router (dragon.c page, "Precision": the router runs in f32).  The sum
      is taken in float64 and rounded once to f32.
  O3  Top-k on the f32 logits; equal logits go to the lower expert index.
  O4  The k ids of a token are listed in ascending expert id, their weights
      aligned with them (reading R1: the order inside the top-k is not given
      by any page; ascending ids make the grouping depend only on the set).
  O5  p = softmax over all E logits (max-subtracted), w[t,j] = p[ids[t,j]],
      divided by their sum when the workload renormalises.  float64.
  O6  Counting-sort permute of the token-slots s = t*k + j by expert id:
      counts, exclusive-scan offsets, stable scatter (Trochilus README,
      "Acknowledgements": (token, expert) pairs sorted by a counting sort).
  O7  Weights dequantised exactly in float64:
        e4m3: W[n,c] = dec_e4m3(q[n,c]) * S[n//128, c//128]   (dragon.c page,
              "Precision" and Round 3: e4m3 with 128x128 blockwise f32 scales,
              256 possible byte values; the 128-column scale structure)
        e2m1: W[n,c] = dec_e2m1(nibble(n,c)) * 2^(S[n, c//32] - 127)
              (dev.to page, DeepSeek-V4.1-Flash post, "Bytes per token decide
              everything": FP4 experts with scales; UE8M0 = a biased power-of-
              two exponent byte; element 2i in the low nibble, reading R11).
        nvfp4: W[n,c] = dec_e2m1(nibble(n,c)) * dec_e4m3(S[n, c//16])
              (dev.to page, post "Running a 133 GB MoE model on an 8 GB GPU
              at 11 tokens/s", "The engine", item 4: expert weights in NVFP4;
              one e4m3 scale byte per 16 codes, reading R18; no second-level
              per-tensor scale is on the page, reading R19).
  O8  Per slot s routed to expert e: g = W_gate x, u = W_up x,
      h = bf16_rne(silu(g) * u), silu(g) = g / (1 + exp(-g))  (SwiGLU experts:
      Trochilus README "How it keeps up" and the dev.to NVFP4 post "The
      engine", item 4; h is stored in bf16 by definition of the workload).
  O9  y_s = W_down h_s, float64.
  O10 out[t] = sum_j w[t,j] y_{t*k+j}, j ascending (WARP BACKENDS.md,
      "Coherent memory": one partial per selected expert, reduced in router
      order), rounded once to f32.

float64 stands in for exact arithmetic everywhere except the two roundings
the definition itself makes (f32 router logits, bf16 h) and the final f32
output.

The steps either side of the layer in a transformer block (dragon.c page,
summary: the MoE reads sub-block 0's normed hidden state, its output is added
to the stream at the end of sub-block 1; "Precision": norms in bf16, the dense
per-sub-block branches quantised like the routed experts):

  B1  RMS normalisation (rmsnorm): xn = bf16_rne(x / sqrt(mean(x^2) + eps) * gamma)
      per row, x and gamma bf16, float64 inside, one rounding (reading N1: the
      page names the norm and its bf16 precision, not its formula; this is the
      RMSNorm form with a gain and an epsilon).
  B2  The dense (shared) branch: one SwiGLU expert on every token with weight 1,
      which is what moe_forward computes with E = 1 and k = 1 (reading N2).
  B3  The add into the residual stream (residual_add):
      out = bf16_rne(residual + (routed + dense)), float64 inside, one rounding.

The activation-quantised variant (opt-in; it changes results by design: the
dev.to DeepSeek-V4.1-Flash post, "Three bugs on RTX 50xx that never raise an
error", item 2: the model's activation quantiser writes fp8 with UE8M0
(power-of-two) scales, always on in that model; WARP BACKENDS.md, the SDOT
mode table and "i8mm/SMMLA for the batched matmul": quantised activations
move results by about 1e-2 relative, a real change rather than rounding
noise):

  Q1  act_quant_e4m3: each bf16 row is cut into groups of 128 consecutive
      inputs (the last group of a row whose length is not a multiple of 128
      is shorter; reading Q-a); a group's scale is the smallest power of two
      2^E with max|x| <= 448 * 2^E, stored as the byte E + 127 (UE8M0; 127 for
      an all-zero group; reading Q-b), and each input becomes the e4m3 code
      nearest x / 2^E (ties to the even mantissa; the sign bit is x's, so -0
      and negatives that round to zero keep it).  x / 2^E is exact, and
      |x / 2^E| <= 448 so nothing saturates.
  Q2  The forward with both expert inputs quantised by Q1 (reading Q-c): the
      token rows x before gate/up, and h (already bf16 by O8) before down;
      the GEMMs then see the dequantised values code * 2^E exactly.  The
      router still reads the unquantised x (O2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

# ---------------------------------------------------------------- formats (O1, O7)


def e4m3_value(code: int) -> float:
    """OCP E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
    Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e2m1_value(code: int) -> float:
    """OCP E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
    Exponent field 0 is subnormal (m * 0.5)."""
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (the bits are the top half of an f32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_rne(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (8 significant bits, ties to even)
    and return the bf16 bit patterns.  Magnitudes that round to 2^128 or beyond
    become infinities; below 2^-126 the quantum stays 2^-133 (subnormals)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(a)                       # a = fr * 2^ex, fr in [0.5, 1)
        e = np.maximum(ex - 1, -126)              # exponent of the leading bit, floored
        q = np.ldexp(1.0, e - 7)                  # quantum: 7 fraction bits
        r = np.rint(a / q) * q                    # np.rint: round half to even
    r = np.where(a == 0, 0.0, r)
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    r = np.where(np.isnan(a), np.nan, r)
    r = np.copysign(r, v)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def unpack_e2m1(q: np.ndarray, K: int) -> np.ndarray:
    """Packed [N, K/2] bytes -> [N, K] codes; element 2i is the low nibble."""
    lo = q & 0x0F
    hi = q >> 4
    return np.stack([lo, hi], axis=-1).reshape(q.shape[0], K)


def dequant(q: np.ndarray, s: np.ndarray, fmt: str, K: int) -> np.ndarray:
    """One expert matrix [N, K] in float64 (O7): each element is its code's
    value times its block's or group's scale, one exact float64 product (the
    scale is broadcast over its block in place)."""
    N = q.shape[0]
    if fmt == "e4m3":
        W = E4M3[q]
        W.reshape(N // 128, 128, K // 128, 128)[...] *= s.astype(np.float64)[:, None, :, None]
        return W
    if fmt == "e2m1":
        W = E2M1[unpack_e2m1(q, K)]
        W.reshape(N, K // 32, 32)[...] *= np.ldexp(1.0, s.astype(np.int64) - 127)[:, :, None]
        return W
    if fmt == "nvfp4":
        W = E2M1[unpack_e2m1(q, K)]
        W.reshape(N, K // 16, 16)[...] *= E4M3[s][:, :, None]
        return W
    raise ValueError(fmt)


# ---------------------------------------------------------------- routing (O2-O6)


def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None):
    """f32 logits [T, E] (O2)."""
    xf = bf16_to_f64(x)
    l = xf @ w_router.astype(np.float64).T
    if bias is not None:
        l = l + bias.astype(np.float64)
    return l.astype(np.float32)


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """ids [T, k] int32: the k largest logits, ties to the lower index (O3),
    listed in ascending expert id (O4)."""
    order = np.argsort(-logits, axis=1, kind="stable")  # stable: equal keys keep index order
    return np.sort(order[:, :k], axis=1).astype(np.int32)


def routing_weights(logits: np.ndarray, ids: np.ndarray, renorm: bool) -> np.ndarray:
    """w [T, k] float64 (O5)."""
    l = logits.astype(np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def permute(ids: np.ndarray, E: int):
    """Counting sort of the slots s = t*k + j by expert (O6).
    Returns counts [E], offsets [E+1], perm [S] (sorted position -> slot) and
    inv_perm [S] (slot -> sorted position), all int32."""
    flat = ids.reshape(-1).astype(np.int64)
    S = flat.size
    counts = np.zeros(E, np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    perm = np.empty(S, np.int64)
    for s in range(S):
        e = flat[s]
        perm[cursor[e]] = s
        cursor[e] += 1
    inv_perm = np.empty(S, np.int64)
    inv_perm[perm] = np.arange(S)
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
            inv_perm.astype(np.int32))


# ---------------------------------------------------------------- experts (O8-O10)


def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(xf: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, act_q: bool = False):
    """Rows xf [M, d] (float64) through one SwiGLU expert: (h bf16 bits [M, f], y [M, d]).
    With act_q, h is quantised by Q1 before the down projection (Q2)."""
    g = xf @ Wg.T
    u = xf @ Wu.T
    h = bf16_rne(silu(g) * u)
    hin = act_dequant(*act_quant_e4m3(h)) if act_q else bf16_to_f64(h)
    y = hin @ Wd.T
    return h, y


def combine(y_sorted: np.ndarray, w: np.ndarray, inv_perm: np.ndarray) -> np.ndarray:
    """out[t] = sum over j ascending of w[t,j] * y[slot t*k+j] (O10), f32."""
    T, k = w.shape
    out = np.zeros((T, y_sorted.shape[1]), np.float64)
    pos = inv_perm.reshape(T, k)
    for j in range(k):
        out = out + w[:, j:j + 1] * y_sorted[pos[:, j]]
    return out.astype(np.float32)


# ---------------------------------------------------------------- activation quantiser (Q1)

ACT_GROUP = 128
E4M3_MAX = 448.0


def e4m3_rne(v: np.ndarray) -> np.ndarray:
    """float64 values with |v| <= 448 -> e4m3 codes, round to nearest with ties
    to the even mantissa; the sign bit is v's sign bit."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    assert np.all(a <= E4M3_MAX), "e4m3_rne: value beyond 448"
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)                   # a = fr * 2^ex, fr in [0.5, 1)
    e = np.maximum(ex - 1, -6)                # exponent of the leading bit, floored (subnormals)
    q = np.ldexp(1.0, e - 3)                  # quantum: 3 fraction bits
    r = np.where(a == 0, 0.0, np.rint(a / q) * q)   # np.rint: half to even
    # codes 0x00 .. 0x7E hold the non-negative values in increasing order
    idx = np.searchsorted(E4M3[:0x7F], r)
    assert np.all(E4M3[idx] == r)
    return (idx | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def ue8m0_for(amax: float) -> int:
    """The byte E + 127 of the smallest power of two 2^E with amax <= 448 * 2^E
    (at least 0); 127 for amax = 0 (Q1)."""
    if amax == 0:
        return 127
    E = max(math.frexp(amax)[1] - 9, -127)    # within one or two of the answer
    while amax > E4M3_MAX * 2.0 ** E:
        E += 1
    while E > -127 and amax <= E4M3_MAX * 2.0 ** (E - 1):
        E -= 1
    return E + 127


def act_quant_e4m3(bits: np.ndarray, group: int = ACT_GROUP):
    """Q1: bf16 rows [R, K] -> (e4m3 codes uint8 [R, K], UE8M0 scale bytes uint8
    [R, ceil(K / group)])."""
    x = bf16_to_f64(bits)
    R, K = x.shape
    ng = -(-K // group)
    codes = np.zeros((R, K), np.uint8)
    scales = np.zeros((R, ng), np.uint8)
    for g in range(ng):
        blk = x[:, g * group:(g + 1) * group]
        amax = np.max(np.abs(blk), axis=1)
        b = np.array([ue8m0_for(float(a)) for a in amax], np.int64)
        scales[:, g] = b
        codes[:, g * group:(g + 1) * group] = e4m3_rne(blk / np.ldexp(1.0, b - 127)[:, None])
    return codes, scales


def act_dequant(codes: np.ndarray, scales: np.ndarray, group: int = ACT_GROUP) -> np.ndarray:
    """code * 2^(byte - 127) per group, float64 (exact)."""
    K = codes.shape[1]
    sc = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), group, axis=1)[:, :K]
    return E4M3[codes] * sc


@dataclass
class Mat:
    """Quantised expert matrices [E, N, K]: codes q and scales s, in `fmt`."""
    q: np.ndarray
    s: np.ndarray
    K: int


@dataclass
class Result:
    logits: np.ndarray     # f32 [T, E]
    ids: np.ndarray        # int32 [T, k]
    w: np.ndarray          # float64 [T, k]
    counts: np.ndarray     # int32 [E]
    offsets: np.ndarray    # int32 [E+1]
    perm: np.ndarray       # int32 [S]
    inv_perm: np.ndarray   # int32 [S]
    h: Optional[np.ndarray]        # bf16 bits [S, f], slot-sorted (None if not computed)
    y: Optional[np.ndarray]        # float64 [S, d], slot-sorted
    out: np.ndarray        # f32 [T, d] (rows of `tokens` only when a subset was asked)


def moe_forward(x, w_router, bias, gate: Mat, up: Mat, down: Mat, k: int, renorm: bool,
                fmt: str, tokens: Optional[Sequence[int]] = None, act_quant: bool = False,
                workers: int = 1) -> Result:
    """The whole layer (O1-O10).  With `tokens`, routing is computed for every
    token (the permutation needs all of them) but the expert FFN and the
    combine only for the listed tokens; `out` then has one row per listed
    token and h/y are not returned.  With `act_quant`, the activation-quantised
    variant (Q1-Q2).  `workers` > 1 runs the per-expert step (O7-O9) of
    different experts on that many threads; each expert's rows are computed by
    the same code either way, so the result does not depend on it."""
    T, d = x.shape
    E = w_router.shape[0]
    f = gate.q.shape[1]
    logits = router_logits(x, w_router, bias)
    ids = select_topk(logits, k)
    w = routing_weights(logits, ids, renorm)
    counts, offsets, perm, inv_perm = permute(ids, E)
    S = T * k
    xf = bf16_to_f64(x) if not act_quant else act_dequant(*act_quant_e4m3(x))
    want = np.ones(S, bool) if tokens is None else np.isin(np.arange(S) // k, list(tokens))
    h = np.zeros((S, f), np.uint16)
    y = np.zeros((S, d), np.float64)

    def one_expert(e):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        pos = np.arange(lo, hi)
        pos = pos[want[perm[lo:hi]]]
        if pos.size == 0:
            return
        rows = perm[pos] // k
        Wg = dequant(gate.q[e], gate.s[e], fmt, gate.K)
        Wu = dequant(up.q[e], up.s[e], fmt, up.K)
        Wd = dequant(down.q[e], down.s[e], fmt, down.K)
        if act_quant:
            h[pos], y[pos] = expert_ffn(xf[rows], Wg, Wu, Wd, act_q=True)
        else:
            h[pos], y[pos] = expert_ffn(xf[rows], Wg, Wu, Wd)

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_expert, range(E)))
    else:
        for e in range(E):
            one_expert(e)
    if tokens is None:
        out = combine(y, w, inv_perm)
        return Result(logits, ids, w, counts, offsets, perm, inv_perm, h, y, out)
    tok = np.asarray(list(tokens), np.int64)
    sub_pos = inv_perm.reshape(T, k)[tok]
    out = np.zeros((tok.size, d), np.float64)
    for j in range(k):
        out = out + w[tok, j:j + 1] * y[sub_pos[:, j]]
    return Result(logits, ids, w, counts, offsets, perm, inv_perm, None, None,
                  out.astype(np.float32))


# ---------------------------------------------------------------- block steps (B1-B3)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """B1: bf16 rows x [T, d] and bf16 gain gamma [d] (bit patterns) -> bf16 bits
    of x / sqrt(mean(x^2) + eps) * gamma, computed in float64, rounded once."""
    xf = bf16_to_f64(x)
    g = bf16_to_f64(gamma)
    ms = np.mean(xf * xf, axis=1, keepdims=True)
    return bf16_rne(xf / np.sqrt(ms + eps) * g)


def residual_add(residual: np.ndarray, routed: np.ndarray,
                 dense: Optional[np.ndarray] = None) -> np.ndarray:
    """B3: bf16 bits of residual + (routed + dense) (dense may be absent),
    float64 inside, rounded once."""
    s = np.asarray(routed, np.float64)
    if dense is not None:
        s = s + np.asarray(dense, np.float64)
    return bf16_rne(bf16_to_f64(residual) + s)


def block_forward(x_hidden, gamma, eps, w_router, bias, gate: Mat, up: Mat, down: Mat, k: int,
                  renorm: bool, fmt: str, dense: Optional[Sequence[Mat]] = None,
                  residual=None):
    """B1 -> the layer (O1-O10) -> B2 -> B3: returns (xn bf16 bits, routed out f32,
    dense out f32 or None, block out bf16 bits).  `dense` is (gate, up, down) of
    the shared expert, each with a leading expert axis of 1; `residual`
    defaults to x_hidden (the plain pre-norm block; the shortcut layout passes
    a later point of the stream)."""
    xn = rmsnorm(x_hidden, gamma, eps)
    routed = moe_forward(xn, w_router, bias, gate, up, down, k, renorm, fmt).out
    dense_out = None
    if dense is not None:
        dg, du, dd = dense
        xf = bf16_to_f64(xn)
        Wg = dequant(dg.q[0], dg.s[0], fmt, dg.K)
        Wu = dequant(du.q[0], du.s[0], fmt, du.K)
        Wd = dequant(dd.q[0], dd.s[0], fmt, dd.K)
        dense_out = expert_ffn(xf, Wg, Wu, Wd)[1].astype(np.float32)
    res = x_hidden if residual is None else residual
    return xn, routed, dense_out, residual_add(res, routed, dense_out)
