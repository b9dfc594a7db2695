"""Seeded synthetic workloads for the MoE FFN layer.

Input preparation only.  This module draws the tensors the layer consumes and
hands the same arrays to the CPU oracle and to the GPU path; it holds none of
the layer's forward arithmetic.  The drawing and quantising is done by
``synth.c`` (counter-based, thread-count independent); this file adds the
workload table and the two acceptance rules of the workloads:

* the router-gap rule: a token whose k-th and (k+1)-th largest router logits
  (computed here in float64, including any skew bias) are closer than 1e-3 is
  redrawn, so that any float32 summation order selects the same experts;
* the skew of the prefill workload: a bias ``delta * u_t`` (u_t ~ U(0, 2)) is
  added to the logits of eight seeded "hot" experts, with ``delta`` found by
  bisection on the drawn batch so that about 30% of token-slots land on them.

Shapes follow the layers the source pages describe: OLMoE-1B-7B (Trochilus
README, "Results"), a LongCat/DeepSeek-class routed-expert layer in e4m3 with
128x128 f32 block scales (dragon.c page, "Precision"), and DeepSeek-V4.1-Flash
FP4 experts of 17.93 MiB each (dev.to page, "Bytes per token decide
everything").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# Stream ids of the counter-based generator.
_S_ROUTER = 1
_S_GATE = 0x100000
_S_UP = 0x200000
_S_DOWN = 0x300000
_S_X = 0x4000000000
_S_SKEW = 0x5000000000
_S_HOT = 0x6000000000

GAP_MIN = 1e-3
HOT_EXPERTS = 8
HOT_SHARE = 0.30


def build(verbose: bool = False) -> str:
    """Compile libsynth.so from synth.c (gcc, OpenMP, no fast-math)."""
    import subprocess

    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-shared", "-fPIC", src, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.synth_stream_key.argtypes = [u64, u64]
        L.synth_stream_key.restype = u64
        L.synth_normal_f32.argtypes = [u64, u64, u64, i64, ctypes.c_double, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, i64, vp]
        L.synth_uniform_f64.argtypes = [u64, u64, u64, i64, vp]
        L.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        L.synth_enc_e4m3.argtypes = [vp, i64, vp]
        L.synth_enc_e2m1.argtypes = [vp, i64, vp]
        L.synth_ue8m0.argtypes = [vp, i64, vp]
        L.synth_quant_e4m3_b128.argtypes = [vp, i64, i64, vp, vp]
        L.synth_quant_e2m1_g32.argtypes = [vp, i64, i64, vp, vp]
        L.synth_quant_nvfp4_g16.argtypes = [vp, i64, i64, vp, vp]
        L.synth_expert_matrices.argtypes = [u64, u64, i64, i64, i64, i64, ctypes.c_double,
                                            ctypes.c_int, vp, vp]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ primitives

def normal_f32(seed: int, stream: int, start: int, n: int, stddev: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(seed, stream, start, n, stddev, _p(out))
    return out


def normal_bf16(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of f32 standard normals, rounded to nearest even."""
    out = np.empty(n, np.uint16)
    lib().synth_normal_bf16(seed, stream, start, n, _p(out))
    return out


def uniform_f64(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform_f64(seed, stream, start, n, _p(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().synth_f32_to_bf16(_p(a), a.size, _p(out))
    return out


def enc_e4m3(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().synth_enc_e4m3(_p(a), a.size, _p(out))
    return out


def enc_e2m1(a: np.ndarray) -> np.ndarray:
    """One 4-bit code per uint8 (unpacked)."""
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().synth_enc_e2m1(_p(a), a.size, _p(out))
    return out


def ue8m0_of_amax(amax: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(amax, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().synth_ue8m0(_p(a), a.size, _p(out))
    return out


def quant_e4m3_b128(w: np.ndarray):
    """[N, K] f32 -> (codes uint8 [N, K], scales f32 [N/128, K/128])."""
    w = np.ascontiguousarray(w, np.float32)
    N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0
    q = np.empty((N, K), np.uint8)
    s = np.empty((N // 128, K // 128), np.float32)
    lib().synth_quant_e4m3_b128(_p(w), N, K, _p(q), _p(s))
    return q, s


def quant_e2m1_g32(w: np.ndarray):
    """[N, K] f32 -> (packed codes uint8 [N, K/2], UE8M0 scales uint8 [N, K/32])."""
    w = np.ascontiguousarray(w, np.float32)
    N, K = w.shape
    assert K % 32 == 0
    q = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // 32), np.uint8)
    lib().synth_quant_e2m1_g32(_p(w), N, K, _p(q), _p(s))
    return q, s


def quant_nvfp4_g16(w: np.ndarray):
    """[N, K] f32 -> (packed codes uint8 [N, K/2], E4M3 scale codes uint8 [N, K/16])."""
    w = np.ascontiguousarray(w, np.float32)
    N, K = w.shape
    assert K % 16 == 0
    q = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // 16), np.uint8)
    lib().synth_quant_nvfp4_g16(_p(w), N, K, _p(q), _p(s))
    return q, s


# ------------------------------------------------------------------ workloads

@dataclass(frozen=True)
class Workload:
    name: str
    d: int          # hidden size
    f: int          # expert FFN width
    E: int          # number of experts
    k: int          # experts per token
    fmt: str        # "e4m3" (128x128 f32 scales), "e2m1" (UE8M0 per 32), "nvfp4" (E4M3 per 16)
    renorm: bool    # renormalise the k routing weights to sum to 1
    batches: tuple = ()
    skew: bool = False
    seed: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", 256, 256, 8, 2, "e4m3", True, (4,), False, 1000),
    "olmoe-decode": Workload("olmoe-decode", 2048, 1024, 64, 8, "e4m3", False, (1, 8), False, 1001),
    "olmoe-prefill-skewed": Workload("olmoe-prefill-skewed", 2048, 1024, 64, 8, "e4m3", False,
                                     (512, 2048), True, 1002),
    "large-e4m3": Workload("large-e4m3", 7168, 2048, 256, 8, "e4m3", True, (1, 64, 4096), False,
                           1003),
    "fp4-e2m1": Workload("fp4-e2m1", 4096, 2880, 384, 6, "e2m1", True, (1, 16, 1024), False, 1004),
    # the FP4 layer's shape with NVFP4 weights (e4m3 scale per 16 inputs)
    "fp4-nvfp4": Workload("fp4-nvfp4", 4096, 2880, 384, 6, "nvfp4", True, (1, 16, 1024), False,
                          1005),
}


def expert_bytes(w: Workload) -> int:
    """Bytes of one expert (three matrices, codes + scales)."""
    if w.fmt == "e4m3":
        return 3 * w.d * w.f + 3 * 4 * (w.d // 128) * (w.f // 128)
    if w.fmt == "nvfp4":
        return 3 * w.d * w.f // 2 + 3 * w.d * w.f // 16
    return 3 * w.d * w.f // 2 + 3 * w.d * w.f // 32


@dataclass
class QMat:
    """Quantised expert matrices [E, N, K]: codes q and scales s (layout per fmt)."""
    q: np.ndarray
    s: np.ndarray
    N: int
    K: int


@dataclass
class Layer:
    wl: Workload
    w_router: np.ndarray        # f32 [E, d]
    gate: QMat                  # [E, f, d]
    up: QMat                    # [E, f, d]
    down: QMat                  # [E, d, f]


@dataclass
class Batch:
    x: np.ndarray                       # bf16 bits, uint16 [T, d]
    bias: Optional[np.ndarray] = None   # f32 [T, E] or None
    resampled: int = 0                  # rows redrawn by the gap rule
    delta: float = 0.0                  # skew strength (skewed workload)
    hot: Optional[np.ndarray] = field(default=None)


def _expert_mats(seed, stream_base, E, N, K, stddev, fmt) -> QMat:
    if fmt == "e4m3":
        assert N % 128 == 0 and K % 128 == 0
        q = np.empty((E, N, K), np.uint8)
        s = np.empty((E, N // 128, K // 128), np.float32)
        f = 0
    elif fmt == "e2m1":
        assert N % 32 == 0 and K % 32 == 0
        q = np.empty((E, N, K // 2), np.uint8)
        s = np.empty((E, N, K // 32), np.uint8)
        f = 1
    else:
        assert fmt == "nvfp4" and N % 32 == 0 and K % 32 == 0
        q = np.empty((E, N, K // 2), np.uint8)
        s = np.empty((E, N, K // 16), np.uint8)
        f = 2
    lib().synth_expert_matrices(seed, stream_base, 0, E, N, K, stddev, f, _p(q), _p(s))
    return QMat(q, s, N, K)


def make_layer(wl: Workload | str, seed: Optional[int] = None) -> Layer:
    """Router f32 ~ N(0, 1/d); gate/up ~ N(0, 1/d) [f x d]; down ~ N(0, 1/f) [d x f],
    each drawn in f32 and quantised to the workload's format."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    seed = wl.seed if seed is None else seed
    d, f, E = wl.d, wl.f, wl.E
    w_router = normal_f32(seed, _S_ROUTER, 0, E * d, 1.0 / np.sqrt(d)).reshape(E, d)
    gate = _expert_mats(seed, _S_GATE, E, f, d, 1.0 / np.sqrt(d), wl.fmt)
    up = _expert_mats(seed, _S_UP, E, f, d, 1.0 / np.sqrt(d), wl.fmt)
    down = _expert_mats(seed, _S_DOWN, E, d, f, 1.0 / np.sqrt(f), wl.fmt)
    return Layer(wl, w_router, gate, up, down)


def _bf16_to_f64(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _kth_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per row: (k-th largest) - ((k+1)-th largest)."""
    part = -np.partition(-logits, k, axis=1)[:, : k + 1]
    part.sort(axis=1)
    return part[:, 1] - part[:, 0]


def _hot_share(logits: np.ndarray, k: int, hot_mask: np.ndarray) -> float:
    top = np.argpartition(-logits, k - 1, axis=1)[:, :k]
    return float(hot_mask[top].mean())


def make_batch(wl: Workload | str, layer: Layer, T: int, batch_index: int = 0,
               seed: Optional[int] = None, gap_rule: bool = True) -> Batch:
    """x ~ N(0,1) in bf16 [T, d]; for the skewed workload also the logit bias.
    Rows failing the router-gap rule are redrawn from fresh counters."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    seed = wl.seed if seed is None else seed
    d, E, k = wl.d, wl.E, wl.k
    xs = _S_X + (batch_index << 20)
    x = normal_bf16(seed, xs, 0, T * d).reshape(T, d)
    wr = layer.w_router.astype(np.float64)
    base = _bf16_to_f64(x) @ wr.T if T > 0 else np.zeros((0, E))
    bias = None
    delta = 0.0
    hot = None
    if wl.skew and T > 0:
        u = 2.0 * uniform_f64(seed, _S_SKEW + batch_index, 0, T)
        order = np.argsort(uniform_f64(seed, _S_HOT, 0, E), kind="stable")
        hot = np.sort(order[:HOT_EXPERTS])
        hot_mask = np.zeros(E, bool)
        hot_mask[hot] = True
        lo, hi = 0.0, 64.0
        for _ in range(60):
            mid = 0.5 * (lo + hi)
            b = (mid * u)[:, None] * hot_mask[None, :]
            if _hot_share(base + b.astype(np.float32).astype(np.float64), k, hot_mask) < HOT_SHARE:
                lo = mid
            else:
                hi = mid
        delta = 0.5 * (lo + hi)
        bias = ((delta * u)[:, None] * hot_mask[None, :]).astype(np.float32)
    resampled = 0
    if gap_rule and T > 0 and E > k:
        logits = base + (bias.astype(np.float64) if bias is not None else 0.0)
        gen = 0
        bad = np.nonzero(_kth_gap(logits, k) < GAP_MIN)[0]
        while bad.size:
            gen += 1
            assert gen < 1000, "gap rule did not converge"
            for t in bad:
                x[t] = normal_bf16(seed, xs + gen, int(t) * d, d)
            rows = _bf16_to_f64(x[bad]) @ wr.T
            if bias is not None:
                rows = rows + bias[bad].astype(np.float64)
            logits[bad] = rows
            resampled += bad.size
            bad = bad[_kth_gap(logits[bad], k) < GAP_MIN]
    return Batch(np.ascontiguousarray(x), bias, resampled, delta, hot)
