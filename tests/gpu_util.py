"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle on the same seeded inputs."""
import os
import sys
import time

import numpy as np

import oracle
import synth

# Output tolerance: max|err| <= 1e-2 * RMS(out) and sum|err| / sum|out| <= 1e-3.
MAX_ERR_RMS = 1e-2
MEAN_REL = 1e-3

# The activation-quantised variant end to end against the oracle's own
# quantised layer, when the grouped path's fp8 x fp8 MFMA computes h: that
# MFMA rounds its 64-product sums inside the instruction (about 2^-14 of the
# sum), so a fraction p_h of h lands one bf16 step from the oracle's h
# (asserted <= 10% by check_h_q8).  h is then quantised to e4m3 with 16 bf16
# steps per e4m3 step, so about p_h / 16 of the codes move by one e4m3 step
# (2^-4 to 2^-3 of the value).  Each moved code adds an independent term to
# out; the relative RMS error is sqrt(p_h / 16 * (2^-3.5)^2) = 0.022 sqrt(p_h),
# 7e-3 at p_h = 10%: the mean relative bound is 1e-2 (also the size of the
# shift the pages measured for quantised activations).  One moved code in a
# slot moves one output by at most 2^-3 |h_i| |W_d[m, i]| w_j, which against
# RMS(out) ~ sqrt(f) RMS(h) RMS(W_d) is 2^-3 * 4 * 4 / sqrt(f) (4-sigma h and
# weight) = 0.11 at the narrowest tested width f = 320: max|err| <= 0.1 RMS.
ACTQ_MAX_ERR_RMS = 1e-1
ACTQ_MEAN_REL = 1e-2

# CPU threads for the oracle's per-expert loop (full-size cases)
ORACLE_WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def omat(m):
    return oracle.Mat(m.q, m.s, m.K)


def oracle_run(wl, layer, batch, tokens=None, act_quant=False):
    return oracle.moe_forward(batch.x, layer.w_router, batch.bias, omat(layer.gate),
                              omat(layer.up), omat(layer.down), wl.k, wl.renorm, wl.fmt,
                              tokens=tokens, act_quant=act_quant, workers=ORACLE_WORKERS)


def device_weights(layer):
    from mixture_experts_layer_f32_amd.device import DeviceWeights
    return DeviceWeights.upload(layer.w_router, layer.gate.q, layer.gate.s, layer.up.q,
                                layer.up.s, layer.down.q, layer.down.s)


def gpu_run(wl, W, batch, path, runner=None, max_tokens=None, options=None):
    """Returns (numpy outputs, runner).  options: {MOE_OPT_*: value} set on the plan."""
    import torch
    from mixture_experts_layer_f32_amd.device import Runner, to_dev
    T = batch.x.shape[0]
    if runner is None:
        runner = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, max_tokens or max(T, 1), path,
                        options=options)
    outs = runner.outputs(T)
    x = to_dev(batch.x)
    bias = to_dev(batch.bias) if batch.bias is not None else None
    runner.forward(W, x, bias, outs)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in outs.items()}
    res["h"] = runner.h(T).cpu().numpy().view(np.uint16) if T > 0 else None
    return res, runner


def check_routing(g, r):
    assert np.array_equal(g["topk_ids"], r.ids), "expert ids differ"
    assert np.array_equal(g["counts"], r.counts), "counts differ"
    assert np.array_equal(g["offsets"], r.offsets), "offsets differ"
    assert np.array_equal(g["perm"], r.perm), "permutation differs"
    np.testing.assert_allclose(g["topk_w"], r.w, rtol=2e-5, atol=1e-7)


def out_errors(got, ref):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(err.max()), rms, float(err.sum() / max(np.abs(ref).sum(), 1e-300))


def check_out(got, ref):
    assert np.all(np.isfinite(got)), "non-finite outputs"
    mx, rms, mrel = out_errors(got, ref)
    assert mx <= MAX_ERR_RMS * rms, f"max|err| {mx:.3e} > 1e-2 * rms {rms:.3e}"
    assert mrel <= MEAN_REL, f"mean relative error {mrel:.3e}"
    return mx, rms, mrel


def check_out_actq(got, ref):
    """The activation-quantised layer end to end against the oracle's own
    quantised layer (bounds derived above)."""
    assert np.all(np.isfinite(got)), "non-finite outputs"
    mx, rms, mrel = out_errors(got, ref)
    assert mx <= ACTQ_MAX_ERR_RMS * rms, f"max|err| {mx:.3e} > 0.1 * rms {rms:.3e}"
    assert mrel <= ACTQ_MEAN_REL, f"mean relative error {mrel:.3e}"
    return mx, rms, mrel


def check_h(h_gpu, h_ref, min_equal=0.98):
    """h is rounded to bf16 on both sides from sums taken in different orders:
    values may differ by one bf16 unit in the last place (rarely), and near
    zero the sign of a product whose factor is itself ~0 may differ."""
    g = oracle.bf16_to_f64(h_gpu)
    r = oracle.bf16_to_f64(h_ref)
    err = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 0.0
    tol = 2.0 ** -7 * np.maximum(np.abs(g), np.abs(r)) + 1e-5 * rms
    bad = err > tol
    assert not bad.any(), f"{int(bad.sum())} h values differ by more than 1 bf16 ulp"
    eq = float((h_gpu == h_ref).mean()) if h_ref.size else 1.0
    assert eq >= min_equal, f"only {eq:.4f} of h values equal"
    return eq
