#!/usr/bin/env python3
"""Benchmark of the MoE FFN layer forward on one MI355X.

One step = one forward of the whole layer (router, top-k, permute, gate/up +
SwiGLU, down, combine) over one batch of T synthetic tokens whose inputs are
already resident in HBM.  Default workload: the OLMoE-1B-7B-shaped decode
layer (d=2048, f=1024, 64 experts, top-8, e4m3 weights with 128x128 f32 block
scales, no renormalisation) at T=8 tokens.

Prints one JSON line with the throughput, the roofline of the dominant kernel
(its duration measured with HIP events recorded on the launch stream by the
library's own timing hooks) and the CPU oracle's throughput on a bounded
sample of the same workload on this host.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; achieved HBM GB/s (decode), MFMA TFLOPS (prefill)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the activation-quantised variant)
KERNEL_SOURCES = ["moe_common.h", "moe_route.h", "moe_decode.h", "moe_gemm.h", "moe_block.h", "moe_q8.h",
                  "moe_api.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_f32_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def expert_stage_bytes(wl, U, T):
    """Algorithmic bytes of the two expert kernels for one launch: every
    selected expert's weights once (codes + scales), activations in, results out."""
    d, f, k = wl.d, wl.f, wl.k
    S = T * k
    if wl.fmt == "e4m3":
        gu = 2 * (f * d + 4 * (f // 128) * (d // 128))
        dn = d * f + 4 * (d // 128) * (f // 128)
    else:  # fp4 codes + one scale byte per 32 (e2m1) or per 16 (nvfp4) inputs
        g = 32 if wl.fmt == "e2m1" else 16
        gu = 2 * (f * d // 2 + f * d // g)
        dn = d * f // 2 + d * f // g
    gateup = U * gu + T * d * 2 + S * f * 2          # weights, x rows, h (bf16) out
    down = U * dn + S * f * 2 + S * d * 4            # weights, h in, y (f32) out
    return gateup, down


COPY_BYTES = 512 * 2 ** 20


def copy_probe():
    """A plain device-to-device copy of COPY_BYTES, 20 times: the reference for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_BYTES, "launches": 20}))


def _pmc_means(path, counter):
    """Mean counter value per dispatch, by kernel name, from a rocprofv3 CSV."""
    import csv
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(args):
    """profiles/traffic.json from four rocprofv3 --pmc CSVs (FETCH_SIZE and
    WRITE_SIZE of the benchmark, then of --copy-probe).  Each counter is scaled
    by the ratio of the copy's known bytes to what the counter read for it."""
    fetch, write, cfetch, cwrite = args.write_traffic
    def copy_kib(path, counter):
        m = _pmc_means(path, counter)
        k = [v for n, v in m.items() if "copyBuffer" in n or "copy" in n.lower()]
        return max(k)
    f_fetch = COPY_BYTES / (copy_kib(cfetch, "FETCH_SIZE") * 1024.0)
    f_write = COPY_BYTES / (copy_kib(cwrite, "WRITE_SIZE") * 1024.0)
    mf, mw = _pmc_means(fetch, "FETCH_SIZE"), _pmc_means(write, "WRITE_SIZE")
    key = args.traffic_key
    kern = args.traffic_kernel
    names = [n for n in mf if kern in n]
    assert names, f"no kernel matching {kern}"
    name = names[0]
    fb = mf[name] * 1024.0 * f_fetch
    wb = mw.get(name, 0.0) * 1024.0 * f_write
    out = {}
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            out = json.load(f)
    out.setdefault("entries", {})[key] = {
        "kernel": name, "kernel_source": kernel_source_hash(),
        "fetch_kib_per_launch": round(mf[name], 1), "write_kib_per_launch": round(mw.get(name, 0.0), 1),
        "copy_scale_fetch": round(f_fetch, 4), "copy_scale_write": round(f_write, 4),
        "bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb), "write_bytes": int(wb)}
    with open(args.traffic, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out["entries"][key]))


def bench_block(args, wl, T, layer, xs, Ws, copies, run, outs, stream, moe, np, torch, synth,
                DeviceWeights, Runner, to_dev):
    """One step = RMSNorm of the bf16 hidden rows -> the routed layer on them ->
    the dense branch (a one-expert top-1 plan, weight exactly 1) -> the add of
    both into the residual stream.  Each piece timed with events on `stream`."""
    d = wl.d
    dwl = synth.Workload(wl.name + "-dense", d, wl.f, 1, 1, wl.fmt, True, (), False, wl.seed + 100)
    dl = synth.make_layer(dwl)
    WD = DeviceWeights.upload(dl.w_router, dl.gate.q, dl.gate.s, dl.up.q, dl.up.s, dl.down.q,
                              dl.down.s)
    WDs = [WD] + [DeviceWeights(*(t.clone() for t in (WD.w_router, WD.gate_q, WD.gate_s, WD.up_q,
                                                      WD.up_s, WD.down_q, WD.down_s)))
                  for _ in range(copies - 1)]
    dense = Runner(d, wl.f, 1, 1, wl.fmt, True, T)
    douts = dense.outputs(T)
    rng = np.random.default_rng(wl.seed)
    gamma = to_dev((np.frombuffer(rng.uniform(0.5, 1.5, d).astype(np.float32).tobytes(), np.uint32)
                    >> 16).astype(np.uint16))
    xn = torch.empty((T, d), dtype=torch.int16, device="cuda")
    hid = [x.clone() for x in xs]
    outb = torch.empty((T, d), dtype=torch.int16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    acc = np.zeros(4)

    def bstep(i, timed=False):
        j = i % len(xs)
        if timed:
            ev[0].record(stream)
        moe.moe_rmsnorm(hid[j], gamma, 1e-6, xn, stream)
        if timed:
            ev[1].record(stream)
        run.forward(Ws[i % copies], xn, None, outs, stream)
        if timed:
            ev[2].record(stream)
        dense.forward(WDs[i % copies], xn, None, douts, stream)
        if timed:
            ev[3].record(stream)
        moe.moe_residual_add(hid[j], outs["out"], douts["out"], outb, stream)
        if timed:
            ev[4].record(stream)

    for i in range(args.warmup):
        bstep(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        bstep(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_t = min(args.steps, 200)
    for i in range(n_t):
        bstep(i, True)
        ev[4].synchronize()
        acc += [ev[k].elapsed_time(ev[k + 1]) for k in range(4)]
    us = acc * 1e3 / n_t
    norm_bytes = 4 * T * d + 2 * d          # x in, xn out, gain
    add_bytes = 2 * T * d + 8 * T * d + 2 * T * d  # residual, two f32 terms, bf16 out
    return {
        "metric": "transformer-block MoE step tokens/s (RMSNorm + routed layer + dense branch + "
                  "residual add)",
        "value": round(T * args.steps / (t1 - t0), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 norm/add, layer as the main line",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{wl.name} block: d={d} routed E={wl.E} k={wl.k} f={wl.f}, dense "
                               f"branch f={wl.f}, {wl.fmt}, T={T}", "tokens_per_step": T},
        "pieces_us": {"rmsnorm": round(us[0], 3), "routed_layer": round(us[1], 3),
                      "dense_branch": round(us[2], 3), "residual_add": round(us[3], 3)},
        "rmsnorm_roofline": {"bound": "hbm", "achieved": round(norm_bytes / (us[0] * 1e-6) / 1e9, 2),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(norm_bytes / (us[0] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes": norm_bytes},
        "residual_add_roofline": {"bound": "hbm",
                                  "achieved": round(add_bytes / (us[3] * 1e-6) / 1e9, 2),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(add_bytes / (us[3] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                                  "algorithmic_bytes": add_bytes},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="olmoe-decode")
    ap.add_argument("--tokens", type=int, default=8)
    ap.add_argument("--path", choices=["auto", "decode", "grouped"], default="auto")
    ap.add_argument("--batches", type=int, default=16, help="distinct x batches rotated")
    ap.add_argument("--copy-gib", type=float, default=1.0,
                    help="rotate weight copies until this many GiB are cycled (defeats the 256 MB "
                         "Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bounded CPU-oracle sample (0 disables)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured with rocprofv3 --pmc")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a known-size copy (counter calibration)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="write --traffic from rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--block", action="store_true",
                    help="time the transformer-block steps around the layer too: RMSNorm of the "
                         "hidden state, a dense (shared) SwiGLU branch of width f in the same "
                         "format, and the add into the bf16 residual stream")
    ap.add_argument("--act-quant", action="store_true",
                    help="the activation-quantised variant: x and h as e4m3 per 128-input group "
                         "(UE8M0 scales), block-scaled fp8 MFMA; opt-in, it changes results")
    ap.add_argument("--traffic-key", default="olmoe-decode/T=8/decode/gateup")
    ap.add_argument("--traffic-kernel", default="dec_mfma<0, true")
    args = ap.parse_args()

    if args.write_traffic:
        write_traffic(args)
        return
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this layer "
              "build runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import mixture_experts_layer_f32_amd as moe
    from mixture_experts_layer_f32_amd.device import DeviceWeights, Runner, to_dev

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    T = args.tokens
    t_gen = time.time()
    layer = synth.make_layer(wl)
    batches = [synth.make_batch(wl, layer, T, batch_index=i) for i in range(args.batches)]
    print(f"# generated {wl.name} layer + {len(batches)} batches of T={T} in "
          f"{time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    W0 = DeviceWeights.upload(layer.w_router, layer.gate.q, layer.gate.s, layer.up.q, layer.up.s,
                              layer.down.q, layer.down.s)
    layer_bytes = W0.nbytes()
    free, _ = torch.cuda.mem_get_info()
    copies = max(1, min(math.ceil(args.copy_gib * 2 ** 30 / layer_bytes),
                        int(0.5 * free // layer_bytes) + 1, 16))
    Ws = [W0] + [DeviceWeights(*(t.clone() for t in (W0.w_router, W0.gate_q, W0.gate_s, W0.up_q,
                                                      W0.up_s, W0.down_q, W0.down_s)))
                 for _ in range(copies - 1)]
    xs = [to_dev(b.x) for b in batches]
    biases = [to_dev(b.bias) if b.bias is not None else None for b in batches]
    path = {"auto": moe.MOE_PATH_AUTO, "decode": moe.MOE_PATH_DECODE,
            "grouped": moe.MOE_PATH_GROUPED}[args.path]
    act_fmt = moe.MOE_ACT_E4M3_G128 if args.act_quant else moe.MOE_ACT_BF16
    run = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T, path, act_fmt=act_fmt)
    outs = run.outputs(T)
    used_path = "decode" if moe.moe_plan_path(run.plan, T) == moe.MOE_PATH_DECODE else "grouped"
    # expert-stage arithmetic (the router is f32 throughout): bf16 products
    # into f32, by MFMA except in the decode matvec, which the plan picks for
    # one token (or always, under MOE_DEC_KERNEL=0)
    mfma = used_path == "grouped" or (os.environ.get("MOE_DEC_KERNEL", "1") != "0"
                                      and T >= int(os.environ.get("MOE_DEC_MFMA_MIN_T", "2")))
    dtype = "bf16-mfma/f32-acc" if mfma else "bf16-dot2/f32-acc"
    if args.act_quant and used_path == "grouped":
        dtype = "e4m3xe4m3-mfma/f32-acc" if wl.fmt == "e4m3" else "e4m3xe2m1-mfma/f32-acc"
    elif args.act_quant:  # the decode kernels on the quantised activations as bf16
        dtype = "e4m3-act-dequantised/" + dtype
    stream = torch.cuda.current_stream()

    def step(i):
        run.forward(Ws[i % copies], xs[i % len(xs)], biases[i % len(xs)], outs, stream)

    if args.block:
        block_line = bench_block(args, wl, T, layer, xs, Ws, copies, run, outs, stream, moe, np,
                                 torch, synth, DeviceWeights, Runner, to_dev)
        print(json.dumps(block_line), flush=True)
        return

    # distinct experts per batch (U) from the GPU's own counts
    Us = []
    for i in range(len(xs)):
        step(i)
        torch.cuda.synchronize()
        Us.append(int((outs["counts"] > 0).sum().item()))
    U = float(np.mean(Us))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = T * args.steps / (t1 - t0)

    # live per-stage durations: HIP events recorded by the library on `stream`
    moe.moe_timing_enable(run.plan, moe.STAGES, max_forwards=args.steps)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    stage_ms, n_fw = moe.moe_timing_collect(run.plan)
    t3 = time.perf_counter()
    moe.moe_timing_disable(run.plan)
    stage_avg_us = {k: 1e3 * v / n_fw for k, v in stage_ms.items()}
    timed_ms_per_step = (t3 - t2) * 1e3 / args.steps

    gu_bytes, dn_bytes = expert_stage_bytes(wl, U, T)
    S = T * wl.k
    flops = {"gateup": 4.0 * S * wl.d * wl.f, "down": 2.0 * S * wl.d * wl.f}
    nbytes = {"gateup": gu_bytes, "down": dn_bytes}
    dom = max(("gateup", "down"), key=lambda s: stage_avg_us[s])
    dur_s = stage_avg_us[dom] * 1e-6
    intensity = flops[dom] / nbytes[dom]
    peak_mfma = PEAK_FP8_TFLOPS if args.act_quant and used_path == "grouped" else PEAK_BF16_TFLOPS
    if intensity > peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved, peak, unit, bound = flops[dom] / dur_s / 1e12, peak_mfma, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = nbytes[dom] / dur_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"

    traffic = None
    ksrc = kernel_source_hash()
    key = f"{wl.name}/T={T}/{used_path}{'-q8' if args.act_quant else ''}/{dom}"
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            tr = json.load(f)
        ent = tr.get("entries", {}).get(key)
        if ent and ent.get("kernel_source") == ksrc:
            traffic = ent["bytes_per_launch"]

    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                "kernel_us": round(stage_avg_us[dom], 3),
                "algorithmic_bytes": int(nbytes[dom]), "algorithmic_flops": int(flops[dom])}

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max([p.get("num_threads", 1) for p in threadpool_info()
                         if p.get("user_api") == "blas"] or [1])
        except Exception:  # noqa: BLE001
            cores = 1
        M = lambda m: oracle.Mat(m.q, m.s, m.K)  # noqa: E731
        done, tok, tc0 = 0, 0, time.perf_counter()
        while True:
            b = batches[done % len(batches)]
            oracle.moe_forward(b.x, layer.w_router, b.bias, M(layer.gate), M(layer.up),
                               M(layer.down), wl.k, wl.renorm, wl.fmt, act_quant=args.act_quant)
            done += 1
            tok += T
            if time.perf_counter() - tc0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - tc0
        cpu = {"value": round(tok / el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"{done} full forwards of T={T} tokens of the {wl.name} workload "
                         f"({el:.1f} s, float64 numpy oracle)"}

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; random-init weights quantised to the workload's format)",
        "config": {
            "workload": f"{wl.name}: d={wl.d} f={wl.f} E={wl.E} k={wl.k} {wl.fmt} "
                        f"renorm={int(wl.renorm)}, T={T} tokens per step",
            "tokens_per_step": T,
            "path": used_path,
            "weights": {"e4m3": "e4m3 + f32 128x128 block scales",
                        "e2m1": "e2m1 + ue8m0 per 32",
                        "nvfp4": "e2m1 + e4m3 per 16 (nvfp4)"}[wl.fmt],
            "activations": "e4m3 per 128-input group, ue8m0 scales" if args.act_quant else "bf16",
            "distinct_experts_per_step": U,
            "weight_copies_rotated": copies,
            "x_batches_rotated": len(xs),
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages_us": {k: round(v, 3) for k, v in stage_avg_us.items()},
        "ms_per_step_with_stage_events": round(timed_ms_per_step, 5),
        "kernel_source": ksrc,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
