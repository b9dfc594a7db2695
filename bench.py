#!/usr/bin/env python3
"""Benchmark of the MoE FFN layer forward on one MI355X.

One step = one forward of the whole layer (router, top-k, permute, gate/up +
SwiGLU, down, combine) over one batch of T synthetic tokens whose inputs are
already resident in HBM.  The headline workload is the largest single-GPU
layer: d=7168, f=2048, 256 experts, top-8 renormalised, e4m3 weights with
128x128 f32 block scales (11.3 GB), at T=4096 tokens.  The same run measures
every (layer, T) point of the five workloads (`per_config`).

Per point: tokens/s from the wall clock over the timed steps (eager launches),
the per-step device span (HIP events before and after each step on the launch
stream; median and min), a HIP-graph replay of the captured forward (launch
overhead removed), an A/A rerun of the timed loop, the dominant kernel's
duration (HIP events around that stage only, recorded by the library on the
launch stream) with its roofline fraction, and the CPU oracle on a bounded
sample of the same batch on this host.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
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

# The five workloads at the token counts they are defined with; the headline
# is the largest layer at its largest batch.
POINTS = [("tiny", 4), ("olmoe-decode", 1), ("olmoe-decode", 8), ("olmoe-prefill-skewed", 512),
          ("olmoe-prefill-skewed", 2048), ("large-e4m3", 1), ("large-e4m3", 64),
          ("large-e4m3", 4096), ("fp4-e2m1", 1), ("fp4-e2m1", 16), ("fp4-e2m1", 1024)]
HEADLINE = ("large-e4m3", 4096)
# tokens of each batch the CPU oracle evaluates (its routing covers the whole
# batch; the expert step and the combine only these tokens)
ORACLE_TOKENS = {("tiny", 4): 4, ("olmoe-decode", 1): 1, ("olmoe-decode", 8): 8,
                 ("olmoe-prefill-skewed", 512): 4, ("olmoe-prefill-skewed", 2048): 4,
                 ("large-e4m3", 1): 1, ("large-e4m3", 64): 2, ("large-e4m3", 4096): 8,
                 ("fp4-e2m1", 1): 1, ("fp4-e2m1", 16): 2, ("fp4-e2m1", 1024): 4}


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


def roofline_of(wl, U, T, stage, us, act_quant=False, grouped=True):
    """Roofline of one expert stage from its duration: HBM or MFMA by the
    stage's arithmetic intensity against the balance point of its peak."""
    gu_bytes, dn_bytes = expert_stage_bytes(wl, U, T)
    S = T * wl.k
    flops = {"gateup": 4.0 * S * wl.d * wl.f, "down": 2.0 * S * wl.d * wl.f}[stage]
    nbytes = {"gateup": gu_bytes, "down": dn_bytes}[stage]
    dur_s = us * 1e-6
    peak_mfma = PEAK_FP8_TFLOPS if act_quant and grouped else PEAK_BF16_TFLOPS
    if flops / nbytes > peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved, peak, unit, bound = flops / dur_s / 1e12, peak_mfma, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = nbytes / dur_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "kernel": stage, "kernel_us": round(us, 3),
            "algorithmic_bytes": int(nbytes), "algorithmic_flops": int(flops)}


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


def host_cpu():
    """CPU model of this host and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def log(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ one layer on the device


class DeviceLayer:
    """A workload's layer generated on the host, uploaded, and copied until at
    least `copy_gib` GiB of weights are cycled (so consecutive steps do not
    find their experts in the 256 MB Infinity Cache)."""

    def __init__(self, wl, copy_gib):
        import torch
        import synth
        from mixture_experts_layer_f32_amd.device import DeviceWeights
        t0 = time.time()
        self.wl = wl
        self.layer = synth.make_layer(wl)
        W0 = DeviceWeights.upload(self.layer.w_router, self.layer.gate.q, self.layer.gate.s,
                                  self.layer.up.q, self.layer.up.s, self.layer.down.q,
                                  self.layer.down.s)
        nbytes = W0.nbytes()
        free, _ = torch.cuda.mem_get_info()
        self.copies = max(1, min(math.ceil(copy_gib * 2 ** 30 / nbytes),
                                 int(0.5 * free // nbytes) + 1, 16))
        self.Ws = [W0] + [DeviceWeights(*(t.clone() for t in (W0.w_router, W0.gate_q, W0.gate_s,
                                                               W0.up_q, W0.up_s, W0.down_q,
                                                               W0.down_s)))
                          for _ in range(self.copies - 1)]
        log(f"{wl.name}: layer generated and uploaded ({nbytes / 1e9:.2f} GB x {self.copies}) "
            f"in {time.time() - t0:.1f}s")


def oracle_sample(wl, layer, batch, n_tok, act_quant, workers):
    """The CPU oracle on the first n_tok tokens of the batch (routing over the
    whole batch): (tokens/s, seconds, tokens)."""
    import oracle
    from threadpoolctl import threadpool_limits
    M = lambda m: oracle.Mat(m.q, m.s, m.K)  # noqa: E731
    toks = list(range(min(n_tok, batch.x.shape[0])))
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        oracle.moe_forward(batch.x, layer.w_router, batch.bias, M(layer.gate), M(layer.up),
                           M(layer.down), wl.k, wl.renorm, wl.fmt, tokens=toks,
                           act_quant=act_quant, workers=workers)
        el = time.perf_counter() - t0
    return len(toks) / el, el, len(toks)


def measure(dl, T, args, act_quant=False, path_opt="auto", oracle_tokens=0, oracle_1thread=False,
            steps=None):
    """All timings of one (layer, T) point; returns a dict.  `steps` timed
    steps (default: --steps; for the other points of the default run enough
    to cover about 0.2 s, at least --steps and at most 1000)."""
    import numpy as np
    import torch
    import synth
    import mixture_experts_layer_f32_amd as moe
    from mixture_experts_layer_f32_amd.device import Runner, to_dev
    wl, layer, Ws, copies = dl.wl, dl.layer, dl.Ws, dl.copies
    nb = args.batches if args.batches else (16 if T <= 64 else 4)
    t0 = time.time()
    batches = [synth.make_batch(wl, layer, T, batch_index=i) for i in range(nb)]
    xs = [to_dev(b.x) for b in batches]
    biases = [to_dev(b.bias) if b.bias is not None else None for b in batches]
    path = {"auto": moe.MOE_PATH_AUTO, "decode": moe.MOE_PATH_DECODE,
            "grouped": moe.MOE_PATH_GROUPED}[path_opt]
    opts = {moe.MOE_OPT_GROUPED_TILE: args.tile} if args.tile else None
    run = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T, path,
                 act_fmt=moe.MOE_ACT_E4M3_G128 if act_quant else moe.MOE_ACT_BF16, options=opts)
    outs = run.outputs(T)
    used_path = "decode" if moe.moe_plan_path(run.plan, T) == moe.MOE_PATH_DECODE else "grouped"
    stream = torch.cuda.current_stream()

    def step(i):
        run.forward(Ws[i % copies], xs[i % nb], biases[i % nb], outs, stream)

    # distinct experts per batch (U) from the GPU's own counts
    Us = []
    for i in range(nb):
        step(i)
        torch.cuda.synchronize()
        Us.append(int((outs["counts"] > 0).sum().item()))
    U = float(np.mean(Us))
    warm = max(args.warmup, 1)
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    per_step = (time.perf_counter() - t_w) / warm
    if steps is None:
        steps = args.steps
    elif steps < 0:
        steps = int(min(1000, max(args.steps, 0.2 / max(per_step, 1e-6))))
    n = steps

    # timed eager loop (twice: A/A): wall clock only, nothing recorded in between
    def timed_loop():
        torch.cuda.synchronize()
        t_a = time.perf_counter()
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t_a) * 1e3 / n

    wall_a = timed_loop()
    wall_b = timed_loop()
    # device span of each step: HIP events before and after it on the stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for i in range(n):
        ev[2 * i].record(stream)
        step(i)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    spans = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]

    # dominant expert stage: all stages once to find it, then that stage alone
    moe.moe_timing_enable(run.plan, moe.STAGES, max_forwards=n)
    for i in range(n):
        step(i)
    stage_ms, n_fw = moe.moe_timing_collect(run.plan)
    moe.moe_timing_disable(run.plan)
    stages_us = {k: 1e3 * v / n_fw for k, v in stage_ms.items()}
    dom = max(("gateup", "down"), key=lambda s: stages_us[s])
    moe.moe_timing_enable(run.plan, (dom,), max_forwards=n)
    for i in range(n):
        step(i)
    dom_ms, n_fw = moe.moe_timing_collect(run.plan)
    moe.moe_timing_disable(run.plan)
    dom_us = 1e3 * dom_ms[dom] / n_fw

    # HIP-graph replay: one captured forward per (weight copy, x batch) pair,
    # replayed round-robin between two events
    n_g = max(1, min(copies, nb, 4))
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        run.forward(Ws[0], xs[0], biases[0], outs, side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    for gi in range(n_g):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run.forward(Ws[gi], xs[gi], biases[gi], outs, torch.cuda.current_stream())
        graphs.append(g)
    torch.cuda.synchronize()
    for gi in range(n_g):
        graphs[gi].replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        graphs[i % n_g].replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / n
    del graphs

    roof = roofline_of(wl, U, T, dom, dom_us, act_quant, used_path == "grouped")
    res = {
        "workload": f"{wl.name}: d={wl.d} f={wl.f} E={wl.E} k={wl.k} {wl.fmt} "
                    f"renorm={int(wl.renorm)}, T={T}",
        "name": wl.name, "T": T, "path": used_path, "tokens_per_s": round(T / (wall_a * 1e-3), 2),
        "ms_per_step": round(wall_a, 5), "steps": n, "warmup": warm,
        "aa_rerun": {"tokens_per_s": round(T / (wall_b * 1e-3), 2), "ms_per_step": round(wall_b, 5),
                     "ratio": round(wall_b / wall_a, 4)},
        "device_span_ms": {"median": round(statistics.median(spans), 5),
                           "min": round(min(spans), 5)},
        "graph_replay": {"ms_per_step": round(graph_ms, 5),
                         "tokens_per_s": round(T / (graph_ms * 1e-3), 2), "graphs": n_g},
        "stages_us": {k: round(v, 3) for k, v in stages_us.items()},
        "distinct_experts_per_step": U, "weight_copies_rotated": copies, "x_batches_rotated": nb,
        "roofline": roof,
    }
    if oracle_tokens:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        tps, el, n = oracle_sample(wl, layer, batches[0], oracle_tokens, act_quant, workers)
        res["oracle"] = {"tokens_per_s": round(tps, 3), "seconds": round(el, 2), "tokens": n,
                         "threads": workers}
        if oracle_1thread:
            tps1, el1, _ = oracle_sample(wl, layer, batches[0], oracle_tokens, act_quant, 1)
            res["oracle"]["tokens_per_s_1thread"] = round(tps1, 3)
            res["oracle"]["seconds_1thread"] = round(el1, 2)
    log(f"{wl.name} T={T} ({used_path}): {res['tokens_per_s']:.0f} tokens/s, "
        f"{wall_a * 1e3:.1f} us/step (A/A {wall_b * 1e3:.1f}), graph {graph_ms * 1e3:.1f} us, "
        f"{dom} {dom_us:.1f} us = {roof['frac']:.3f} {roof['bound']} ({time.time() - t0:.1f}s)")
    return res


def traffic_for(args, wl, T, path, dom, act_quant):
    """HBM bytes per launch of the dominant kernel from profiles/traffic.json,
    if measured on the current kernel sources; else None."""
    key = f"{wl.name}/T={T}/{path}{'-q8' if act_quant else ''}/{dom}"
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            ent = json.load(f).get("entries", {}).get(key)
        if ent and ent.get("kernel_source") == kernel_source_hash():
            return ent["bytes_per_launch"]
    return None


def bench_block(args, wl, T, dl):
    """One step = RMSNorm of the bf16 hidden rows -> the layer with its shared
    expert (one launch set: the shared expert's rows ride in the routed
    experts' tile lists) -> the combine, which also adds the residual and
    writes bf16.  The same block run unfused (routed layer, shared expert as a
    one-expert plan, separate add) is timed beside it."""
    import numpy as np
    import torch
    import synth
    import mixture_experts_layer_f32_amd as moe
    from mixture_experts_layer_f32_amd.device import DeviceWeights, Runner, to_dev
    d = wl.d
    layer, Ws, copies = dl.layer, dl.Ws, dl.copies
    batches = [synth.make_batch(wl, layer, T, batch_index=i) for i in range(4)]
    xs = [to_dev(b.x) for b in batches]
    stream = torch.cuda.current_stream()
    swl = synth.Workload(wl.name + "-shared", d, wl.f, 1, 1, wl.fmt, True, (), False, wl.seed + 100)
    slay = synth.make_layer(swl)
    WS = DeviceWeights.upload(slay.w_router, slay.gate.q, slay.gate.s, slay.up.q, slay.up.s,
                              slay.down.q, slay.down.s)
    WSs = [WS] + [DeviceWeights(*(t.clone() for t in (WS.w_router, WS.gate_q, WS.gate_s, WS.up_q,
                                                      WS.up_s, WS.down_q, WS.down_s)))
                  for _ in range(copies - 1)]
    fused = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T, shared_expert=True)
    fouts = fused.outputs(T)
    del fouts["out"]  # the bf16 block output only
    run = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T)
    outs = run.outputs(T)
    dense = Runner(d, wl.f, 1, 1, wl.fmt, True, T)
    douts = dense.outputs(T)
    rng = np.random.default_rng(wl.seed)
    gamma = to_dev((np.frombuffer(rng.uniform(0.5, 1.5, d).astype(np.float32).tobytes(), np.uint32)
                    >> 16).astype(np.uint16))
    xn = torch.empty((T, d), dtype=torch.int16, device="cuda")
    hid = [x.clone() for x in xs]
    outb = torch.empty((T, d), dtype=torch.int16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]

    def fstep(i, timed=False):
        j = i % len(xs)
        if timed:
            ev[0].record(stream)
        moe.moe_rmsnorm(hid[j], gamma, 1e-6, xn, stream)
        if timed:
            ev[1].record(stream)
        fused.forward_block(Ws[i % copies], WSs[i % copies], xn, None, hid[j], outb, fouts, stream)
        if timed:
            ev[2].record(stream)

    def ustep(i, timed=False):
        j = i % len(xs)
        moe.moe_rmsnorm(hid[j], gamma, 1e-6, xn, stream)
        if timed:
            ev[3].record(stream)
        run.forward(Ws[i % copies], xn, None, outs, stream)
        dense.forward(WSs[i % copies], xn, None, douts, stream)
        if timed:
            ev[4].record(stream)
        moe.moe_residual_add(hid[j], outs["out"], douts["out"], outb, stream)
        if timed:
            ev[5].record(stream)

    def wall(step):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    tf = wall(fstep)
    tu = wall(ustep)
    n_t = min(args.steps, 200)
    acc = np.zeros(4)
    for i in range(n_t):
        fstep(i, True)
        ev[2].synchronize()
        ustep(i, True)
        ev[5].synchronize()
        acc += [ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]),
                ev[3].elapsed_time(ev[4]), ev[4].elapsed_time(ev[5])]
    us = acc * 1e3 / n_t
    norm_bytes = 4 * T * d + 2 * d          # x in, xn out, gain
    return {
        "metric": "transformer-block MoE step tokens/s (RMSNorm + routed layer with its shared "
                  "expert + residual add)",
        "value": round(T * args.steps / tf, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(tf * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{wl.name} block: d={d} routed E={wl.E} k={wl.k} f={wl.f}, shared "
                               f"expert f={wl.f}, {wl.fmt}, T={T}", "tokens_per_step": T},
        "pieces_us": {"rmsnorm": round(us[0], 3), "layer_with_shared_and_add": round(us[1], 3)},
        "unfused": {"ms_per_step": round(tu * 1e3 / args.steps, 5),
                    "tokens_per_s": round(T * args.steps / tu, 2),
                    "pieces_us": {"routed_layer_plus_shared_plan": round(us[2], 3),
                                  "residual_add": round(us[3], 3)}},
        "rmsnorm_roofline": {"bound": "hbm", "achieved": round(norm_bytes / (us[0] * 1e-6) / 1e9, 2),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(norm_bytes / (us[0] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes": norm_bytes},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="measure this workload only (default: the headline plus every point)")
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--path", choices=["auto", "decode", "grouped"], default="auto")
    ap.add_argument("--batches", type=int, default=0,
                    help="distinct x batches rotated (0: 16 up to 64 tokens, else 4)")
    ap.add_argument("--copy-gib", type=float, default=1.0,
                    help="rotate weight copies until this many GiB are cycled (defeats the 256 MB "
                         "Infinity Cache)")
    ap.add_argument("--no-oracle", action="store_true", help="skip the CPU oracle samples")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured with rocprofv3 --pmc")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a known-size copy (counter calibration)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="write --traffic from rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--block", action="store_true",
                    help="time the transformer-block step: RMSNorm of the hidden state, then the "
                         "layer with a shared SwiGLU expert of width f in the same format inside "
                         "the routed launches and the add into the bf16 residual stream inside "
                         "the combine; the unfused sequence is timed beside it")
    ap.add_argument("--act-quant", action="store_true",
                    help="the activation-quantised variant: x and h as e4m3 per 128-input group "
                         "(UE8M0 scales), block-scaled fp8 MFMA; opt-in, it changes results")
    ap.add_argument("--tile", type=int, default=0,
                    help="grouped-GEMM tile shape code (MOE_OPT_GROUPED_TILE; 0: by shape)")
    ap.add_argument("--traffic-key", default="large-e4m3/T=4096/grouped/gateup")
    ap.add_argument("--traffic-kernel", default="gemm_big<0, true")
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

    import torch
    import synth
    import mixture_experts_layer_f32_amd  # noqa: F401  (fails loudly without libmoe.so)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cpu_model, cpu_cores = host_cpu()

    if args.workload is not None:
        wl = synth.WORKLOADS[args.workload]
        T = args.tokens if args.tokens is not None else wl.batches[-1]
        points, head = [(wl.name, T)], (wl.name, T)
    else:
        points, head = list(POINTS), HEADLINE
    by_wl = {}
    for name, T in points:
        by_wl.setdefault(name, []).append(T)
    results = {}
    for name, Ts in by_wl.items():
        dl = DeviceLayer(synth.WORKLOADS[name], args.copy_gib)
        if args.block:
            print(json.dumps(bench_block(args, dl.wl, Ts[-1], dl)), flush=True)
            return
        for T in Ts:
            n_or = 0 if args.no_oracle else ORACLE_TOKENS.get((name, T), 4)
            steps = None
            if (name, T) != head:  # the other points: about 0.2 s of steps each
                steps = -1
            results[(name, T)] = measure(dl, T, args, args.act_quant, args.path, n_or,
                                         oracle_1thread=name in ("tiny", "olmoe-decode"),
                                         steps=steps)
        del dl
        torch.cuda.empty_cache()

    h = results[head]
    wl = synth.WORKLOADS[head[0]]
    grouped = h["path"] == "grouped"
    # dtype: the type the products are taken in; "arithmetic" says how
    dtype, arith = "bf16", "bf16 MFMA, f32 accumulate"
    if h["path"] == "decode" and head[1] < 2:
        arith = "bf16 dot2, f32 accumulate"
    if args.act_quant and grouped:
        dtype = "fp8"
        arith = "e4m3 x " + ("e4m3" if wl.fmt == "e4m3" else "e2m1") + " MFMA, f32 accumulate"
    elif args.act_quant:
        arith = "e4m3 activations dequantised to bf16; " + arith
    roof = dict(h["roofline"])
    roof["traffic"] = traffic_for(args, wl, head[1], h["path"], roof["kernel"], args.act_quant)
    cpu = None
    if "oracle" in h:
        o = h["oracle"]
        cpu = {"value": o["tokens_per_s"], "unit": "tokens/s", "cores": o["threads"],
               "kind": "oracle", "cpu_model": cpu_model, "cores_available": cpu_cores,
               "sample": f"the first {o['tokens']} tokens of a T={head[1]} batch of the {wl.name} "
                         f"workload (routing over all {head[1]} tokens; each touched expert "
                         f"dequantised once), {o['seconds']} s on {o['threads']} threads "
                         f"(float64 numpy oracle, BLAS 1 thread per worker)"}
    line = {
        "metric": METRIC,
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; random-init weights quantised to the workload's format)",
        "config": {
            "workload": h["workload"] + " tokens per step",
            "tokens_per_step": head[1],
            "path": h["path"],
            "weights": {"e4m3": "e4m3 + f32 128x128 block scales",
                        "e2m1": "e2m1 + ue8m0 per 32",
                        "nvfp4": "e2m1 + e4m3 per 16 (nvfp4)"}[wl.fmt],
            "activations": "e4m3 per 128-input group, ue8m0 scales" if args.act_quant else "bf16",
            "arithmetic": arith,
            "distinct_experts_per_step": h["distinct_experts_per_step"],
            "weight_copies_rotated": h["weight_copies_rotated"],
            "x_batches_rotated": h["x_batches_rotated"],
            "parallelism": "single GPU",
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "device_span_ms": h["device_span_ms"],
        "graph_replay": h["graph_replay"],
        "aa_rerun": h["aa_rerun"],
        "stages_us": h["stages_us"],
        "host": {"cpu_model": cpu_model, "cores_available": cpu_cores},
        "kernel_source": kernel_source_hash(),
    }
    if len(results) > 1:
        line["per_config"] = [{k: v for k, v in r.items() if k not in ("name",)}
                              for r in results.values()]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
