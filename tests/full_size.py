"""Shared body of the full-size parity tests: one layer of a named workload at
its real size, every token of the batch run through the GPU path and through
the oracle (its per-expert loop on several CPU threads), and compared
element by element: routing bit for bit, h for every slot, out for every
token.  The oracle's result for a batch is kept for the other path of the
same batch."""
import numpy as np

import synth
from gpu_util import (check_h, check_out, check_routing, device_weights, gpu_run, log,
                      oracle_run)


class FullSize:
    def __init__(self, name):
        self.wl = synth.WORKLOADS[name]
        self.layer = None
        self.W = None
        self._ref = {}

    def setup(self):
        wl = self.wl
        log(f"generating {wl.name} layer ({synth.expert_bytes(wl) * wl.E / 1e9:.1f} GB)")
        self.layer = synth.make_layer(wl)
        log("uploading")
        self.W = device_weights(self.layer)
        return self

    def teardown(self):
        self.W = None
        self._ref.clear()

    def oracle(self, T, act_quant=False):
        key = (T, act_quant)
        if key not in self._ref:
            self._ref.clear()  # one batch at a time: y of the largest case is ~2 GB
            batch = synth.make_batch(self.wl, self.layer, T)
            log(f"{self.wl.name} T={T}{' act-quant' if act_quant else ''}: oracle on every token")
            ref = oracle_run(self.wl, self.layer, batch, act_quant=act_quant)
            ref.y = None
            self._ref[key] = (batch, ref)
        return self._ref[key]

    def check(self, T, path):
        batch, ref = self.oracle(T)
        log(f"{self.wl.name} T={T} path={path}: gpu")
        g, _ = gpu_run(self.wl, self.W, batch, path)
        check_routing(g, ref)
        eq = check_h(g["h"], ref.h)
        mx, rms, mrel = check_out(g["out"], ref.out)
        log(f"all {T} tokens: h equal {eq:.4f}, max|err| {mx:.3e} rms {rms:.3e} "
            f"mean rel {mrel:.3e}")

    def check_act_quant(self, T, n_step=6):
        """The activation-quantised plan: every token end to end against the
        oracle's own quantised layer, and a seeded sample of tokens step by
        step (the oracle's down projection fed the GPU's h)."""
        from test_gpu_actquant import check_h_q8, check_out_q8_e2e, q8_reference, run_q8
        wl, L = self.wl, self.layer
        batch, ref = self.oracle(T, act_quant=True)
        log(f"{wl.name} act-quant T={T}: gpu")
        g = run_q8(wl, self.W, batch)
        check_routing(g, ref)
        eq = check_h_q8(g["h"], ref.h)
        mx, rms, mrel = check_out_q8_e2e(g, ref.out)
        rng = np.random.default_rng(T)
        toks = sorted({0, T - 1, *rng.choice(T, min(T, n_step) - 1 if T > 1 else 0,
                                               replace=False).tolist()})
        h_ref, out_ref = q8_reference(wl, L, batch, ref, g["h"], toks)
        mxs, _, mrels = check_out(g["out"][toks], out_ref)
        log(f"act-quant all {T} tokens ({g['path']}): h equal {eq:.4f}, end to end max|err| "
            f"{mx:.3e} rms {rms:.3e} mean rel {mrel:.3e}; tokens {toks} with the GPU's h: "
            f"max|err| {mxs:.3e} mean rel {mrels:.3e}")
