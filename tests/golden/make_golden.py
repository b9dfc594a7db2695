"""Writes tests/golden/tiny_canary.json: hashes of the oracle's result on the
tiny workload (d=256, 8 experts, top-2, f=256, 4 tokens).  Calls only the
oracle and the input generator.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def canary():
    wl = synth.WORKLOADS["tiny"]
    layer = synth.make_layer(wl)
    batch = synth.make_batch(wl, layer, wl.batches[0])
    M = lambda m: oracle.Mat(m.q, m.s, m.K)  # noqa: E731
    r = oracle.moe_forward(batch.x, layer.w_router, batch.bias, M(layer.gate), M(layer.up),
                           M(layer.down), wl.k, wl.renorm, wl.fmt)
    h = lambda a: hashlib.sha256(a.tobytes()).hexdigest()  # noqa: E731
    return {
        "workload": "tiny: d=256, f=256, E=8, k=2, e4m3, renormalised, T=4, seed 1000",
        "x_sha256": h(batch.x),
        "ids": r.ids.tolist(),
        "perm": r.perm.tolist(),
        "counts": r.counts.tolist(),
        "h_sha256": h(r.h),
        "out_sha256": h(r.out),
        "out_first_row_head": [float(v) for v in r.out[0, :4]],
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_canary.json")
    with open(path, "w") as f:
        json.dump(canary(), f, indent=1)
        f.write("\n")
    print("wrote", path)
