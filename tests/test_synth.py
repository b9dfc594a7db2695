"""The seeded input generator: determinism, the acceptance rules of the
workloads, and the shapes it hands to both sides."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _digest_script(name, T):
    return ("import hashlib, synth; L = synth.make_layer('%s'); B = synth.make_batch('%s', L, %d); "
            "h = hashlib.sha256(); [h.update(a.tobytes()) for a in (L.w_router, L.gate.q, L.gate.s, "
            "L.up.q, L.down.q, L.down.s, B.x)]; print(h.hexdigest())" % (name, name, T))


@pytest.mark.parametrize("name,T", [("tiny", 4), ("olmoe-decode", 8)])
def test_bytes_independent_of_thread_count(name, T):
    outs = []
    for n in ("1", "7"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        r = subprocess.run([sys.executable, "-c", _digest_script(name, T)], cwd=ROOT, env=env,
                           capture_output=True, text=True, check=True)
        outs.append(r.stdout.strip())
    assert outs[0] == outs[1]


def test_seed_changes_bytes():
    a = synth.make_layer("tiny")
    b = synth.make_layer("tiny", seed=4242)
    assert not np.array_equal(a.gate.q, b.gate.q)


def _bf(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("name,T", [("tiny", 4), ("olmoe-decode", 8), ("olmoe-prefill-skewed", 512)])
def test_gap_rule_holds(name, T):
    wl = synth.WORKLOADS[name]
    L = synth.make_layer(wl)
    B = synth.make_batch(wl, L, T)
    l = _bf(B.x) @ L.w_router.astype(np.float64).T
    if B.bias is not None:
        l = l + B.bias
    s = -np.sort(-l, axis=1)
    assert np.all(s[:, wl.k - 1] - s[:, wl.k] >= synth.GAP_MIN)


def test_skew_sends_about_30_percent_to_hot_experts():
    wl = synth.WORKLOADS["olmoe-prefill-skewed"]
    L = synth.make_layer(wl)
    for T in wl.batches:
        B = synth.make_batch(wl, L, T)
        l = _bf(B.x) @ L.w_router.astype(np.float64).T + B.bias
        top = np.argsort(-l, axis=1)[:, :wl.k]
        share = np.isin(top, B.hot).mean()
        assert abs(share - 0.30) <= 0.01, share
        assert B.hot.size == 8 and B.delta > 0


def test_x_is_standard_normal_bf16():
    wl = synth.WORKLOADS["olmoe-decode"]
    L = synth.make_layer(wl)
    B = synth.make_batch(wl, L, 8)
    xf = _bf(B.x)
    assert B.x.dtype == np.uint16 and B.x.shape == (8, 2048)
    assert abs(xf.mean()) < 0.05 and abs(xf.std() - 1) < 0.05


def test_weight_scales_follow_recipe():
    """e4m3: scale = amax/448 of each 128x128 block, so every block has a code of
    magnitude 448 (0x7E); e2m1: 2^E >= amax/6 > 2^(E-1), so each 32-group's largest
    scaled magnitude lies in (3, 6] and is coded as 3, 4 or 6."""
    L = synth.make_layer("tiny")
    q = L.gate.q[0]
    for bn in range(2):
        for bk in range(2):
            blk = q[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]
            assert ((blk & 0x7F) == 0x7E).any()
    wl = synth.Workload("e2m1-tiny", 64, 64, 2, 1, "e2m1", True, (1,), False, 5)
    L = synth.make_layer(wl)
    codes = np.stack([L.gate.q[0] & 0xF, L.gate.q[0] >> 4], -1).reshape(64, 64)
    mags = (codes & 0x7).reshape(64, 2, 32).max(axis=2)
    assert np.all(mags >= 5)   # codes 5, 6, 7 are 3.0, 4.0, 6.0
