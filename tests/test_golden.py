"""Golden fixtures: numbers printed on the pages, and the canary hash of the
oracle's result on the tiny workload (regenerate with
tests/golden/make_golden.py only with a reason stated in the commit)."""
import json
import os

import numpy as np

import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def facts():
    with open(os.path.join(GOLD, "page_facts.json")) as f:
        return json.load(f)


def test_fp4_expert_bytes_match_page():
    F = facts()
    wl = synth.WORKLOADS["fp4-e2m1"]
    codes = 3 * wl.d * wl.f // 2          # two e2m1 codes per byte
    scales = 3 * wl.d * wl.f // 32        # one UE8M0 byte per 32 inputs
    assert codes + scales == synth.expert_bytes(wl) == 18_800_640
    assert round((codes + scales) / 2 ** 20, 2) == F["fp4_expert_mib"]["value"]
    assert round(codes / 1e6, 1) == F["fp4_expert_matrices_mb"]["value"]
    assert round(scales / 1e6, 1) == F["fp4_expert_scales_mb"]["value"]
    per_tok = F["fp4_bytes_per_token_gib"]
    assert wl.k == per_tok["experts_per_token"]
    assert round(wl.k * per_tok["layers"] * (codes + scales) / 2 ** 30, 1) == per_tok["value"]


def test_generated_fp4_layout_sizes():
    """The generator's arrays for the FP4 dims have exactly the page's bytes per expert."""
    wl = synth.Workload("fp4-2experts", 4096, 2880, 2, 6, "e2m1", True, (1,), False, 1004)
    L = synth.make_layer(wl)
    per_expert = sum(m.q[0].nbytes + m.s[0].nbytes for m in (L.gate, L.up, L.down))
    assert per_expert == 18_800_640


def test_e4m3_code_count():
    import oracle.moe_oracle as om
    assert om.E4M3.size == facts()["e4m3_code_count"]["value"]


def test_tiny_canary():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLD, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(GOLD, "tiny_canary.json")) as f:
        want = json.load(f)
    assert mod.canary() == want
