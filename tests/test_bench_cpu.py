"""Host logic of bench.py (no GPU): the algorithmic bytes of the expert
kernels, the counter scaling that turns rocprofv3 FETCH_SIZE / WRITE_SIZE
into HBM bytes, and the refusal of more than one GPU."""
import argparse
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_expert_stage_bytes_e4m3():
    """Weights once per distinct expert (codes + one f32 per 128 x 128 block),
    bf16 x rows in and h out for gate/up; h in and f32 y out for down."""
    wl = synth.Workload("b-e4m3", 256, 384, 8, 2, "e4m3", False, (4,), False, 1)
    gu, dn = bench.expert_stage_bytes(wl, U=3, T=4)
    d, f, S = 256, 384, 8
    assert gu == 3 * 2 * (d * f + 4 * 2 * 3) + 4 * d * 2 + S * f * 2
    assert dn == 3 * (d * f + 4 * 2 * 3) + S * f * 2 + S * d * 4


@pytest.mark.parametrize("fmt,g", [("e2m1", 32), ("nvfp4", 16)])
def test_expert_stage_bytes_fp4(fmt, g):
    """Half a byte per weight plus one scale byte per group of g inputs."""
    wl = synth.Workload("b-fp4", 128, 96, 8, 3, fmt, True, (5,), False, 1)
    gu, dn = bench.expert_stage_bytes(wl, U=5, T=5)
    d, f, S = 128, 96, 15
    assert gu == 5 * 2 * (d * f // 2 + d * f // g) + 5 * d * 2 + S * f * 2
    assert dn == 5 * (d * f // 2 + d * f // g) + S * f * 2 + S * d * 4


def _csv(path, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for k, c, v in rows:
            f.write(f'"{k}",{c},{v}\n')


def test_write_traffic_scales_by_the_copy(tmp_path):
    """A 512 MiB copy that reads FETCH_SIZE = half its KiB scales fetches by 2;
    WRITE_SIZE read exactly scales by 1; per-dispatch means are taken."""
    kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cf, cw = tmp_path / "cf.csv", tmp_path / "cw.csv"
    _csv(fetch, [("void moe::gemm_big<0, true, 1, 3, 2>(x)", "FETCH_SIZE", 1000.0),
                 ("void moe::gemm_big<0, true, 1, 3, 2>(x)", "FETCH_SIZE", 3000.0),
                 ("void moe::other(x)", "FETCH_SIZE", 9.0)])
    _csv(write, [("void moe::gemm_big<0, true, 1, 3, 2>(x)", "WRITE_SIZE", 100.0)])
    _csv(cf, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2)])
    _csv(cw, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", kib)])
    out = tmp_path / "traffic.json"
    args = argparse.Namespace(write_traffic=[str(fetch), str(write), str(cf), str(cw)],
                              traffic=str(out), traffic_key="k/T=1/grouped/gateup",
                              traffic_kernel="gemm_big<0, true")
    bench.write_traffic(args)
    e = json.load(open(out))["entries"]["k/T=1/grouped/gateup"]
    assert e["copy_scale_fetch"] == 2.0 and e["copy_scale_write"] == 1.0
    assert e["fetch_bytes"] == int(2000.0 * 1024 * 2) and e["write_bytes"] == 100 * 1024
    assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    assert e["kernel_source"] == bench.kernel_source_hash()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
