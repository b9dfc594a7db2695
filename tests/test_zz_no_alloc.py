"""moe_forward_noalloc (the entry point for callers that cannot allocate)
against moe_forward with a caller workspace, through the C ABI: the same
kernels on the same inputs, so every output is compared bit for bit, and both
against the oracle at the output bars.  Calls run back to back on one device,
each smaller than the one before, so stale scratch contents from the larger
call are present when the smaller one runs; grouped and decode sizes both
occur.  A size whose workspace exceeds the scratch is refused before any
launch."""
import numpy as np
import pytest

import synth
from gpu_util import check_out, check_routing, device_weights, log, oracle_run

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["olmoe-decode"]   # d=2048, f=1024, 64 experts, top-8
SIZES = [200, 100, 48, 5]             # grouped, grouped, decode (MFMA tiles), decode


@pytest.fixture(scope="module")
def layer():
    L = synth.make_layer(WL)
    return L, device_weights(L)


def test_noalloc_matches_workspace_forward(layer):
    import torch
    import mixture_experts_layer_f32_amd as moe
    from mixture_experts_layer_f32_amd.device import Runner, to_dev
    L, W = layer
    run = Runner(WL.d, WL.f, WL.E, WL.k, WL.fmt, WL.renorm, max(SIZES))
    assert moe.moe_noalloc_scratch_bytes() == 64 << 20
    g, u, dn = W.mats()
    for T in SIZES:
        assert moe.moe_workspace_size(run.plan, T) <= moe.moe_noalloc_scratch_bytes()
        batch = synth.make_batch(WL, L, T, batch_index=T)
        x = to_dev(batch.x)
        ref_ws = run.outputs(T)
        run.forward(W, x, None, ref_ws)
        got = run.outputs(T)
        for t in got.values():
            t.fill_(-7)
        moe.moe_forward_noalloc(run.plan, T, x, W.w_router, None, g, u, dn, got["out"],
                                got["topk_ids"], got["topk_w"], got["counts"], got["offsets"],
                                got["perm"])
        torch.cuda.synchronize()
        for k in got:
            assert torch.equal(got[k], ref_ws[k]), f"T={T}: {k} differs from moe_forward"
        ref = oracle_run(WL, L, batch)
        res = {k: v.cpu().numpy() for k, v in got.items()}
        check_routing(res, ref)
        mx, rms, mrel = check_out(res["out"], ref.out)
        path = "decode" if moe.moe_plan_path(run.plan, T) == moe.MOE_PATH_DECODE else "grouped"
        log(f"noalloc T={T} ({path}): equal to moe_forward; max|err| {mx:.3e} mean rel {mrel:.3e}")


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import mixture_experts_layer_f32_amd as moe
    plan = moe.moe_plan(7168, 2048, 256, 8, 4096, "e4m3", True)
    assert moe.moe_workspace_size(plan, 4096) > moe.moe_noalloc_scratch_bytes()
    z = moe.moe_mat(None, None, 0, 0)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(plan, 4096, None, None, None, z, z, z, None)
    assert e.value.status == moe.MOE_ERR_WORKSPACE
