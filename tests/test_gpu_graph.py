"""The forward captured in a HIP graph (torch.cuda.CUDAGraph on ROCm): the
library launches kernels only (no allocation, no memset, no host sync), so a
captured forward replays on new inputs copied into the captured buffers.
Every replay, with eager work and synchronisations between replays, must give
the same bits as an eager forward on the same inputs."""
import numpy as np
import pytest

import synth
from gpu_util import device_weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl_name,T,act_fmt", [("olmoe-decode", 8, 0), ("tiny", 4, 0),
                                               ("olmoe-prefill-skewed", 128, 0),
                                               ("olmoe-prefill-skewed", 128, 1)])
def test_graph_replay_matches_eager(wl_name, T, act_fmt):
    """act_fmt 1: the activation-quantised plan (its two quantiser launches
    and the block-scaled GEMMs) captured the same way."""
    import torch
    from mixture_experts_layer_f32_amd.device import Runner, to_dev
    wl = synth.WORKLOADS[wl_name]
    layer = synth.make_layer(wl)
    W = device_weights(layer)
    batches = [synth.make_batch(wl, layer, T, batch_index=i) for i in range(3)]
    run = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T, act_fmt=act_fmt)
    x_static = to_dev(batches[0].x)
    has_bias = batches[0].bias is not None
    b_static = to_dev(batches[0].bias) if has_bias else None
    outs = run.outputs(T)

    # eager references
    refs = []
    for b in batches:
        o = run.outputs(T)
        run.forward(W, to_dev(b.x), to_dev(b.bias) if has_bias else None, o)
        torch.cuda.synchronize()
        refs.append({k: v.clone() for k, v in o.items()})

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        run.forward(W, x_static, b_static, outs, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.forward(W, x_static, b_static, outs, torch.cuda.current_stream())

    for rep in range(2):
        for i, b in enumerate(batches):
            x_static.copy_(to_dev(b.x))
            if has_bias:
                b_static.copy_(to_dev(b.bias))
            # unrelated eager work between replays
            junk = torch.randn(1 << 16, device="cuda").sum()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k in ("out", "topk_ids", "topk_w", "counts", "offsets", "perm"):
                assert torch.equal(outs[k], refs[i][k]), (rep, i, k)
            del junk
