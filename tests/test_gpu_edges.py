"""GPU edge cases: argument errors (checked on the host before any launch),
empty and maximal batches, routing extremes forced through the logit bias
(every token on one expert, exact ties), zero input, the one-block-per-
expert weight layout described by strides, and non-finite input rows."""
import numpy as np
import pytest

import synth
from gpu_util import check_h, check_out, check_routing, device_weights, gpu_run, oracle_run

pytestmark = pytest.mark.gpu

WL = synth.Workload("edge-e4m3", 256, 384, 6, 2, "e4m3", True, (9,), False, 4001)
WL4 = synth.Workload("edge-e2m1", 128, 96, 8, 3, "e2m1", False, (9,), False, 4002)
WLN = synth.Workload("edge-nvfp4", 128, 96, 8, 3, "nvfp4", False, (9,), False, 4003)
_cache = {}


def get(wl):
    if wl.name not in _cache:
        L = synth.make_layer(wl)
        _cache[wl.name] = (L, device_weights(L))
    return _cache[wl.name]


def runner(wl, max_tokens, path=0):
    from mixture_experts_layer_f32_amd.device import Runner
    return Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, max_tokens, path)


def test_argument_errors_launch_nothing():
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import to_dev
    L, W = get(WL)
    run = runner(WL, 4)
    batch = synth.make_batch(WL, L, 4)
    x = to_dev(batch.x)
    outs = run.outputs(4)
    outs["out"].fill_(7.0)
    g, u, d = W.mats()

    def call(**kw):
        args = dict(plan=run.plan, n_tokens=4, x=x, w_router=W.w_router, logit_bias=None, gate=g,
                    up=u, down=d, out=outs["out"], workspace=run.workspace)
        args.update(kw)
        with pytest.raises(m.MoeError) as e:
            m.moe_forward(**args)
        return e.value.status

    assert call(n_tokens=5) == m.MOE_ERR_BAD_SHAPE
    assert call(n_tokens=-1) == m.MOE_ERR_BAD_SHAPE
    assert call(x=0) == m.MOE_ERR_NULL_ARG
    assert call(out=0) == m.MOE_ERR_NULL_ARG
    assert call(workspace=0) == m.MOE_ERR_NULL_ARG
    assert call(workspace_bytes=m.moe_workspace_size(run.plan, 4) - 1) == m.MOE_ERR_WORKSPACE
    assert call(x=x.data_ptr() + 2) == m.MOE_ERR_ALIGNMENT
    assert call(out=outs["out"].data_ptr() + 4) == m.MOE_ERR_ALIGNMENT
    bad = m.moe_mat(g.q + 8, g.scale, g.q_expert_stride, g.s_expert_stride)
    assert call(gate=bad) == m.MOE_ERR_ALIGNMENT
    bad = m.moe_mat(g.q, None, g.q_expert_stride, g.s_expert_stride)
    assert call(up=bad) == m.MOE_ERR_NULL_ARG
    torch.cuda.synchronize()
    assert torch.all(outs["out"] == 7.0)          # nothing was written
    # T = 0 is a no-op
    m.moe_forward(run.plan, 0, x, W.w_router, None, g, u, d, outs["out"], workspace=run.workspace)
    torch.cuda.synchronize()
    assert torch.all(outs["out"] == 7.0)
    assert m.moe_workspace_size(run.plan, 0) == 0


@pytest.mark.parametrize("wl", [WL, WL4, WLN], ids=lambda w: w.name)
@pytest.mark.parametrize("path", [1, 2])
def test_all_tokens_on_one_expert(wl, path):
    """A large bias on expert 3 sends every token there: one expert gets all T
    slots (several M tiles in the grouped path), the others share the rest."""
    L, W = get(wl)
    T = 150
    batch = synth.make_batch(wl, L, T)
    bias = np.zeros((T, wl.E), np.float32)
    bias[:, 3] = 100.0
    batch = synth.Batch(batch.x, bias)
    ref = oracle_run(wl, L, batch)
    assert ref.counts[3] == T
    g, _ = gpu_run(wl, W, batch, path)
    check_routing(g, ref)
    check_h(g["h"], ref.h)
    check_out(g["out"], ref.out)


@pytest.mark.parametrize("path", [1, 2])
def test_exact_ties_go_to_lower_index(path):
    """Zero router weights and a bias with three equal maxima: the top-2 are
    the two lowest of the three."""
    L, W = get(WL)
    import torch
    T = 5
    batch = synth.make_batch(WL, L, T)
    bias = np.zeros((T, WL.E), np.float32)
    bias[:, [1, 2, 4]] = 1.0
    wr = np.zeros_like(L.w_router)
    Lz = synth.Layer(WL, wr, L.gate, L.up, L.down)
    Wz = device_weights(Lz)
    batch = synth.Batch(batch.x, bias)
    ref = oracle_run(WL, Lz, batch)
    assert ref.ids.tolist() == [[1, 2]] * T
    g, _ = gpu_run(WL, Wz, batch, path)
    check_routing(g, ref)
    check_out(g["out"], ref.out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", [1, 2])
def test_zero_input(path):
    L, W = get(WL)
    x = np.zeros((3, WL.d), np.uint16)
    g, _ = gpu_run(WL, W, synth.Batch(x, None), path)
    assert np.all(g["out"] == 0)
    assert g["topk_ids"].tolist() == [[0, 1]] * 3


def test_max_tokens_boundary():
    L, W = get(WL)
    batch = synth.make_batch(WL, L, 40)
    ref = oracle_run(WL, L, batch)
    g, run = gpu_run(WL, W, batch, 0, max_tokens=40)
    check_routing(g, ref)
    check_out(g["out"], ref.out)


@pytest.mark.parametrize("wl", [WL, WL4, WLN], ids=lambda w: w.name)
def test_one_block_per_expert_layout(wl):
    """Each expert's gate | up | down codes and scales packed in one block,
    described by expert strides: same bits as the one-buffer-per-matrix layout."""
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import to_dev
    L, W = get(wl)
    T = 7
    batch = synth.make_batch(wl, L, T)
    a, _ = gpu_run(wl, W, batch, 0)
    parts = [L.gate.q, L.up.q, L.down.q, L.gate.s, L.up.s, L.down.s]
    sizes = [p[0].nbytes for p in parts]
    offs = np.concatenate([[0], np.cumsum([(s + 255) // 256 * 256 for s in sizes])])
    blk = int(offs[-1])
    buf = np.zeros((wl.E, blk), np.uint8)
    for i, p in enumerate(parts):
        buf[:, offs[i]:offs[i] + sizes[i]] = p.reshape(wl.E, -1).view(np.uint8)
    dbuf = to_dev(buf)
    base = dbuf.data_ptr()
    mk = lambda qi, si: m.moe_mat(base + int(offs[qi]), base + int(offs[si]), blk, blk)  # noqa
    run = runner(wl, T)
    outs = run.outputs(T)
    m.moe_forward(run.plan, T, to_dev(batch.x), W.w_router, None, mk(0, 3), mk(1, 4), mk(2, 5),
                  outs["out"], workspace=run.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(outs["out"].cpu().numpy().view(np.uint32), a["out"].view(np.uint32))


def test_nvfp4_scale_alignment():
    """NVFP4 reads a row's two 16-input group scales as one 16-bit word: an
    odd scale pointer or expert stride is rejected before any launch."""
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import to_dev
    L, W = get(WLN)
    run = runner(WLN, 4)
    batch = synth.make_batch(WLN, L, 4)
    outs = run.outputs(4)
    outs["out"].fill_(7.0)
    g, u, d = W.mats()
    for bad in (m.moe_mat(g.q, g.scale + 1, g.q_expert_stride, g.s_expert_stride),
                m.moe_mat(g.q, g.scale, g.q_expert_stride, g.s_expert_stride + 1)):
        with pytest.raises(m.MoeError) as e:
            m.moe_forward(run.plan, 4, to_dev(batch.x), W.w_router, None, bad, u, d, outs["out"],
                          workspace=run.workspace)
        assert e.value.status == m.MOE_ERR_ALIGNMENT
    torch.cuda.synchronize()
    assert torch.all(outs["out"] == 7.0)


WL4W = synth.Workload("edge-e2m1-wide", 512, 288, 8, 2, "e2m1", False, (9,), False, 4004)
WLNW = synth.Workload("edge-nvfp4-wide", 512, 288, 8, 2, "nvfp4", False, (9,), False, 4005)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("wl", [WL4W, WLNW], ids=lambda w: w.name)
def test_fp4_scales_at_unaligned_addresses(wl, path):
    """Group scales read as whole runs of a row: scale buffers moved to the
    smallest alignment the format allows (e2m1: 1 byte, nvfp4: 2 bytes, both
    for the pointer and the expert stride) give the same bits.  d = 512 takes
    full 256-input steps, f = 288 a ragged last one."""
    import torch
    import mixture_experts_layer_f32_amd as m
    from mixture_experts_layer_f32_amd.device import to_dev
    L, W = get(wl)
    T = 9
    batch = synth.make_batch(wl, L, T)
    a, _ = gpu_run(wl, W, batch, path)
    step = 1 if wl.fmt == "e2m1" else 2
    moved = []
    for q, sc in ((L.gate.q, L.gate.s), (L.up.q, L.up.s), (L.down.q, L.down.s)):
        per = sc[0].nbytes
        stride = per + step
        buf = np.zeros(step + wl.E * stride, np.uint8)
        for e in range(wl.E):
            buf[step + e * stride:step + e * stride + per] = sc[e].reshape(-1).view(np.uint8)
        dq, ds = to_dev(q), to_dev(buf)
        moved.append((dq, ds, m.moe_mat(dq.data_ptr(), ds.data_ptr() + step, q[0].nbytes, stride)))
    run = runner(wl, T, path)
    outs = run.outputs(T)
    m.moe_forward(run.plan, T, to_dev(batch.x), W.w_router, None, moved[0][2], moved[1][2],
                  moved[2][2], outs["out"], workspace=run.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(outs["out"].cpu().numpy().view(np.uint32), a["out"].view(np.uint32))
    ref = oracle_run(wl, L, batch)
    check_out(a["out"], ref.out)


def test_nonfinite_input_row_does_not_fault():
    """A NaN activation row is outside the contract: the call must still
    complete, and the other tokens' outputs are unaffected."""
    L, W = get(WL)
    T = 6
    batch = synth.make_batch(WL, L, T)
    ref = oracle_run(WL, L, batch)
    x = batch.x.copy()
    x[2, :] = 0x7FC0  # bf16 quiet NaN
    g, _ = gpu_run(WL, W, synth.Batch(x, None), 0)
    ok = [t for t in range(T) if t != 2]
    check_out(g["out"][ok], ref.out[ok])


WL_MAX = synth.Workload("edge-max-experts", 128, 128, 1024, 16, "e4m3", True, (9,), False, 4006)
WL_MAX4 = synth.Workload("edge-max-experts-fp4", 64, 96, 1024, 16, "e2m1", False, (9,), False, 4007)


@pytest.mark.parametrize("wl", [WL_MAX, WL_MAX4], ids=lambda w: w.name)
@pytest.mark.parametrize("T,path", [(1, 0), (16, 0), (40, 1), (100, 2)])
def test_largest_expert_count_and_top_k(wl, T, path):
    """The plan's limits: 1024 experts (16 groups of 64 in the top-k) and
    top-16, through the one-workgroup routing (T <= 16), the multi-launch
    permute (40, 100) and both expert paths."""
    L, W = get(wl)
    batch = synth.make_batch(wl, L, T)
    ref = oracle_run(wl, L, batch)
    g, _ = gpu_run(wl, W, batch, path)
    check_routing(g, ref)
    check_h(g["h"], ref.h)
    check_out(g["out"], ref.out)


@pytest.mark.parametrize("T", [1, 16, 100])
def test_largest_expert_count_and_top_k_act_quant(T):
    """The same limits (1024 experts, top-16) on the activation-quantised plan:
    routing bit-exact, h and out against the oracle's quantised layer, end to
    end and with the down projection fed the GPU's own h."""
    from test_gpu_actquant import check_h_q8, check_out_q8_e2e, oracle_q8, q8_reference, run_q8
    L, W = get(WL_MAX)
    batch = synth.make_batch(WL_MAX, L, T)
    ref = oracle_q8(WL_MAX, L, batch)
    g = run_q8(WL_MAX, W, batch)
    check_routing(g, ref)
    check_h_q8(g["h"], ref.h)
    _, out_ref = q8_reference(WL_MAX, L, batch, ref, g["h"], np.arange(T))
    check_out(g["out"], out_ref)
    check_out_q8_e2e(g, ref.out)


@pytest.mark.parametrize("stages", [("gateup",), ("router", "combine"), None])
def test_stage_timing_leaves_no_error(stages):
    """Stage timing with any subset of stages: the recorded times are positive
    for the timed stages and zero for the others, and after the timing is
    switched off the next forward runs and matches the oracle (destroying the
    timing events must not leave an error behind for the next launch check)."""
    import torch
    import mixture_experts_layer_f32_amd as moe
    from mixture_experts_layer_f32_amd.device import Runner, to_dev
    wl = WL
    L, W = get(wl)
    T = 8
    batch = synth.make_batch(wl, L, T)
    run = Runner(wl.d, wl.f, wl.E, wl.k, wl.fmt, wl.renorm, T)
    outs = run.outputs(T)
    x = to_dev(batch.x)
    sel = moe.STAGES if stages is None else stages
    moe.moe_timing_enable(run.plan, sel, max_forwards=4)
    for _ in range(3):
        run.forward(W, x, None, outs)
    ms, n = moe.moe_timing_collect(run.plan)
    moe.moe_timing_disable(run.plan)
    assert n == 3
    assert all(ms[s] > 0 for s in ("gateup",) if s in sel)
    assert all(ms[s] == 0 for s in moe.STAGES if s not in sel)
    run.forward(W, x, None, outs)
    torch.cuda.synchronize()
    ref = oracle_run(wl, L, batch)
    check_out(outs["out"].cpu().numpy(), ref.out)
