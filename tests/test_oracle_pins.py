"""The oracle against its pins (brute force, closed forms, invariants)."""
import numpy as np
import pytest

import oracle.moe_oracle as om
import oracle_pins as P


@pytest.mark.parametrize("name,biased", [("tiny", False), ("tiny", True), ("e4m3-nonsquare", False),
                                         ("e4m3-nonsquare", True), ("e2m1-small", False)])
def test_bruteforce_small(name, biased):
    P.pin_bruteforce(om, name, biased=biased)


@pytest.mark.parametrize("pin", [P.pin_onehot, P.pin_routing_closed_form, P.pin_router_exact,
                                 P.pin_topk_ties, P.pin_permute, P.pin_silu, P.pin_scale_doubling,
                                 P.pin_identical_experts, P.pin_relabel, P.pin_zero_input,
                                 P.pin_single_expert, P.pin_lossless_grid, P.pin_token_subset,
                                 P.pin_rmsnorm, P.pin_residual_add, P.pin_act_quant,
                                 P.pin_block_forward])
def test_pin(pin):
    pin(om)


@pytest.mark.parametrize("name", ["e4m3-nonsquare", "e2m1-small"])
def test_act_quant_forward_bruteforce(name):
    P.pin_act_quant_forward(om, name)


def test_bruteforce_olmoe_decode_shapes():
    """The OLMoE-shaped decode layer (d=2048, E=64, k=8, f=1024) at 1 and 8 tokens."""
    import synth
    import bruteforce as bf
    wl = synth.WORKLOADS["olmoe-decode"]
    layer = synth.make_layer(wl)
    for T in (1, 8):
        batch = synth.make_batch(wl, layer, T)
        r = P.run(om, wl, layer, batch)
        ids, w, out = bf.forward(batch.x, layer.w_router, batch.bias,
                                 (layer.gate.q, layer.gate.s, layer.up.q, layer.up.s,
                                  layer.down.q, layer.down.s), wl.k, wl.renorm, wl.fmt)
        assert np.array_equal(r.ids, ids)
        np.testing.assert_allclose(r.w, w, rtol=1e-12)
        P.assert_out_close(r.out, out)


def test_bruteforce_fp4_shapes_reduced_experts():
    """FP4 layer dims (d=4096, f=2880, k=6) with 12 experts instead of 384, one token."""
    import synth
    import bruteforce as bf
    wl = synth.Workload("fp4-reduced", 4096, 2880, 12, 6, "e2m1", True, (1,), False, 1004)
    layer = synth.make_layer(wl)
    batch = synth.make_batch(wl, layer, 1)
    r = P.run(om, wl, layer, batch)
    ids, w, out = bf.forward(batch.x, layer.w_router, None,
                             (layer.gate.q, layer.gate.s, layer.up.q, layer.up.s, layer.down.q,
                              layer.down.s), wl.k, wl.renorm, wl.fmt)
    assert np.array_equal(r.ids, ids)
    np.testing.assert_allclose(r.w, w, rtol=1e-12)
    P.assert_out_close(r.out, out)
