"""Pins of the number formats: the oracle's decoders and the generator's
encoders, each against something other than itself (torch's casts, brute-force
nearest-value search over the whole code set, closed forms)."""
import math

import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
import synth

# ---------------------------------------------------------------- helpers (independent of the oracle)


def all_bf16_values():
    """All finite bf16 values, sorted, with their bit patterns (via torch)."""
    bits = np.arange(65536, dtype=np.int32).astype(np.int16)
    vals = torch.from_numpy(bits).view(torch.bfloat16).to(torch.float64).numpy()
    ok = np.isfinite(vals)
    vals, bits = vals[ok], bits[ok].astype(np.uint16)
    # keep +0 only once (drop -0) so that the search has unique keys
    keep = ~((vals == 0) & (bits == 0x8000))
    vals, bits = vals[keep], bits[keep]
    order = np.argsort(vals, kind="stable")
    return vals[order], bits[order]


def brute_bf16_rne(v):
    """Nearest finite bf16 by search over every bf16 value; ties -> even bit pattern."""
    vals, bits = all_bf16_values()
    out = np.empty(v.shape, np.uint16)
    i = np.clip(np.searchsorted(vals, v), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = v - lo, hi - v
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((bits[i] & 1) == 0))
    out = np.where(pick_hi, bits[i], bits[i - 1])
    return out


# ---------------------------------------------------------------- e4m3


def test_e4m3_table_matches_torch_all_256_codes():
    # dragon.c page, section 8 Round 3: e4m3 has exactly 256 possible values.
    assert om.E4M3.shape == (256,)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(om.E4M3)
    assert np.all(both_nan | (ref == om.E4M3))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(om.E4M3[~both_nan]))


def test_e4m3_closed_form_points():
    T = om.E4M3
    assert T[0x00] == 0.0 and T[0x80] == 0.0 and np.signbit(T[0x80])
    assert T[0x01] == 2.0 ** -9          # smallest subnormal
    assert T[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert T[0x08] == 2.0 ** -6          # smallest normal
    assert T[0x38] == 1.0
    assert T[0x7E] == 448.0 and T[0xFE] == -448.0
    assert np.isnan(T[0x7F]) and np.isnan(T[0xFF])
    finite = T[np.isfinite(T)]
    assert finite.size == 254 and np.unique(finite).size == 253  # +0 and -0 coincide


# ---------------------------------------------------------------- e2m1


def test_e2m1_table_closed_form():
    pos = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(om.E2M1[:8]) == pos
    assert list(om.E2M1[8:]) == [-v for v in pos]
    assert np.signbit(om.E2M1[8])


def test_unpack_e2m1_low_nibble_first():
    # Reading R11: element 2i is the low nibble, 2i+1 the high nibble.
    q = np.array([[0x21, 0xF7]], np.uint8)
    codes = om.unpack_e2m1(q, 4)
    assert codes.tolist() == [[0x1, 0x2, 0x7, 0xF]]
    assert om.E2M1[codes].tolist() == [[0.5, 1.0, 6.0, -6.0]]


# ---------------------------------------------------------------- bf16


def test_bf16_widening_exact_all_patterns():
    bits = np.arange(65536, dtype=np.int64).astype(np.uint16)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = om.bf16_to_f64(bits)
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    assert same.all()


def test_bf16_rne_vs_torch_on_f32_inputs():
    rng = np.random.default_rng(0)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),      # subnormal range
        (rng.standard_normal(20000) * 1e38).astype(np.float32),       # near overflow
        # exact ties: 9 significant bits with the 9th set
        (np.arange(1, 5000, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -9) + 1.0,
        np.array([0.0, -0.0, 3.3895314e38, 3.40282347e38, 1e-45], np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = om.bf16_rne(f.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_rne_vs_brute_force_on_f64_inputs():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(50000), rng.standard_normal(5000) * 1e-3,
                        # f64 values just above / below bf16 ties (not representable in f32)
                        1.0 + 2.0 ** -8 + np.array([2.0 ** -40, -2.0 ** -40, 0.0]),
                        -(3.0 + 2.0 ** -7 + np.array([2.0 ** -45, -2.0 ** -45, 0.0]))])
    assert np.array_equal(om.bf16_rne(v), brute_bf16_rne(v))


# ---------------------------------------------------------------- dequantisation layout


def test_dequant_e4m3_scale_block_index():
    # 256 x 384 matrix: a 2 x 3 grid of 128x128 blocks, each with its own scale.
    s = np.array([[1.0, 2.0, 4.0], [8.0, 16.0, 32.0]], np.float32)
    q = np.full((256, 384), 0x38, np.uint8)  # every code is 1.0
    W = om.dequant(q, s, "e4m3", 384)
    for n in (0, 127, 128, 255):
        for c in (0, 127, 128, 255, 256, 383):
            assert W[n, c] == s[n // 128, c // 128]


def test_dequant_e2m1_group_index():
    # 2 rows x 64 columns: two 32-wide groups per row, scale bytes 127 + j.
    s = np.array([[127, 128], [126, 130]], np.uint8)
    q = np.full((2, 32), 0x22, np.uint8)     # codes (1.0, 1.0)
    W = om.dequant(q, s, "e2m1", 64)
    assert np.all(W[0, :32] == 1.0) and np.all(W[0, 32:] == 2.0)
    assert np.all(W[1, :32] == 0.5) and np.all(W[1, 32:] == 8.0)


def test_dequant_nvfp4_group_index():
    # 2 rows x 48 columns: three 16-wide groups per row; E4M3 scale codes with
    # non-power-of-two values (0x3C = 1.5, 0x44 = 3.0, 0x33 = 0.6875) and a
    # subnormal one (0x05 = 5 * 2^-9).
    s = np.array([[0x38, 0x3C, 0x44], [0x30, 0x33, 0x05]], np.uint8)
    q = np.full((2, 24), 0x22, np.uint8)     # codes (1.0, 1.0)
    q[1, 16:] = 0xBF                          # low nibble 0xF = -6.0, high nibble 0xB = -1.5
    W = om.dequant(q, s, "nvfp4", 48)
    assert np.all(W[0, :16] == 1.0) and np.all(W[0, 16:32] == 1.5) and np.all(W[0, 32:] == 3.0)
    assert np.all(W[1, :16] == 0.5) and np.all(W[1, 16:32] == 0.6875)
    sub = 5 * 2.0 ** -9
    assert np.all(W[1, 32::2] == -6.0 * sub) and np.all(W[1, 33::2] == -1.5 * sub)


def test_generator_nvfp4_layout():
    import synth
    w = (np.arange(2 * 64, dtype=np.float32).reshape(2, 64) - 40.0) / 7.0
    q, s = synth.quant_nvfp4_g16(w)
    assert q.shape == (2, 32) and s.shape == (2, 4)
    # group scale = E4M3 code of amax/6; codes within the group saturate at 6
    amax = np.abs(w.reshape(2, 4, 16)).max(axis=2)
    assert np.array_equal(s, synth.enc_e4m3((amax / 6.0).astype(np.float32)))
    W = om.dequant(q, s, "nvfp4", 64)
    err = np.abs(W - w)
    # half an e2m1 step (at most one scale unit) plus the scale's own rounding
    # (codes are taken against amax/6, the stored scale is its E4M3 rounding)
    assert np.all(err <= np.repeat(om.E4M3[s], 16, axis=1) * 1.5)


# ---------------------------------------------------------------- generator encoders


def test_generator_e4m3_encoder_vs_torch():
    rng = np.random.default_rng(2)
    grid = om.E4M3[np.isfinite(om.E4M3)]
    grid = np.unique(grid)
    mids = (grid[1:] + grid[:-1]) / 2
    mids32 = mids.astype(np.float32)
    ulp = np.spacing(mids32)
    x = np.concatenate([mids32, mids32 + ulp, mids32 - ulp, grid.astype(np.float32),
                        (rng.standard_normal(100000) * 100).astype(np.float32),
                        (rng.standard_normal(10000) * 1e-3).astype(np.float32),
                        np.array([447.9, 448.0, 449.0, 463.9, 464.0, 465.0, 1e6, -1e6], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.enc_e4m3(x), ref)


def test_generator_e2m1_encoder_vs_brute_force():
    rng = np.random.default_rng(3)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mids = (grid[1:] + grid[:-1]) / 2
    x = np.concatenate([grid, mids, np.nextafter(mids.astype(np.float32), 10),
                        np.nextafter(mids.astype(np.float32), -10),
                        rng.uniform(-8, 8, 50000), [6.5, 100.0]]).astype(np.float32)
    x = np.concatenate([x, -x])
    got = synth.enc_e2m1(x)
    a = np.abs(x.astype(np.float64))
    dist = np.abs(a[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # ties go to the code with an even mantissa bit (grid index even)
    even = np.arange(8) % 2 == 0
    idx = np.where((cand & even).any(axis=1), np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))
    idx = np.where(a >= 6.0, 7, idx)
    ref = idx.astype(np.uint8) | np.where(np.signbit(x), 0x8, 0).astype(np.uint8)
    assert np.array_equal(got, ref)


def test_generator_ue8m0_is_ceil_log2():
    amax = np.array([6.0, 6.0 * 2 ** -7, 6.0 * (1 + 2 ** -23), 5.9, 3.0, 1e-30, 0.75, 7.0],
                    np.float32)
    got = synth.ue8m0_of_amax(amax)
    for a, b in zip(amax, got):
        v = np.float32(a) / np.float32(6.0)
        assert b == math.ceil(math.log2(float(v))) + 127
    assert synth.ue8m0_of_amax(np.array([0.0], np.float32))[0] == 0


def test_generator_bf16_vs_torch():
    rng = np.random.default_rng(4)
    f = np.concatenate([rng.standard_normal(100000), rng.standard_normal(1000) * 1e-39]).astype(
        np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(synth.f32_to_bf16(f), ref)
