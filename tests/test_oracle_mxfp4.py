"""Pins for the MXFP4 weight format of the W4A8 path (oracle readings
R29-R31), each against something other than the oracle's own formula: the
hand-written e2m1 table, brute-force nearest search, a block worked by hand,
a dense float64 product, and planted mutants that must fail."""

import os

import numpy as np
import pytest

from oracle import moe_ref, mx_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")
RNG = np.random.default_rng(29)


def golden_table():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        c, v = line.split()
        vals[int(c)] = float(v)
    return vals


def test_e2m1_decode_matches_hand_table():
    table = golden_table()
    assert sorted(table) == list(range(16))
    got = mx_ref.e2m1_decode(np.arange(16))
    for c in range(16):
        assert got[c] == table[c] and np.signbit(got[c]) == np.signbit(table[c]), c


def _brute_encode(v):
    """Nearest of the 8 magnitudes (after clamping to 6), ties to the even
    code, sign kept: a direct search over the hand table."""
    table = golden_table()
    a = min(abs(v), 6.0)
    best = min(range(8), key=lambda c: (abs(table[c] - a), c % 2, c))
    return best | (8 if np.signbit(v) else 0)


def test_e2m1_encode_vs_brute_force():
    grid = [golden_table()[c] for c in range(8)]
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    vals = grid + mids + [m + d for m in mids for d in (-1e-9, 1e-9)] + [6.5, 7.0, 100.0, 1e-30]
    vals += list(RNG.uniform(-8, 8, 500))
    vals = np.array(vals + [-v for v in vals] + [0.0, -0.0])
    got = mx_ref.e2m1_encode(vals)
    want = np.array([_brute_encode(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, want)


def test_mxfp4_worked_block():
    """One block worked by hand: amax 7 -> s = floor(log2 7) - 2 = 0, scale
    byte 127; 7 saturates to 6; 0.25 ties to 0 (even), 0.75 to 1.0, 2.5 to
    2.0, 5.0 to 4.0; -0.1 rounds to -0 (code 8); packed low nibble first."""
    v = np.zeros((1, 32))
    v[0, :8] = [7.0, 0.25, 0.75, 2.5, 5.0, -0.1, -1.5, 3.0]
    q, s = mx_ref.mxfp4_quantize_ref(v)
    assert s.shape == (1, 1, 2) and s[0, 0, 0] == 127 and s[0, 0, 1] == 0
    codes = [7, 0, 2, 4, 6, 8, 11, 5]
    assert list(q[0, :4]) == [codes[0] | codes[1] << 4, codes[2] | codes[3] << 4,
                              codes[4] | codes[5] << 4, codes[6] | codes[7] << 4]
    assert np.all(q[0, 4:] == 0)


def test_mxfp4_scale_rule_and_saturation():
    for e in range(-20, 20):
        for frac in (1.0, 1.3, 1.99):
            amax = frac * 2.0 ** e
            v = np.zeros((1, 32))
            v[0, 3] = amax
            q, s = mx_ref.mxfp4_quantize_ref(v)
            assert int(s[0, 0, 0]) == e - 2 + 127
            # the largest element scales into [4, 8): codes 6 (4.0) or 7 (6.0)
            c = mx_ref.fp4_unpack(q)[0, 3]
            assert c in (6, 7)
    q, s = mx_ref.mxfp4_quantize_ref(np.zeros((2, 64)))
    assert np.all(s == 0) and np.all(q == 0)


def test_mxfp4_roundtrip_is_nearest_in_block_grid():
    v = RNG.standard_normal((20, 96)) * np.exp2(RNG.integers(-8, 8, (20, 1)))
    q, s = mx_ref.mxfp4_quantize_ref(v)
    d = mx_ref.mxfp4_dequantize_ref(q, s)
    sc = mx_ref.e8m0_decode(mx_ref.scales_flat(s, 96))
    table = np.array([golden_table()[c] for c in range(8)])
    for r in range(20):
        for kk in range(96):
            g = table * sc[r, kk // 32]
            a = min(abs(v[r, kk]), g[-1])
            assert abs(abs(d[r, kk]) - a) <= np.min(np.abs(g - a)) + 1e-300


def test_pack_unpack_order():
    codes = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    assert list(mx_ref.fp4_pack(codes)[0]) == [0x21, 0x43, 0x0F]
    assert np.array_equal(mx_ref.fp4_unpack(mx_ref.fp4_pack(codes)), codes)


def test_w4a8_gemm_equals_dense_dequantised_product():
    M, K, N = 19, 256, 40
    a = RNG.standard_normal((M, K)) * np.exp2(RNG.integers(-4, 4, (M, 1)))
    w = RNG.standard_normal((N, K)) * 0.05
    aq, as_ = mx_ref.mx_quantize_ref(a)
    wq, ws = mx_ref.mxfp4_quantize_ref(w)
    ref = mx_ref.mx_dequantize_ref(aq, as_) @ mx_ref.mxfp4_dequantize_ref(wq, ws).T
    y = moe_ref.gmm_mx_ref(aq, as_, wq[None], ws[None], np.array([M]), 1, "e2m1")
    r32 = ref.astype(np.float32)
    diff = np.abs(mx_ref.bf16_to_f64(y) - mx_ref.bf16_to_f64(mx_ref.f32_to_bf16(r32)))
    ulp = np.exp2(np.floor(np.log2(np.abs(r32) + 1e-30)) - 7)
    assert np.all(diff <= ulp)
    # GEMM1 with e2m1 weights: gate/up halves and SwiGLU as for e4m3
    w13 = RNG.standard_normal((1, 2 * 64, K)) * 0.05
    w13q, w13s = mx_ref.mxfp4_quantize_ref(w13[0])
    hq, hs, h = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, w13q[None], w13s[None], np.array([M]), 1, 64, "e2m1")
    acc = (mx_ref.mx_dequantize_ref(aq, as_) @ mx_ref.mxfp4_dequantize_ref(w13q, w13s).T).astype(np.float32)
    np.testing.assert_allclose(h, moe_ref.silu_mul_ref(acc[:, :64], acc[:, 64:]), rtol=1e-6, atol=1e-30)


@pytest.mark.parametrize("mutant", ["nibbles_swapped", "ties_up", "emax_1"])
def test_mutants_fail(mutant, monkeypatch):
    if mutant == "nibbles_swapped":
        monkeypatch.setattr(mx_ref, "fp4_pack", lambda c: (np.asarray(c)[..., 1::2] | (np.asarray(c)[..., 0::2] << 4)).astype(np.uint8))
        with pytest.raises(AssertionError):
            test_mxfp4_worked_block()
    elif mutant == "ties_up":
        def enc(v):
            v = np.asarray(v, np.float64)
            grid = mx_ref.e2m1_decode(np.arange(8))
            a = np.minimum(np.abs(v), 6.0)
            d = np.abs(a[..., None] - grid)
            code = np.argmax(np.where(d == d.min(axis=-1, keepdims=True), np.arange(8), -1), axis=-1)
            return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)
        monkeypatch.setattr(mx_ref, "e2m1_encode", enc)
        with pytest.raises(AssertionError):
            test_e2m1_encode_vs_brute_force()
    else:
        monkeypatch.setattr(mx_ref, "E2M1_EMAX", 1)
        with pytest.raises(AssertionError):
            test_mxfp4_scale_rule_and_saturation()
