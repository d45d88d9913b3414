"""Pins for the oracle's routing, grouped GEMMs, SwiGLU requant, finalize and
the whole layer (CPU only).  Mutation tests at the bottom plant plausible
mistakes in the oracle and check a pin fails."""

import math

import numpy as np
import pytest

from oracle import moe_ref, mx_ref
from workloads import CONFIGS, custom_config, make_inputs, to_bf16_bits

RNG = np.random.default_rng(99)


# --------------------------------------------------------------------------
# routing (P7) and a hand-worked example
# --------------------------------------------------------------------------

def check_routing(route):
    # hand-worked: T=3, k=2, E=3; ids (flat) = [2,0, 0,1, 2,0]
    ids = np.array([[2, 0], [0, 1], [2, 0]], np.int32)
    counts, sr, eri = route(ids, 3)
    assert counts.tolist() == [3, 1, 2]
    # expert 0 gets flat 1, 2, 5; expert 1 gets 3; expert 2 gets 0, 4
    assert sr.tolist() == [1, 2, 5, 3, 0, 4]
    assert eri.tolist() == [4, 0, 1, 3, 5, 2]
    # invariants on random inputs, including empty experts and k = E
    for T, k, E in [(50, 4, 16), (7, 3, 3), (100, 1, 5), (33, 8, 64)]:
        ids = np.stack([RNG.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts, sr, eri = route(ids, E)
        M = T * k
        assert counts.sum() == M
        assert np.array_equal(np.sort(sr), np.arange(M))
        assert np.array_equal(eri[sr], np.arange(M))
        e_sorted = ids.reshape(-1)[sr]
        assert np.all(np.diff(e_sorted) >= 0)
        off = np.concatenate([[0], np.cumsum(counts)])
        for e in range(E):
            seg = sr[off[e]:off[e + 1]]
            assert np.all(np.diff(seg) > 0)
            assert np.all(ids.reshape(-1)[seg] == e)


def test_routing_pins():
    check_routing(moe_ref.route_ref)


def test_routing_fast_equals_definition():
    check_routing(moe_ref.route_ref_fast)
    ids = RNG.integers(0, 40, (500, 6)).astype(np.int32)
    a = moe_ref.route_ref(ids, 40)
    b = moe_ref.route_ref_fast(ids, 40)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_route_quant_rows_are_token_quantisations():
    """P6: every expanded row p is the MX quantisation of x[sorted_row[p]//k],
    i.e. routing-with-quant equals quantise-then-permute byte for byte."""
    T, K, k, E = 20, 96, 3, 7
    x = to_bf16_bits(RNG.standard_normal((T, K)).astype(np.float32))
    ids = np.stack([RNG.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    xq, xs, sr, eri, counts = moe_ref.route_quant_ref(x, ids, E)
    for p in range(T * k):
        t = sr[p] // k
        q1, s1 = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(x[t:t + 1]))
        assert np.array_equal(xq[p], q1[0]) and np.array_equal(xs[p], s1[0])


# --------------------------------------------------------------------------
# grouped GEMM special cases (P8, P10)
# --------------------------------------------------------------------------

def check_gmm(gmm):
    # all-ones payload with unit scales: every output is K exactly
    M, K, N, E = 10, 256, 64, 3
    aq = np.full((M, K), 0x38, np.uint8)
    as_ = np.full((M, K // 64, 2), 127, np.uint8)
    wq = np.full((E, N, K), 0x38, np.uint8)
    ws = np.full((E, N, K // 64, 2), 127, np.uint8)
    y = mx_ref.bf16_to_f64(gmm(aq, as_, wq, ws, np.array([4, 0, 6]), 1))
    assert np.all(y == K)
    # single nonzero per row: y[m, n] = a * w * 2^(sa+sb)
    aq = np.zeros((M, K), np.uint8)
    aq[np.arange(M), 5] = 0x40                            # 2.0 at k = 5
    as_ = np.full((M, K // 64, 2), 127, np.uint8)
    as_[:, 0, 0] = 129                                    # block 0 scale 4
    wq = np.zeros((E, N, K), np.uint8)
    wq[:, :, 5] = 0xB8                                    # -1.0
    wq[1, :, 5] = 0x3C                                    # expert 1: 1.5
    ws = np.full((E, N, K // 64, 2), 127, np.uint8)
    ws[2, :, 0, 0] = 125                                  # expert 2 block 0 scale 1/4
    y = mx_ref.bf16_to_f64(gmm(aq, as_, wq, ws, np.array([3, 3, 4]), 1))
    assert np.all(y[:3] == -8.0) and np.all(y[3:6] == 12.0) and np.all(y[6:] == -2.0)
    # E=1 equals a dense GEMM of the dequantised operands (float64, then f32, then bf16)
    M, K, N = 33, 320, 48
    a = RNG.standard_normal((M, K)) * np.exp2(RNG.integers(-6, 6, (M, 1)))
    w = RNG.standard_normal((N, K)) * 0.05
    aq, as_ = mx_ref.mx_quantize_ref(a)
    wq, ws = mx_ref.mx_quantize_ref(w)
    ref = mx_ref.mx_dequantize_ref(aq, as_) @ mx_ref.mx_dequantize_ref(wq, ws).T
    y = gmm(aq, as_, wq[None], ws[None], np.array([M]), 1)
    r32 = ref.astype(np.float32)
    diff = np.abs(mx_ref.bf16_to_f64(y) - mx_ref.bf16_to_f64(mx_ref.f32_to_bf16(r32)))
    ulp = np.exp2(np.floor(np.log2(np.abs(r32) + 1e-30)) - 7)
    assert np.all(diff <= ulp)          # at most one bf16 ulp (fp64 summation order)
    # count and cumulative group lists give the same result (P8)
    counts = np.array([10, 0, 23])
    wq3 = np.stack([wq, wq[::-1], np.roll(wq, 1, axis=0)])
    ws3 = np.stack([ws, ws[::-1], np.roll(ws, 1, axis=0)])
    y1 = gmm(aq, as_, wq3, ws3, counts, 1)
    y0 = gmm(aq, as_, wq3, ws3, np.cumsum(counts), 0)
    assert np.array_equal(y0, y1)
    y_e0 = gmm(aq[:10], as_[:10], wq3[:1], ws3[:1], np.array([10]), 1)
    y_e2 = gmm(aq[10:], as_[10:], wq3[2:], ws3[2:], np.array([23]), 1)
    assert np.array_equal(y1[:10], y_e0) and np.array_equal(y1[10:], y_e2)


def test_gmm_special_cases():
    check_gmm(moe_ref.gmm_mx_ref)


def test_mx_dot_is_order_independent():
    """Batching does not change a result: a row alone equals the row in a batch."""
    K, N = 512, 40
    a = RNG.standard_normal((16, K)) * np.exp2(RNG.integers(-20, 20, (16, K // 32)).repeat(32, 1))
    w = RNG.standard_normal((N, K))
    aq, as_ = mx_ref.mx_quantize_ref(a)
    wq, ws = mx_ref.mx_quantize_ref(w)
    full = moe_ref._mx_dot(aq, as_.reshape(16, -1), wq, ws.reshape(N, -1))
    for r in range(16):
        one = moe_ref._mx_dot(aq[r:r + 1], as_[r:r + 1].reshape(1, -1), wq, ws.reshape(N, -1))
        assert np.array_equal(one[0], full[r])
    ref = (mx_ref.mx_dequantize_ref(aq, as_) @ mx_ref.mx_dequantize_ref(wq, ws).T)
    assert np.allclose(full, ref, rtol=1e-6, atol=0)


# --------------------------------------------------------------------------
# SwiGLU + requant (P11, R13, R14)
# --------------------------------------------------------------------------

def check_swiglu(gmm1):
    """Weights built so gate outputs g and up outputs u exactly; h must be
    silu(g) * u (and not silu(u) * g), hq/hs its MX quantisation."""
    K, I, E, M = 64, 64, 2, 4
    aq = np.zeros((M, K), np.uint8)
    aq[:, 0] = 0x38                                       # a[:, 0] = 1
    as_ = np.full((M, 1, 2), 127, np.uint8)
    w13 = np.zeros((E, 2 * I, K), np.uint8)
    g_code, u_code = 0x40, 0x44                          # gate 2.0, up 3.0
    w13[:, :I, 0] = g_code
    w13[:, I:, 0] = u_code
    w13[1, :I, 0] = 0                                     # expert 1: gate 0 -> h 0
    w13s = np.full((E, 2 * I, 1, 2), 127, np.uint8)
    hq, hs, h = gmm1(aq, as_, w13, w13s, np.array([2, 2]), 1, I)
    expect = 2.0 / (1 + math.exp(-2.0)) * 3.0
    assert np.allclose(h[:2], expect, rtol=1e-7)
    assert np.all(h[2:] == 0)
    assert np.all(hs[2:] == 0) and np.all(hq[2:] == 0)   # zero rows: scale 0, payload 0
    q_ref, s_ref = mx_ref.mx_quantize_ref(h[:2].astype(np.float64))
    assert np.array_equal(hq[:2], q_ref) and np.array_equal(hs[:2], s_ref)
    # negative gate: silu(-2) * 3
    w13[0, :I, 0] = 0xC0
    _, _, h = gmm1(aq, as_, w13, w13s, np.array([2, 2]), 1, I)
    assert np.allclose(h[:2], -2.0 / (1 + math.exp(2.0)) * 3.0, rtol=1e-7)


def test_swiglu_requant_closed_form():
    check_swiglu(moe_ref.gmm_swiglu_mxquant_ref)


def test_silu_values():
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0], np.float32)
    u = np.ones(5, np.float32)
    h = moe_ref.silu_mul_ref(g, u)
    assert h[0] == 0 and abs(h[1] - 1 / (1 + math.exp(-1))) < 1e-7
    assert abs(h[2] + 1 / (1 + math.exp(1))) < 1e-7 and h[3] == np.float32(30.0)
    assert abs(h[4]) < 1e-11


# --------------------------------------------------------------------------
# finalize (R18)
# --------------------------------------------------------------------------

def check_finalize(fin):
    T, K, k = 3, 16, 2
    y = np.zeros((T * k, K), np.float32)
    y[:, :] = np.arange(T * k)[:, None] + 1.0             # row r holds r+1
    yb = mx_ref.f32_to_bf16(y)
    w = np.array([[1.0, 0.5], [0.25, 0.25], [2.0, -1.0]], np.float32)
    eri = np.array([5, 0, 1, 2, 3, 4])
    out = mx_ref.bf16_to_f64(fin(yb, w, eri))
    assert np.all(out[0] == 6 + 0.5) and np.all(out[1] == 0.25 * 2 + 0.25 * 3)
    assert np.all(out[2] == 2 * 4 - 5)
    # float32 accumulation in ascending j: 2^24 + 1 rounds back to 2^24 in
    # float32, so 2^24 + 1 - 2^24 = 0 (float64 or another order would give 1)
    y = mx_ref.f32_to_bf16(np.array([[2.0 ** 24], [1.0], [-(2.0 ** 24)]], np.float32))
    w = np.array([[1.0, 1.0, 1.0]], np.float32)
    out = fin(y, w, np.array([0, 1, 2]))
    assert mx_ref.bf16_to_f64(out)[0, 0] == 0.0


def test_finalize_closed_form():
    check_finalize(moe_ref.finalize_ref)


# --------------------------------------------------------------------------
# the whole layer: brute force (P9) and a quantisation-error sanity check
# --------------------------------------------------------------------------

def _quantised_weights(d):
    if "w13q" in d:
        return d["w13q"], d["w13s"], d["w2q"], d["w2s"]
    E, twoI, K = d["w13"].shape
    w13q, w13s = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(d["w13"].reshape(-1, K)))
    w2q, w2s = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(d["w2"].reshape(-1, d["w2"].shape[-1])))
    I = twoI // 2
    return (w13q.reshape(E, twoI, K), w13s.reshape(E, twoI, -1, 2),
            w2q.reshape(E, K, I), w2s.reshape(E, K, -1, 2))


def check_pipeline_vs_bruteforce(forward, cfg):
    d = make_inputs(cfg)
    w13q, w13s, w2q, w2s = _quantised_weights(d)
    r = forward(d["x"], d["topk_ids"], d["topk_w"], w13q, w13s, w2q, w2s)
    bf = moe_ref.moe_dense_bruteforce_ref(d["x"], d["topk_ids"], d["topk_w"], w13q, w13s, w2q, w2s)
    assert np.array_equal(r["out"], bf)
    return d, r


def test_pipeline_equals_bruteforce_tiny():
    d, r = check_pipeline_vs_bruteforce(moe_ref.moe_forward_ref, CONFIGS["tiny"])
    # quantisation error vs the un-quantised layer is small but nonzero
    ref = moe_ref.moe_unquantized_ref(d["x"], d["topk_ids"], d["topk_w"], d["w13"], d["w2"])
    got = mx_ref.bf16_to_f64(r["out"])
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert 1e-4 < rel < 0.1


@pytest.mark.parametrize("shape", [(9, 128, 64, 5, 3), (17, 64, 128, 4, 4), (5, 256, 64, 16, 1)])
def test_pipeline_equals_bruteforce_random(shape):
    T, K, I, E, k = shape
    check_pipeline_vs_bruteforce(moe_ref.moe_forward_ref, custom_config("r", T, K, I, E, k))


def test_layer_outputs_are_consistent():
    d = make_inputs("tiny")
    w13q, w13s, w2q, w2s = _quantised_weights(d)
    r = moe_ref.moe_forward_ref(d["x"], d["topk_ids"], d["topk_w"], w13q, w13s, w2q, w2s)
    M = d["topk_ids"].size
    assert r["xq"].shape == (M, 256) and r["hq"].shape == (M, 128) and r["y"].shape == (M, 256)
    assert r["counts"].sum() == M and r["out"].shape == (64, 256)


# --------------------------------------------------------------------------
# mutation tests
# --------------------------------------------------------------------------

def test_mutant_unstable_routing_fails():
    def reversed_within_expert(ids, E):
        counts, sr, eri = moe_ref.route_ref(ids, E)
        off = np.concatenate([[0], np.cumsum(counts)])
        sr = sr.copy()
        for e in range(E):
            sr[off[e]:off[e + 1]] = sr[off[e]:off[e + 1]][::-1]
        eri = np.empty_like(sr)
        eri[sr] = np.arange(sr.size)
        return counts, sr, eri
    with pytest.raises(AssertionError):
        check_routing(reversed_within_expert)


def test_mutant_inverse_map_swapped_fails():
    def swapped(ids, E):
        c, sr, eri = moe_ref.route_ref(ids, E)
        return c, eri, sr
    with pytest.raises(AssertionError):
        check_routing(swapped)


def test_mutant_weight_scale_ignored_fails():
    def gmm_unit_weight_scale(aq, as_, wq, ws, gl, t):
        return moe_ref.gmm_mx_ref(aq, as_, wq, np.full_like(ws, 127), gl, t)
    with pytest.raises(AssertionError):
        check_gmm(gmm_unit_weight_scale)


def test_mutant_cumulative_misread_fails():
    def gmm_cum_as_count(aq, as_, wq, ws, gl, t):
        return moe_ref.gmm_mx_ref(aq, as_, wq, ws, gl, 1)  # ignores the type
    with pytest.raises(AssertionError):
        check_gmm(gmm_cum_as_count)


def test_mutant_gate_up_swapped_fails():
    def swapped(aq, as_, w13q, w13s, gl, t, I):
        w = np.concatenate([w13q[:, I:], w13q[:, :I]], axis=1)
        s = np.concatenate([w13s[:, I:], w13s[:, :I]], axis=1)
        return moe_ref.gmm_swiglu_mxquant_ref(aq, as_, w, s, gl, t, I)
    with pytest.raises(AssertionError):
        check_swiglu(swapped)


def test_mutant_finalize_fma_or_order_fails():
    def fin_weights_reversed(y, w, eri):
        return moe_ref.finalize_ref(y, w[:, ::-1], eri)
    with pytest.raises(AssertionError):
        check_finalize(fin_weights_reversed)

    def fin_f64_accumulate(y, w, eri):
        T, k = w.shape
        yy = mx_ref.bf16_to_f64(y)
        acc = sum(w[:, j:j + 1].astype(np.float64) * yy[np.asarray(eri).reshape(T, k)[:, j]] for j in range(k))
        return mx_ref.f32_to_bf16(acc.astype(np.float32) + np.float32(0))
    # float64 accumulation differs from the float32 chain only in edge cases;
    # the 2^24 + 1 - 2^24 case catches it
    with pytest.raises(AssertionError):
        check_finalize(fin_f64_accumulate)


def test_mutant_dropped_requant_fails():
    def forward_no_requant(x, ids, w, w13q, w13s, w2q, w2s):
        r = moe_ref.moe_forward_ref(x, ids, w, w13q, w13s, w2q, w2s)
        # pretend GEMM2 read h rounded to bf16 instead of the MX bytes
        h = r["h"]
        hq, hs = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(mx_ref.f32_to_bf16(h)))
        y = moe_ref.gmm_mx_ref(hq, hs, w2q, w2s, r["counts"], 1)
        r["out"] = moe_ref.finalize_ref(y, w, r["expanded_row_idx"])
        return r
    with pytest.raises(AssertionError):
        check_pipeline_vs_bruteforce(forward_no_requant, CONFIGS["tiny"])
