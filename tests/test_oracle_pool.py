"""The pooled oracle helpers (used by the full-size GPU parity tests) give
exactly the bytes of the oracle's whole-matrix routines.

Row chunks are made deliberately small and ragged here so that every expert
is split across several worker tasks."""

import numpy as np
import pytest

import oracle_pool
from oracle import moe_ref, mx_ref
from workloads import to_bf16_bits

RNG = np.random.default_rng(99)


def _case(M_per_e, K, N, w_format="e4m3"):
    E = len(M_per_e)
    counts = np.array(M_per_e, np.int64)
    M = int(counts.sum())
    x = to_bf16_bits(RNG.standard_normal((M, K)).astype(np.float32))
    aq, as_ = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(x))
    w = to_bf16_bits((RNG.standard_normal((E * N, K)) * 0.05).astype(np.float32))
    if w_format == "e4m3":
        wq, ws = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(w))
        wq = wq.reshape(E, N, K)
    else:
        wq, ws = mx_ref.mxfp4_quantize_ref(mx_ref.bf16_to_f64(w))
        wq = wq.reshape(E, N, K // 2)
    return counts, x, aq, as_, wq, ws.reshape(E, N, -1, 2)


@pytest.mark.parametrize("w_format", ["e4m3", "e2m1"])
def test_pooled_gemms_equal_the_oracle(w_format):
    counts, _, aq, as_, wq, ws = _case([5, 0, 13, 1, 9], 128, 64, w_format)
    I = 32
    _, _, h_ref = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, wq, ws, counts, 1, I, w_format)
    h = oracle_pool.gemm1_h(aq, as_, wq, ws, counts, 1, I, w_format, rows=3)
    assert np.array_equal(h.view(np.uint32), h_ref.view(np.uint32))
    y_ref = moe_ref.gmm_mx_ref(aq, as_, wq, ws, np.cumsum(counts), 0, w_format)
    y = oracle_pool.gemm2_y(aq, as_, wq, ws, np.cumsum(counts), 0, w_format, rows=4)
    assert np.array_equal(y, y_ref)
    # a subset of rows, written into an existing array
    rows = np.array([0, 4, 6, 17, 27])
    part = np.zeros_like(y_ref)
    oracle_pool.gemm2_y(aq, as_, wq, ws, counts, 1, w_format, rows=2, only_rows=rows, out=part)
    assert np.array_equal(part[rows], y_ref[rows])
    others = np.setdiff1d(np.arange(part.shape[0]), rows)
    assert not part[others].any()


def test_pooled_quantisers_equal_the_oracle():
    v = (RNG.standard_normal((37, 96)) * np.exp2(RNG.integers(-20, 20, (37, 1)))).astype(np.float32)
    q, s = oracle_pool.quantize_f32(v, rows=5)
    qr, sr = mx_ref.mx_quantize_ref(v.astype(np.float64))
    assert np.array_equal(q, qr) and np.array_equal(s, sr)
    bits = to_bf16_bits(v)
    q, s = oracle_pool.quantize_bf16(bits, rows=6)
    qr, sr = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(bits))
    assert np.array_equal(q, qr) and np.array_equal(s, sr)
    q, s = oracle_pool.quantize_bf16(bits, rows=6, fp4=True)
    qr, sr = mx_ref.mxfp4_quantize_ref(mx_ref.bf16_to_f64(bits))
    assert np.array_equal(q, qr) and np.array_equal(s, sr)


def test_pooled_routing_and_finalize_equal_the_oracle():
    T, K, k, E = 53, 96, 3, 7
    x = to_bf16_bits(RNG.standard_normal((T, K)).astype(np.float32))
    ids = np.stack([RNG.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    got = oracle_pool.route_quant(x, ids, E, rows=5)
    ref = moe_ref.route_quant_ref(x, ids, E)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    y = to_bf16_bits((RNG.standard_normal((T * k, K)) * np.exp2(RNG.integers(-9, 9, (T * k, 1)))).astype(np.float32))
    w = RNG.random((T, k)).astype(np.float32)
    eri = RNG.permutation(T * k).astype(np.int32)
    assert np.array_equal(oracle_pool.finalize(y, w, eri, tokens=4), moe_ref.finalize_ref(y, w, eri))
