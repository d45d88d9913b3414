"""Pins for the router oracle (``oracle.moe_ref.router_ref``, reading R28),
each against something other than its own formula: brute force over expert
subsets, closed forms, invariants, and an exactly rounded dot product."""

import itertools
import math

import numpy as np
import pytest

from oracle.moe_ref import router_ref
from oracle.mx_ref import bf16_to_f64
from workloads import to_bf16_bits


def _bits(a):
    return to_bf16_bits(np.asarray(a, np.float32))


def _integer_router_inputs(rng, T, E, K):
    """x and gate with small integer entries (exact in bf16): the logits are
    exact integers, so ties between experts are common."""
    x = rng.integers(-2, 3, size=(T, K)).astype(np.float32)
    g = rng.integers(-2, 3, size=(E, K)).astype(np.float32)
    return _bits(x), _bits(g), x.astype(np.float64) @ g.astype(np.float64).T


@pytest.mark.parametrize("E,k", [(5, 1), (6, 2), (7, 3), (4, 4)])
@pytest.mark.parametrize("renormalize", [True, False])
def test_router_matches_subset_brute_force(E, k, renormalize):
    rng = np.random.default_rng(100 + 10 * E + k)
    xb, gb, logits = _integer_router_inputs(rng, 64, E, 3)
    ids, w, _ = router_ref(xb, gb, None, k, renormalize)
    for t in range(logits.shape[0]):
        lt = logits[t]
        # the k-subset with the largest logit sum; among equal sums the
        # lexicographically smallest id tuple (= lower ids win ties)
        best = max(itertools.combinations(range(E), k), key=lambda S: (sum(lt[list(S)]), [-e for e in S]))
        order = sorted(best, key=lambda e: (-lt[e], e))
        assert list(ids[t]) == order, (t, lt, ids[t], order)
        # weights from the closed form 1 / sum_j exp(l_j - l_e)
        pool = order if renormalize else range(E)
        want = [1.0 / sum(math.exp(lt[j] - lt[e]) for j in pool) for e in order]
        np.testing.assert_allclose(w[t], np.float32(want), rtol=1e-6)


@pytest.mark.parametrize("renormalize", [True, False])
def test_router_uniform_logits(renormalize):
    """A zero gate makes every logit equal: experts 0..k-1, weight 1/k (or 1/E)."""
    T, E, K, k = 7, 16, 32, 5
    xb = _bits(np.random.default_rng(1).standard_normal((T, K)))
    gb = _bits(np.zeros((E, K)))
    ids, w, _ = router_ref(xb, gb, None, k, renormalize)
    assert (ids == np.arange(k)[None, :]).all()
    np.testing.assert_allclose(w, 1.0 / (k if renormalize else E), rtol=1e-7)


def test_router_two_experts_closed_form():
    """E=2, k=1, no renormalisation: w = 1 / (1 + exp(l_other - l_chosen))."""
    rng = np.random.default_rng(2)
    xb = _bits(rng.standard_normal((40, 8)))
    gb = _bits(rng.standard_normal((2, 8)))
    ids, w, logits = router_ref(xb, gb, None, 1, False)
    for t in range(40):
        e = int(ids[t, 0])
        assert logits[t, e] >= logits[t, 1 - e]
        assert w[t, 0] == np.float32(1.0 / (1.0 + math.exp(logits[t, 1 - e] - logits[t, e])))


def test_router_shift_invariance():
    rng = np.random.default_rng(3)
    xb = _bits(rng.standard_normal((32, 64)))
    gb = _bits(0.02 * rng.standard_normal((12, 64)))
    ids0, w0, _ = router_ref(xb, gb, None, 4, True)
    ids1, w1, _ = router_ref(xb, gb, np.full(12, 37.25), 4, True)
    assert (ids0 == ids1).all()
    np.testing.assert_allclose(w0, w1, rtol=1e-6)


def test_router_minus_inf_bias_never_chosen():
    rng = np.random.default_rng(4)
    xb = _bits(rng.standard_normal((200, 32)))
    gb = _bits(rng.standard_normal((10, 32)))
    bias = np.zeros(10)
    bias[[2, 7]] = -np.inf
    ids, w, _ = router_ref(xb, gb, bias, 8, True)
    assert not np.isin(ids, [2, 7]).any()
    assert np.isfinite(w).all()
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    # weights follow the logits' order
    assert (np.diff(w, axis=1) <= 0).all()


def test_router_logits_against_exact_sums():
    """The logits equal exactly rounded sums of the decoded bf16 products
    (catches a transposed or mis-decoded operand)."""
    rng = np.random.default_rng(5)
    T, E, K = 5, 6, 48
    xb = _bits(rng.standard_normal((T, K)))
    gb = _bits(0.02 * rng.standard_normal((E, K)))
    bias = rng.standard_normal(E)
    _, _, logits = router_ref(xb, gb, bias, 2, True)
    xd, gd = bf16_to_f64(xb), bf16_to_f64(gb)
    for t in range(T):
        for e in range(E):
            exact = math.fsum([float(xd[t, c]) * float(gd[e, c]) for c in range(K)] + [float(bias[e])])
            assert abs(logits[t, e] - exact) <= 1e-12 * max(1.0, abs(exact))
