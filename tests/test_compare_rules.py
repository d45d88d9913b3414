"""CPU checks of the comparison rules the GPU parity tests use."""

import numpy as np

from gpu_util import explain_hq_mismatches, row_rel_err
from oracle import mx_ref

RNG = np.random.default_rng(5)


def _h(M=64, I=256):
    g = RNG.standard_normal((M, I))
    return (g / (1 + np.exp(-g)) * RNG.standard_normal((M, I)) * np.exp2(RNG.integers(-8, 8, (M, 1))))


def test_requant_of_perturbed_h_is_accepted():
    h = _h()
    hq, hs = mx_ref.mx_quantize_ref(h)
    rowmax = np.abs(h).max(axis=1, keepdims=True)
    h2 = h + RNG.uniform(-1, 1, h.shape) * 2e-4 * rowmax        # within the 1e-3 row tolerance
    q2, s2 = mx_ref.mx_quantize_ref(h2)
    n_mis, n_bad = explain_hq_mismatches(q2, s2, hq, h)
    assert n_mis > 0 and n_bad == 0


def test_planted_errors_are_rejected():
    h = _h()
    hq, hs = mx_ref.mx_quantize_ref(h)
    bad = hq.copy()
    big = np.abs(h) > 0.5 * np.abs(h).max(axis=1, keepdims=True)
    idx = np.argwhere(big)[:5]
    for r, c in idx:
        bad[r, c] = (bad[r, c] & 0x80) | max(0, (bad[r, c] & 0x7F) - 3)   # three codes down
    _, n_bad = explain_hq_mismatches(bad, hs, hq, h)
    assert n_bad == len(idx)
    s_bad = hs.copy()
    s_bad[0, 0, 0] += 1                                                   # scale one step up
    _, n_bad = explain_hq_mismatches(hq, s_bad, hq, h)
    assert n_bad > 0
    flipped = hq.copy()
    r, c = idx[0]
    flipped[r, c] ^= 0x80                                                 # sign flip
    _, n_bad = explain_hq_mismatches(flipped, hs, hq, h)
    assert n_bad == 1


def test_row_rel_err_rule():
    ref = np.array([[1.0, -2.0, 0.5], [0.0, 0.0, 0.0]])
    got = np.array([[1.01, -2.0, 0.5], [0.0, 0.0, 0.0]])
    e = row_rel_err(got, ref)
    assert abs(e[0] - 0.005) < 1e-12 and e[1] == 0
    got[1, 2] = 1e-3
    assert row_rel_err(got, ref)[1] == 1e-3
