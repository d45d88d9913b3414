"""Pins for the oracle's MX codecs and block quantiser (CPU only).

Each check is written as a function of the implementation under test so the
mutation tests at the bottom can show that a plausible mistake planted in the
oracle fails at least one pin.
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import mx_ref

RNG = np.random.default_rng(1234)


# --------------------------------------------------------------------------
# e4m3 decode (P1): closed forms from the format definition
# --------------------------------------------------------------------------

def check_decode(decode):
    v = decode(np.arange(256))
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9                 # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert v[0x08] == 2.0 ** -6                 # smallest normal
    assert v[0x38] == 1.0                       # exponent field 7 = bias
    assert v[0x3C] == 1.5
    assert v[0x7E] == 448.0                     # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)             # codes ordered by value
    assert np.array_equal(v[0x80:0xFF], -pos)   # sign bit
    # every normal code: (1 + m/8) 2^(e-7)
    for c in range(0x08, 0x7F):
        e, m = c >> 3, c & 7
        assert v[c] == math.ldexp(1 + m / 8, e - 7)


def test_e4m3_decode_closed_form():
    check_decode(mx_ref.e4m3_decode)


def test_e4m3_decode_matches_torch():
    """Library cross-check: torch's float8_e4m3fn view of every byte."""
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = t.to(torch.float64).numpy()
    ours = mx_ref.e4m3_decode(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.all(both_nan | (ref == ours))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(ours[~both_nan]))


# --------------------------------------------------------------------------
# e4m3 encode (P2): torch's RNE cast after clamping, and brute force
# --------------------------------------------------------------------------

def torch_encode(v):
    """torch's float8_e4m3fn cast is RNE but not saturating: clamp first."""
    a = np.clip(np.asarray(v, np.float32), -448.0, 448.0)
    return torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def brute_encode(v):
    """Nearest finite e4m3 value; ties to the even mantissa; saturating."""
    grid = mx_ref.e4m3_decode(np.arange(0x7F))          # 0 .. 448, ascending
    out = []
    for x in np.asarray(v, np.float64).ravel():
        a = min(abs(x), 448.0)
        d = np.abs(grid - a)
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        out.append(code | (0x80 if np.signbit(x) else 0))
    return np.array(out, np.uint8).reshape(np.shape(v))


def midpoints():
    g = mx_ref.e4m3_decode(np.arange(0x7F))
    mids = (g[:-1] + g[1:]) / 2
    mids = np.append(mids, 464.0)                        # 448 / 480 midpoint
    m32 = mids.astype(np.float32)
    up = np.nextafter(m32, np.float32(1e9))
    dn = np.nextafter(m32, np.float32(0))
    pts = np.concatenate([g, m32, up, dn]).astype(np.float32)
    return np.concatenate([pts, -pts])


def check_encode(encode):
    pts = midpoints()
    assert np.array_equal(encode(pts.astype(np.float64)), torch_encode(pts))
    r = (RNG.standard_normal(20000) * np.exp2(RNG.integers(-14, 10, 20000))).astype(np.float32)
    assert np.array_equal(encode(r.astype(np.float64)), torch_encode(r))
    # saturation and signed zero
    big = np.array([448.0, 463.99, 464.0, 465.0, 1e6, -1e6], np.float64)
    assert encode(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    tiny = np.array([0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 1e-30, -1e-30], np.float64)
    assert encode(tiny).tolist() == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]
    assert encode(np.array([1.5 * 2.0 ** -9]))[0] == 0x02       # tie -> even (2)
    assert encode(np.array([2.5 * 2.0 ** -9]))[0] == 0x02
    assert encode(np.array([1.0625]))[0] == 0x38                 # tie 1 / 1.125 -> 1
    assert encode(np.array([1.1875]))[0] == 0x3A                 # tie 1.125/1.25 -> 1.25


def test_e4m3_encode_vs_torch_and_closed_forms():
    check_encode(mx_ref.e4m3_encode)


def test_e4m3_encode_brute_force():
    pts = np.concatenate([midpoints().astype(np.float64),
                          RNG.uniform(-500, 500, 3000), RNG.uniform(-0.02, 0.02, 1000)])
    assert np.array_equal(mx_ref.e4m3_encode(pts), brute_encode(pts))


def test_e4m3_encode_all_bf16_values():
    """Every finite bf16 value (what the activation path feeds the encoder)."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(mx_ref.e4m3_encode(f.astype(np.float64)), torch_encode(f))


def test_e4m3_roundtrip_on_grid():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(mx_ref.e4m3_encode(mx_ref.e4m3_decode(codes)), codes)


# --------------------------------------------------------------------------
# e8m0 and the block exponent (P3, R1, R3, R4)
# --------------------------------------------------------------------------

def test_format_constants_from_pages():
    g = read_golden("mx_format.txt")
    assert mx_ref.BLOCK == g["block"]
    assert mx_ref.E8M0_BIAS == g["e8m0_bias"]
    assert mx_ref.e8m0_decode(np.array([g["e8m0_bias"]]))[0] == 1.0


def check_block_exponent(fn):
    cases = {1.0: -8, 448.0: 0, 256.0: 0, 255.99: -1, 511.0: 0, 512.0: 1,
             2.0 ** -6: -14, 0.0: -127, 3.0e38: 119, 2.0 ** -119: -127,
             2.0 ** -118: -126, 2.0 ** -133: -127, 1.5: -8}
    for a, s in cases.items():
        assert int(fn(np.array([a]))[0]) == s, (a, s)


def test_block_exponent_closed_form():
    check_block_exponent(mx_ref.block_scale_exponent)


def test_e8m0_decode():
    b = np.arange(255)
    assert np.array_equal(mx_ref.e8m0_decode(b), np.exp2(b - 127.0))


# --------------------------------------------------------------------------
# bf16 rounding vs torch
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    u = RNG.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38)]
    ties = ((RNG.integers(0, 2 ** 16, 5000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) < 3e38)]
    f = np.concatenate([f, ties])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mx_ref.f32_to_bf16(f), ref)
    back = mx_ref.bf16_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


# --------------------------------------------------------------------------
# the block quantiser (P4, P5, P12)
# --------------------------------------------------------------------------

def test_pair_split_worked_example():
    g = read_golden("offline_scale_padding.txt")
    K = g["K"]
    x = RNG.standard_normal((3, K))
    q, s = mx_ref.mx_quantize_ref(x)
    assert q.shape == (3, K)
    assert -(-K // 32) == g["scales"]
    assert s.shape == (3, g["pairs"], 2) and s.shape[1] * 2 == g["padded"]
    assert s.shape[1] == mx_ref.n_scale_pairs(K)
    flat = s.reshape(3, -1)
    assert np.all(flat[:, g["scales"]:] == 0)            # the synthetic partner
    assert np.all(flat[:, :g["scales"]] > 0)


def test_pair_split_is_contiguous_pairing():
    """[R, K/32] scales viewed as [R, K/64, 2]: pair j = scales 2j, 2j+1."""
    x = np.zeros((1, 256))
    for b in range(8):                                    # block b amax = 2^b
        x[0, 32 * b + 5] = 2.0 ** b
    _, s = mx_ref.mx_quantize_ref(x)
    assert s.shape == (1, 4, 2)
    expect = np.array([119 + b for b in range(8)]).reshape(4, 2)
    assert np.array_equal(s[0], expect)


def check_quantizer(quant, dequant):
    R, K = 64, 512
    x = RNG.standard_normal((R, K)) * np.exp2(RNG.integers(-20, 20, (R, 1)))
    x[3, 64:96] = 0.0                                   # all-zero block
    x[4, :32] = 1e-42                                   # subnormal block (float32 range)
    q, s = quant(x)
    sf = s.reshape(R, -1)
    xb = x.reshape(R, K // 32, 32)
    qb = q.reshape(R, K // 32, 32)
    # all-zero block: scale byte 0, payload 0 (R3)
    assert sf[3, 2] == 0 and np.all(qb[3, 2] == 0)
    # scale byte from amax (R1): floor(log2 amax) - 8 + 127
    amax = np.abs(xb).max(axis=2)
    nz = amax > 1e-30
    expect = np.clip(np.floor(np.log2(amax[nz])) - 8 + 127, 0, 254)
    assert np.array_equal(sf[nz], expect.astype(np.uint8))
    # largest element's code has exponent field 15 when the scale is not clamped (P5)
    idx = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(qb, idx[..., None], axis=2)[..., 0]
    ok = nz & (sf > 0)
    assert np.all(((top[ok] >> 3) & 0xF) == 15)
    # round-trip error bounds (P5)
    deq = dequant(q, s).reshape(R, K // 32, 32)
    scale = np.exp2(sf.astype(np.float64) - 127)[..., None]
    v = xb / scale
    err = np.abs(deq - xb) / scale
    unsat = np.abs(v) <= 448
    half_ulp = np.where(np.abs(v) < 2.0 ** -6, 2.0 ** -10,
                        np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 1e-300))) - 4))
    assert np.all(err[unsat] <= half_ulp[unsat] * (1 + 1e-12))
    assert np.all(err[~unsat] < 64)


def test_quantizer_invariants():
    check_quantizer(mx_ref.mx_quantize_ref, mx_ref.mx_dequantize_ref)


def test_quantizer_saturates_top_element():
    x = np.zeros((1, 32))
    x[0, 0] = 1.99                                       # s = -8, 1.99*256 = 509 -> 448
    x[0, 1] = -1.99
    q, s = mx_ref.mx_quantize_ref(x)
    assert s[0, 0, 0] == 119 and q[0, 0] == 0x7E and q[0, 1] == 0xFE


def test_quantizer_exact_on_grid():
    """Values already of the form e4m3 * 2^s with a max-exponent element
    round-trip exactly."""
    codes = RNG.integers(0, 0x7F, (8, 64)).astype(np.uint8)
    codes[:, 0] = 0x78                                   # 256 -> top element exponent 15
    codes[:, 32] = 0x7E
    vals = mx_ref.e4m3_decode(codes) * np.exp2(RNG.integers(-30, 30, (8, 1)))
    q, s = mx_ref.mx_quantize_ref(vals)
    assert np.array_equal(mx_ref.mx_dequantize_ref(q, s), vals)


def test_no_zero_point():
    """P12: zero payload dequantises to zero at every scale (no offset)."""
    q = np.zeros((1, 255 * 32), np.uint8)
    s = np.concatenate([np.arange(255, dtype=np.uint8), [0]]).reshape(1, -1, 2)
    assert np.all(mx_ref.mx_dequantize_ref(q, s) == 0)


def test_partial_block():
    x = RNG.standard_normal((2, 40))
    q, s = mx_ref.mx_quantize_ref(x)
    assert q.shape == (2, 40) and s.shape == (2, 1, 2)
    q2, s2 = mx_ref.mx_quantize_ref(x[:, 32:])          # last partial block alone
    assert np.array_equal(q[:, 32:], q2) and np.array_equal(s[:, 0, 1], s2[:, 0, 0])


# --------------------------------------------------------------------------
# mutation tests: a planted mistake in the oracle must fail a pin
# --------------------------------------------------------------------------

def _enc_round_half_up(v):
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), 448.0)
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    sp = np.exp2(e - 3.0)
    qq = np.floor(a / sp + 0.5).astype(np.int64)
    return ((8 * (e + 6) + qq) | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _enc_drop_sign_of_zero(v):
    c = mx_ref.e4m3_encode(v)
    return np.where((c & 0x7F) == 0, 0, c).astype(np.uint8)


def _enc_no_subnormals(v):
    v = np.asarray(v, np.float64)
    c = mx_ref.e4m3_encode(v)
    return np.where(np.abs(v) < 2.0 ** -6, c & 0x80, c).astype(np.uint8)


@pytest.mark.parametrize("mutant", [_enc_round_half_up, _enc_drop_sign_of_zero, _enc_no_subnormals])
def test_mutant_encoders_fail(mutant):
    with pytest.raises(AssertionError):
        check_encode(mutant)


def test_mutant_decode_fails():
    def bad(c):                                          # exponent bias off by one
        v = mx_ref.e4m3_decode(c)
        return v * 2.0
    with pytest.raises(AssertionError):
        check_decode(bad)


@pytest.mark.parametrize("shift", [-1, 1])
def test_mutant_block_exponent_fails(shift):
    with pytest.raises(AssertionError):
        check_block_exponent(lambda a: mx_ref.block_scale_exponent(a) + shift)


def test_mutant_ceil_exponent_fails():
    """The no-saturation alternative s = ceil(log2(amax/448)) is rejected."""
    def ceil_rule(amax):
        amax = np.asarray(amax, np.float64)
        with np.errstate(divide="ignore"):
            s = np.ceil(np.log2(amax / 448.0))
        s = np.where(amax == 0, -127, s)
        return np.clip(s, -127, 127).astype(np.int64)
    with pytest.raises(AssertionError):
        check_block_exponent(ceil_rule)


def test_mutant_quantizer_fails():
    def quant_no_scale(x):                               # forgets to divide by the scale
        q, s = mx_ref.mx_quantize_ref(x)
        return mx_ref.e4m3_encode(np.asarray(x, np.float64)), s
    with pytest.raises(AssertionError):
        check_quantizer(quant_no_scale, mx_ref.mx_dequantize_ref)
