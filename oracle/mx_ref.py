"""MX codecs and block quantiser (oracle; test infrastructure only).

Formats, as the pages fix them:

* Payload is FP8 e4m3 ("float8_e4m3fn"): "Quantization on Ascend", MXFP8 for
  LLM MoE implementation notes (offline path loads float8_e4m3fn expert
  weights).  The bit layout (1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits, no infinities, S.1111.111 = NaN, largest finite 448) is the OCP FP8
  e4m3 definition; the pages name the dtype but print none of its constants.
* Scale is e8m0 held in a uint8 as exponent + 127: same page and section
  (offline scales described as uint8, exponent plus 127).
* One scale per 32 consecutive elements along the reduction dimension:
  same page, dense MXFP8 implementation notes (block size 32).
* ceil(K/32) scales per row; an odd count gets one zero-valued partner so the
  row can be viewed as [ceil(K/64), 2] pairs: "[WIP] Fix offline W8A8 MXFP8
  quantization for Qwen3.5 on Ascend NPU", Summary, offline partial MXFP8
  block-scale layout and offline scale padding (worked example K = 4304).

Readings of points the pages leave open (numbered as in the design notes):

* R1  scale exponent s = floor(log2(amax)) - 8, clamped to [-127, 127]
      (OCP MX rule: shared exponent minus the element format's largest
      exponent, 8 for e4m3).  The largest element may then saturate to 448.
* R2  element rounding is round-to-nearest, ties to even mantissa, with
      saturation to +-448.
* R3  an all-zero block gets scale byte 0 and zero payload.
* R5  the sign is kept, so a negative value that rounds to zero (and -0.0)
      encodes as 0x80.
* R7  e4m3 subnormals are kept.

MXFP4 weights (the W4A8 path): "Quantization on Ascend", W4A8 implementation
notes: weights packed FP4 (float4_e2m1fn_x2, two nibbles per byte) with a
UE8M0 shared exponent per block of 32; activations stay MXFP8.

* R29 e2m1 is 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no
      infinities or NaN: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (the OCP
      e2m1 definition; the pages name the dtype only).
* R30 two codes per byte, element 2i in the low nibble, 2i+1 in the high
      nibble (the x2 dtype's order).
* R31 the MXFP4 scale exponent is floor(log2(amax)) - 2 (2 = e2m1's largest
      exponent), clamped to [-127, 127]; elements round to nearest, ties to
      even code, saturating at +-6, sign kept (a negative that rounds to 0
      gives code 8).

Everything is computed in float64 on exact values; no step depends on
summation order.
"""

import numpy as np

BLOCK = 32            # elements per MX block
E4M3_MAX = 448.0      # largest finite e4m3 magnitude (S.1111.110)
E4M3_EMAX = 8         # exponent of the largest e4m3 binade
E8M0_BIAS = 127       # scale byte = exponent + 127
E2M1_MAX = 6.0        # largest e2m1 magnitude
E2M1_EMAX = 2         # exponent of the largest e2m1 binade


# --------------------------------------------------------------------------
# e4m3
# --------------------------------------------------------------------------

def e4m3_decode(codes):
    """Value of each e4m3 code as float64 (NaN for 0x7F / 0xFF).

    Normal codes: (1 + m/8) * 2^(e - 7) for exponent field e in 1..15;
    subnormal codes: m * 2^-9 for e = 0.  No infinities.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    mag = np.where(ef == 0, mf * 2.0 ** -9, (1.0 + mf / 8.0) * np.exp2(ef - 7.0))
    mag = np.where((ef == 15) & (mf == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e4m3_encode(v):
    """Round float64 values to e4m3 codes: nearest, ties to even, saturating.

    a = min(|v|, 448).  For a >= 2^-6 the grid spacing in a's binade
    [2^e, 2^(e+1)) is 2^(e-3); below 2^-6 it is the subnormal spacing 2^-9
    (the e = -6 spacing, so the formula is the same with e clamped at -6).
    q = a / spacing is rounded to the nearest integer, halves to even; the
    parity of q is the parity of the mantissa field, so this is RNE on the
    code.  The code is 8*(e+6) + q (q = 16 rolls into the next binade with the
    same formula).  The sign bit comes from v's sign bit.
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(a)                    # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    e = np.where(a == 0, -6, e)
    spacing = np.exp2(e.astype(np.float64) - 3.0)
    q = np.rint(a / spacing).astype(np.int64)   # exact division; rint = half-even
    code = 8 * (e + 6) + q
    assert np.all((code >= 0) & (code <= 0x7E))
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


# --------------------------------------------------------------------------
# e8m0
# --------------------------------------------------------------------------

def e8m0_decode(b):
    """2^(b - 127) for a scale byte b in 0..254 (255 is NaN, never produced)."""
    b = np.asarray(b).astype(np.int64)
    assert np.all(b != 255)
    return np.exp2(b.astype(np.float64) - E8M0_BIAS)


def block_scale_exponent(amax):
    """Shared exponent s of one block from its largest magnitude (R1, R3, R4).

    s = floor(log2(amax)) - 8 clamped to [-127, 127]; amax = 0 gives -127.
    floor(log2) is read exactly with frexp, which also covers subnormal amax.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    s = ex.astype(np.int64) - 1 - E4M3_EMAX
    s = np.where(amax == 0, -E8M0_BIAS, s)
    return np.clip(s, -127, 127)


# --------------------------------------------------------------------------
# bf16 (bit patterns held in uint16)
# --------------------------------------------------------------------------

def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    u = np.asarray(bits).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16(x):
    """Round float32 values to bf16 bit patterns, nearest with ties to even.

    The low 16 bits are dropped after adding 0x7FFF plus the bit that will
    become the last kept bit; finite inputs only (the oracle never makes
    NaN or Inf).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    assert np.all((u & 0x7F800000) != 0x7F800000), "non-finite value"
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


# --------------------------------------------------------------------------
# MX block quantise / dequantise
# --------------------------------------------------------------------------

def n_scale_pairs(kd):
    """Number of scale pairs per row: ceil(ceil(Kd/32) / 2) = ceil(Kd/64)."""
    return -(-kd // 64)


def mx_quantize_ref(v):
    """MX-quantise each row of v [R, Kd] (exact float values, e.g. bf16 or fp32).

    Per row, per block c of 32 consecutive elements (the last block may be
    partial): amax over the block, shared exponent s (R1), scale byte s + 127,
    payload e4m3_encode(v * 2^-s).  Scales are laid out as [R, ceil(Kd/64), 2]
    with a zero partner byte when ceil(Kd/32) is odd.

    Returns (q uint8 [R, Kd], s uint8 [R, ceil(Kd/64), 2]).
    """
    v = np.asarray(v, dtype=np.float64)
    assert v.ndim == 2
    R, Kd = v.shape
    nb = -(-Kd // BLOCK)
    pad = nb * BLOCK - Kd
    vp = np.concatenate([v, np.zeros((R, pad))], axis=1) if pad else v
    blocks = vp.reshape(R, nb, BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    s = block_scale_exponent(amax)                              # [R, nb]
    scaled = blocks * np.exp2(-s.astype(np.float64))[:, :, None]  # exact
    q = e4m3_encode(scaled).reshape(R, nb * BLOCK)[:, :Kd]
    sb = (s + E8M0_BIAS).astype(np.uint8)
    if nb % 2:
        sb = np.concatenate([sb, np.zeros((R, 1), np.uint8)], axis=1)
    return q.copy(), sb.reshape(R, sb.shape[1] // 2, 2)


def mx_dequantize_ref(q, s, kd=None):
    """Dequantise: e4m3 value times 2^(scale byte - 127); no zero point.

    q uint8 [R, Kd]; s uint8 [R, ceil(Kd/64), 2] (or any shape whose last
    two dims flatten to >= ceil(Kd/32) per row).  Returns float64 [R, Kd].
    There is no offset term: the pages state MXFP8 has no zero point
    ("[WIP] Fix offline W8A8 MXFP8 ...", commit on the missing weight offset).
    """
    q = np.asarray(q)
    R, Kd = q.shape
    if kd is not None:
        assert kd == Kd
    nb = -(-Kd // BLOCK)
    sf = np.asarray(s).reshape(R, -1)[:, :nb]
    scale = e8m0_decode(sf)                               # [R, nb]
    scale_el = np.repeat(scale, BLOCK, axis=1)[:, :Kd]
    return e4m3_decode(q) * scale_el


def scales_flat(s, kd):
    """[R, ceil(Kd/64), 2] pair-split scales -> [R, ceil(Kd/32)] (drops pad)."""
    s = np.asarray(s)
    R = s.shape[0]
    return s.reshape(R, -1)[:, : -(-kd // BLOCK)]


# --------------------------------------------------------------------------
# e2m1 and MXFP4 (weights of the W4A8 path; R29-R31)
# --------------------------------------------------------------------------

def e2m1_decode(codes):
    """e2m1 code (0..15) -> value (R29): exponent field 0 is subnormal
    (m * 0.5), otherwise 2^(e - 1) * (1 + m / 2); bit 3 is the sign."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.exp2(e - 1.0) * (1.0 + 0.5 * m))
    return sign * mag


def e2m1_encode(v):
    """Nearest e2m1 code to each value, ties to the even code, magnitudes
    above 6 saturate to 6, sign kept (R31)."""
    v = np.asarray(v, dtype=np.float64)
    grid = e2m1_decode(np.arange(8))                 # 0, .5, 1, 1.5, 2, 3, 4, 6
    a = np.minimum(np.abs(v), E2M1_MAX)
    d = np.abs(a[..., None] - grid)                  # distance to every grid point
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                 # one or two nearest points
    even = cand & ((np.arange(8) % 2) == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def block_scale_exponent_fp4(amax):
    """MXFP4 shared exponent (R31): floor(log2 amax) - 2 clamped to
    [-127, 127]; an all-zero block gets -127 (scale byte 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.full(amax.shape, -127, np.int64)
    nz = amax > 0
    e[nz] = np.floor(np.log2(amax[nz])).astype(np.int64) - E2M1_EMAX
    return np.clip(e, -127, 127)


def fp4_pack(codes):
    """[R, Kd] codes (Kd even) -> [R, Kd/2] bytes, element 2i low nibble (R30)."""
    c = np.asarray(codes).astype(np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def fp4_unpack(q):
    """[R, Kd/2] bytes -> [R, Kd] codes (R30)."""
    q = np.asarray(q).astype(np.uint8)
    out = np.empty(q.shape[:-1] + (2 * q.shape[-1],), np.uint8)
    out[..., 0::2] = q & 15
    out[..., 1::2] = q >> 4
    return out


def mxfp4_quantize_ref(v):
    """MXFP4-quantise each row of v [R, Kd] (Kd even): per block of 32, the
    shared exponent s (R31), scale byte s + 127, codes e2m1_encode(v * 2^-s)
    packed two per byte (R30).  Scales [R, ceil(Kd/64), 2] as for MXFP8.

    Returns (q uint8 [R, Kd/2], s uint8 [R, ceil(Kd/64), 2]).
    """
    v = np.asarray(v, dtype=np.float64)
    R, Kd = v.shape
    assert Kd % 2 == 0, "two codes per byte"
    nb = -(-Kd // BLOCK)
    pad = nb * BLOCK - Kd
    vp = np.concatenate([v, np.zeros((R, pad))], axis=1) if pad else v
    blocks = vp.reshape(R, nb, BLOCK)
    s = block_scale_exponent_fp4(np.max(np.abs(blocks), axis=2))
    codes = e2m1_encode(blocks * np.exp2(-s.astype(np.float64))[:, :, None]).reshape(R, nb * BLOCK)[:, :Kd]
    sb = (s + E8M0_BIAS).astype(np.uint8)
    if nb % 2:
        sb = np.concatenate([sb, np.zeros((R, 1), np.uint8)], axis=1)
    return fp4_pack(codes), sb.reshape(R, sb.shape[1] // 2, 2)


def mxfp4_dequantize_ref(q, s):
    """e2m1 value times 2^(scale byte - 127).  q [R, Kd/2]; returns [R, Kd]."""
    codes = fp4_unpack(q)
    R, Kd = codes.shape
    nb = -(-Kd // BLOCK)
    scale = e8m0_decode(np.asarray(s).reshape(R, -1)[:, :nb])
    return e2m1_decode(codes) * np.repeat(scale, BLOCK, axis=1)[:, :Kd]
