"""W4A8 path (MXFP4 e2m1 weights x MXFP8 activations) on the GPU against the
oracle (readings R29-R31)."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_topk_amd as mx
from gpu_util import bf16_dev, host, say
from oracle import mx_ref
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


def _check_fp4_quant(x_bits, q, s):
    rq, rs = mx_ref.mxfp4_quantize_ref(mx_ref.bf16_to_f64(x_bits))
    assert np.array_equal(host(s).reshape(rs.shape), rs), "scale bytes differ"
    assert np.array_equal(host(q).reshape(rq.shape), rq), "e2m1 codes differ"


def test_mx_quantize_fp4_random_rows():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((97, 512)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (97, 1))).astype(np.float32)
    x[5, 64:96] = 0.0                                    # an all-zero block
    x[6, :32] = np.float32(-0.0)
    bits = to_bf16_bits(x)
    say("mx_quantize_fp4 random rows 97x512")
    q, s = mx.mx_quantize_fp4(bf16_dev(bits))
    torch.cuda.synchronize()
    _check_fp4_quant(bits, q, s)


@pytest.mark.parametrize("shape", [(11, 4128), (6, 2080), (1, 32)])
def test_mx_quantize_fp4_long_and_short_rows(shape):
    """Rows longer than one pass of a wave's loads, with a ragged last pass."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal(shape).astype(np.float32) * np.exp2(rng.integers(-20, 20, (shape[0], 1))).astype(np.float32)
    bits = to_bf16_bits(x)
    say(f"mx_quantize_fp4 rows {shape}")
    q, s = mx.mx_quantize_fp4(bf16_dev(bits))
    torch.cuda.synchronize()
    _check_fp4_quant(bits, q, s)


def test_mx_quantize_fp4_every_bf16_value():
    """Every finite bf16 bit pattern, 32 per block in ascending order."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[((allb >> 7) & 0xFF) != 0xFF]
    n = len(fin) // 32 * 32
    bits = fin[:n].reshape(-1, 256)
    say(f"mx_quantize_fp4 every finite bf16 value ({bits.size})")
    q, s = mx.mx_quantize_fp4(bf16_dev(bits))
    torch.cuda.synchronize()
    _check_fp4_quant(bits, q, s)


def test_mx_quantize_fp4_strided_and_odd_scale_count():
    rng = np.random.default_rng(32)
    x = to_bf16_bits(rng.standard_normal((40, 160)).astype(np.float32))
    xd = bf16_dev(x)[:, :96]                             # row stride 160, kd = 96 (3 scales)
    say("mx_quantize_fp4 strided kd=96")
    q, s = mx.mx_quantize_fp4(xd)
    torch.cuda.synchronize()
    _check_fp4_quant(x[:, :96], q, s)
    assert np.all(host(s)[:, 1, 1] == 0)                 # the pad partner of the odd count


# --------------------------------------------------------------------------
# grouped GEMMs with e2m1 weights
# --------------------------------------------------------------------------

from gpu_util import bf16_host, bf16_rows_rel_err, check_layer_every_row, explain_hq_mismatches, f32_dev, \
    guard_alloc, guards_intact, i32_dev, i64_dev, row_rel_err, u8_dev  # noqa: E402
from oracle import moe_ref  # noqa: E402
from workloads import CONFIGS, custom_config, make_inputs, make_weights_w4a8  # noqa: E402

RNG = np.random.default_rng(41)
TOL = 2e-2
E2E_TOL = 5e-2


def _w4_operands(M, Kd, E, N, spread=4):
    a = RNG.standard_normal((M, Kd)) * np.exp2(RNG.integers(-spread, spread, (M, 1)))
    w = RNG.standard_normal((E * N, Kd)) * 0.05 * np.exp2(RNG.integers(-spread, spread, (E * N, 1)))
    aq, as_ = mx_ref.mx_quantize_ref(a)
    wq, ws = mx_ref.mxfp4_quantize_ref(w)
    return aq, as_, wq.reshape(E, N, Kd // 2), ws.reshape(E, N, -1, 2)


W4_GMM_CASES = {
    "ragged": ([0, 1, 127, 128, 129, 255, 256, 257, 300, 0, 5], 256, 256),
    "single-expert": ([515], 384, 256),
    "wide-k": ([64, 200, 33], 1024, 256),
    "multi-tile-n": ([700, 20], 256, 768),
    # 128-row tiles (three-slot ring): 3 k stages, tails at 16/32/128 rows
    "small-tiles-3stage": ([16, 33, 129, 0, 255] + [0] * 2, 384, 256),
    "small-tiles-4stage": ([16, 33, 129, 0, 255] + [0] * 2, 512, 256),
}


@pytest.mark.parametrize("name", list(W4_GMM_CASES))
def test_gmm_mx_w4a8_parity(name):
    counts, Kd, N = W4_GMM_CASES[name]
    counts = np.array(counts, np.int64)
    M, E = int(counts.sum()), len(counts)
    say(f"gmm_mx_w4a8 {name} M={M} Kd={Kd} N={N} E={E}")
    aq, as_, wq, ws = _w4_operands(M, Kd, E, N)
    y = mx.gmm_mx_w4a8(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(counts), 1)
    y0 = mx.gmm_mx_w4a8(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(np.cumsum(counts)), 0)
    torch.cuda.synchronize()
    ref = moe_ref.gmm_mx_ref(aq, as_, wq, ws, counts, 1, "e2m1")
    err = bf16_rows_rel_err(bf16_host(y), ref)
    say(f"  max row rel err {err.max():.3g}")
    assert err.max() <= TOL
    assert np.array_equal(bf16_host(y0), bf16_host(y))


def test_gmm_mx_w4a8_exact_case():
    """One nonzero weight code per row and scale 1: y = a[:, k] * value exactly."""
    M, Kd, N = 40, 128, 256
    aq = np.zeros((M, Kd), np.uint8)
    aq[:, 7] = 0x40                                       # 2.0 at k = 7
    as_ = np.full((M, Kd // 64, 2), 127, np.uint8)
    wq = np.zeros((1, N, Kd // 2), np.uint8)
    wq[0, :, 3] = 0x70                                    # high nibble of byte 3 = k 7: code 7 = 6.0
    ws = np.full((1, N, Kd // 64, 2), 127, np.uint8)
    say("gmm_mx_w4a8 exact case")
    y = mx.gmm_mx_w4a8(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev([M]), 1)
    torch.cuda.synchronize()
    assert np.all(mx_ref.bf16_to_f64(bf16_host(y)) == 12.0)


W4_GMM1_CASES = {
    "ragged": ([3, 0, 128, 129, 1, 260, 256, 511], 256, 128),
    "wide-i": ([70, 150], 128, 384),
    # 128-row tiles (three-slot ring)
    "small-tiles-3stage": ([16, 17, 31, 33, 127, 129, 1], 384, 128),
    "small-tiles-4stage": ([16, 17, 31, 33, 127, 129, 1], 512, 128),
}


@pytest.mark.parametrize("name", list(W4_GMM1_CASES))
def test_gmm_swiglu_mxquant_w4a8_parity(name):
    counts, K, I = W4_GMM1_CASES[name]
    counts = np.array(counts, np.int64)
    M, E = int(counts.sum()), len(counts)
    say(f"gmm_swiglu_mxquant_w4a8 {name} M={M} K={K} I={I} E={E}")
    aq, as_, wq, ws = _w4_operands(M, K, E, 2 * I)
    hq, hs, h = mx.gmm_swiglu_mxquant_w4a8(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(counts), 1,
                                           h_debug=True)
    torch.cuda.synchronize()
    rq, rs, rh = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, wq, ws, counts, 1, I, "e2m1")
    hk = host(h)
    herr = row_rel_err(hk, rh)
    say(f"  h max row rel err {herr.max():.3g}")
    assert herr.max() <= 1e-3
    kq, ks = mx_ref.mx_quantize_ref(hk.astype(np.float64))
    assert np.array_equal(host(hq), kq) and np.array_equal(host(hs), ks)
    n_mis, n_bad = explain_hq_mismatches(host(hq), host(hs), rq, rh)
    say(f"  hq/hs mismatches vs oracle {n_mis} of {rq.size}, unexplained {n_bad}")
    assert n_bad == 0 and n_mis <= 0.01 * rq.size


# --------------------------------------------------------------------------
# the layer with e2m1 weights
# --------------------------------------------------------------------------

def _run_w4a8(d, wdev, name):
    cfg = d["cfg"]
    T, K, I, E, k = cfg.T, cfg.K, cfg.I, cfg.E, cfg.k
    need = mx.forward_workspace_size(T, K, I, E, k)
    raw_ws, ws = guard_alloc(need, torch.uint8, fill=0x3C)
    raw_out, out = guard_alloc(T * K, torch.bfloat16, fill=0x6B)
    say(f"moe_w4a8_forward {name} T={T} K={K} I={I} E={E} k={k}")
    mx.moe_w4a8_forward(bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"]), *wdev,
                        out=out.view(T, K), workspace=ws)
    torch.cuda.synchronize()
    assert guards_intact(raw_ws, need, fill=0x3C) and guards_intact(raw_out, T * K * 2, fill=0x6B)
    iv = mx.forward_intermediates(ws, T, K, I, E, k)
    inter = {n: host(v) for n, v in iv.items() if n != "y"}
    inter["y"] = bf16_host(iv["y"])
    return bf16_host(out.view(T, K)), inter


@pytest.mark.parametrize("shape", [("tiny", None), ("several-tiles", (300, 512, 256, 12, 4))])
def test_w4a8_forward_small(shape):
    """bf16 weights quantised to MXFP4 by the library (checked byte for byte),
    then every stage of the layer against the oracle on every row."""
    name, dims = shape
    cfg = CONFIGS["tiny"] if dims is None else custom_config(name, *dims)
    d = make_inputs(cfg)
    T, K, I, E, k = cfg.T, cfg.K, cfg.I, cfg.E, cfg.k
    w13q, w13s = mx.mx_quantize_fp4(bf16_dev(d["w13"]))
    w2q, w2s = mx.mx_quantize_fp4(bf16_dev(d["w2"]))
    torch.cuda.synchronize()
    r13q, r13s = mx_ref.mxfp4_quantize_ref(mx_ref.bf16_to_f64(d["w13"].reshape(-1, K)))
    r2q, r2s = mx_ref.mxfp4_quantize_ref(mx_ref.bf16_to_f64(d["w2"].reshape(-1, I)))
    assert np.array_equal(host(w13q).reshape(r13q.shape), r13q) and np.array_equal(host(w13s).reshape(r13s.shape), r13s)
    assert np.array_equal(host(w2q).reshape(r2q.shape), r2q) and np.array_equal(host(w2s).reshape(r2s.shape), r2s)
    out, inter = _run_w4a8(d, [w13q, w13s, w2q, w2s], cfg.name)
    check_layer_every_row(d, out, inter, r13q.reshape(E, 2 * I, K // 2), r13s.reshape(E, 2 * I, -1, 2),
                          r2q.reshape(E, K, I // 2), r2s.reshape(E, K, -1, 2), "e2m1", TOL, E2E_TOL)


@pytest.mark.timeout(900)
def test_w4a8_forward_prefill_every_row():
    """The 16K prefill layer with checkpoint-style MXFP4 weights, in the
    benchmark's launch configuration: every row of every stage against the
    oracle (GEMM2 on identical operands at 2e-2, finalize bit-exact)."""
    cfg = CONFIGS["prefill"]
    d = make_inputs(cfg, weights=False)
    wts = make_weights_w4a8(cfg)
    wdev = [u8_dev(wts[n]) for n in ("w13q4", "w13s4", "w2q4", "w2s4")]
    out, inter = _run_w4a8(d, wdev, "prefill")
    del wdev
    check_layer_every_row(d, out, inter, wts["w13q4"], wts["w13s4"], wts["w2q4"], wts["w2s4"], "e2m1", TOL,
                          E2E_TOL)
