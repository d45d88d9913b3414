"""Seeded random sweeps of the layer's kernels against the oracle.

Complements the hand-picked cases in test_gpu_kernels.py with drawn ones,
each case's sizes and data from its own seed:

* both grouped GEMMs: expert counts from three mixes (decode-like 0-5 rows
  per expert, counts at and around the 32/64/128/256-row boundaries, and
  large ragged experts), reduction sizes that switch between per-stage scale
  loads (stages not a multiple of 4) and 4-stage scale groups, and group lists
  that select either tile height (128-token tiles when the experts average at
  most 64 rows and there are at least 3 k stages); the same weights
  tile-packed must give the same bytes, and MXFP4 (e2m1) weights are held to
  the same bars;
* moe_route_quant: token counts on both sides of the one-chunk boundary and
  up to several leader batches, expert counts up to 1024, skewed and uniform
  expert choice; bit-exact;
* moe_finalize: row widths on both sides of the wave-per-token layout (K a
  multiple of 512 or not), a few dropped assignments; bit-exact;
* moe_router: token counts around the 64-token workgroup, 2 to 256 experts,
  no bias, a finite bias or experts barred by a -inf bias, with and without
  renormalisation; checked as the router tests check it (the selection
  exact wherever no float32 near-tie decides it);
* the whole layer (moe_mxfp8_forward) on drawn sizes, routings (plain, Zipf
  bias, hot and never-chosen experts) and outlier channels: every row of every
  stage against the oracle, with the weights quantised on the GPU equal to
  the oracle's; the same layer on tile-packed weights gives the same bytes,
  and with MXFP4 weights (moe_w4a8_forward) meets the same bars;
* mx_linear (the dense linear) on drawn sizes, every row.
"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_topk_amd as mx
import oracle_pool
from gpu_util import (bf16_dev, bf16_host, bf16_rows_rel_err, check_layer_every_row, check_router, explain_hq_mismatches,
                      f32_dev, host, i32_dev, i64_dev, row_rel_err, run_router, say, u8_dev)
from oracle import moe_ref, mx_ref
from workloads import custom_config, make_inputs, to_bf16_bits

pytestmark = pytest.mark.gpu
TOL = 2e-2
MAX_ROWS = 4096
SEEDS = list(range(8))


def draw_case(seed, n_choices):
    """(rng, counts [E] int64, Kd, n): the case's group counts, reduction
    size and output size (N for GEMM2, I for GEMM1) from its seed."""
    rng = np.random.default_rng(1000 + seed)
    kind = seed % 3
    if kind == 0:
        E = int(rng.choice([8, 40, 96]))
        counts = rng.integers(0, 6, E)
    elif kind == 1:
        E = int(rng.choice([3, 8, 17]))
        counts = rng.choice([0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257], E)
    else:
        E = int(rng.choice([1, 3, 6]))
        counts = rng.integers(0, 700, E)
    counts = counts.astype(np.int64)
    while counts.sum() > MAX_ROWS:
        counts = counts // 2
    Kd = int(rng.choice([128, 256, 384, 512, 640, 768, 1024]))
    n = int(rng.choice(n_choices))
    return rng, counts, Kd, n


def mx_operands(rng, M, Kd, E, N):
    a = rng.standard_normal((M, Kd)) * np.exp2(rng.integers(-4, 4, (M, 1)))
    w = rng.standard_normal((E * N, Kd)) * 0.05 * np.exp2(rng.integers(-4, 4, (E * N, 1)))
    aq, as_ = mx_ref.mx_quantize_ref(a)
    wq, ws = mx_ref.mx_quantize_ref(w)
    return aq, as_, wq.reshape(E, N, Kd), ws.reshape(E, N, -1, 2)


def tile_rows(counts, Kd):
    """The token-tile height the library picks for these counts."""
    M, E = int(counts.sum()), len(counts)
    return 128 if Kd // 128 >= 3 and M <= 64 * E else 256


@pytest.mark.parametrize("seed", SEEDS)
def test_gmm_mx_sweep(seed):
    rng, counts, Kd, N = draw_case(seed, [256, 512, 768])
    M, E = int(counts.sum()), len(counts)
    gl_type = int(rng.integers(0, 2))
    say(f"gmm_mx sweep seed={seed} M={M} Kd={Kd} N={N} E={E} gl_type={gl_type} "
        f"tiles={tile_rows(counts, Kd)} stages={Kd // 128}")
    aq, as_, wq, ws = mx_operands(rng, M, Kd, E, N)
    gl = counts if gl_type == 1 else np.cumsum(counts)
    y = mx.gmm_mx(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(gl), gl_type)
    torch.cuda.synchronize()
    ref = moe_ref.gmm_mx_ref(aq, as_, wq, ws, gl, gl_type)
    err = bf16_rows_rel_err(bf16_host(y), ref) if M else np.zeros(1)
    say(f"  max row rel err {err.max():.3g}")
    assert err.max() <= TOL
    # the same weights tile-packed: the same bytes
    wp = mx.mx_pack_weights(u8_dev(wq), mx.PACK_GEMM2)
    yp = mx.gmm_mx_packed(u8_dev(aq), u8_dev(as_), wp, u8_dev(ws), i64_dev(gl), gl_type)
    torch.cuda.synchronize()
    assert torch.equal(yp, y)


@pytest.mark.parametrize("seed", SEEDS)
def test_gmm_swiglu_mxquant_sweep(seed):
    rng, counts, K, I = draw_case(seed, [128, 256, 384])
    M, E = int(counts.sum()), len(counts)
    say(f"gmm_swiglu_mxquant sweep seed={seed} M={M} K={K} I={I} E={E} "
        f"tiles={tile_rows(counts, K)} stages={K // 128}")
    aq, as_, wq, ws = mx_operands(rng, M, K, E, 2 * I)
    hq, hs, h = mx.gmm_swiglu_mxquant(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(counts), 1,
                                      h_debug=True)
    torch.cuda.synchronize()
    rq, rs, rh = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, wq, ws, counts, 1, I)
    hk = host(h)
    if M:
        herr = row_rel_err(hk, rh)
        say(f"  h max row rel err {herr.max():.3g}")
        assert herr.max() <= 1e-3
    # requant bytes exact given the kernel's own h; against the oracle's h
    # every differing byte explained by the requant rule
    kq, ks = mx_ref.mx_quantize_ref(hk.astype(np.float64))
    assert np.array_equal(host(hq), kq)
    assert np.array_equal(host(hs), ks)
    n_mis, n_bad = explain_hq_mismatches(host(hq), host(hs), rq, rh)
    say(f"  hq/hs mismatches vs oracle {n_mis} of {rq.size}, unexplained {n_bad}")
    assert n_bad == 0 and n_mis <= 0.01 * max(rq.size, 1)
    # the same weights tile-packed: the same bytes
    wp = mx.mx_pack_weights(u8_dev(wq), mx.PACK_GEMM1)
    hqp, hsp = mx.gmm_swiglu_mxquant_packed(u8_dev(aq), u8_dev(as_), wp, u8_dev(ws), i64_dev(counts), 1)
    torch.cuda.synchronize()
    assert torch.equal(hqp, hq) and torch.equal(hsp, hs)


def w4_operands(rng, M, Kd, E, N):
    a = rng.standard_normal((M, Kd)) * np.exp2(rng.integers(-4, 4, (M, 1)))
    w = rng.standard_normal((E * N, Kd)) * 0.05 * np.exp2(rng.integers(-4, 4, (E * N, 1)))
    aq, as_ = mx_ref.mx_quantize_ref(a)
    wq, ws = mx_ref.mxfp4_quantize_ref(w)
    return aq, as_, wq.reshape(E, N, Kd // 2), ws.reshape(E, N, -1, 2)


@pytest.mark.parametrize("seed", SEEDS)
def test_gmm_w4a8_sweep(seed):
    """Both GEMMs with MXFP4 (e2m1) weights on the GEMM sweep's drawn sizes."""
    rng, counts, Kd, N = draw_case(seed, [256, 512, 768])
    M, E = int(counts.sum()), len(counts)
    say(f"w4a8 GEMM sweep seed={seed} M={M} Kd={Kd} N={N} E={E} tiles={tile_rows(counts, Kd)}")
    aq, as_, wq, ws = w4_operands(rng, M, Kd, E, N)
    y = mx.gmm_mx_w4a8(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(counts), 1)
    torch.cuda.synchronize()
    ref = moe_ref.gmm_mx_ref(aq, as_, wq, ws, counts, 1, "e2m1")
    if M:
        err = bf16_rows_rel_err(bf16_host(y), ref)
        say(f"  GEMM2 max row rel err {err.max():.3g}")
        assert err.max() <= TOL
    I = N // 2 if (N // 2) % 128 == 0 else 128
    aq1, as1, wq1, ws1 = w4_operands(rng, M, Kd, E, 2 * I)
    hq, hs, h = mx.gmm_swiglu_mxquant_w4a8(u8_dev(aq1), u8_dev(as1), u8_dev(wq1), u8_dev(ws1), i64_dev(counts), 1,
                                           h_debug=True)
    torch.cuda.synchronize()
    rq, rs, rh = moe_ref.gmm_swiglu_mxquant_ref(aq1, as1, wq1, ws1, counts, 1, I, "e2m1")
    hk = host(h)
    if M:
        herr = row_rel_err(hk, rh)
        say(f"  GEMM1 h max row rel err {herr.max():.3g}")
        assert herr.max() <= 1e-3
    kq, ks = mx_ref.mx_quantize_ref(hk.astype(np.float64))
    assert np.array_equal(host(hq), kq) and np.array_equal(host(hs), ks)
    n_mis, n_bad = explain_hq_mismatches(host(hq), host(hs), rq, rh)
    assert n_bad == 0 and n_mis <= 0.01 * max(rq.size, 1)


def rand_bf16(rng, shape, spread):
    x = rng.standard_normal(shape) * np.exp2(rng.integers(-spread, spread + 1, shape[:-1] + (1,)))
    return to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("seed", SEEDS)
def test_route_quant_sweep(seed):
    rng = np.random.default_rng(2000 + seed)
    E = int(rng.choice([1, 5, 64, 128, 300, 1024]))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.choice([1, 7, 256 // k, 256 // k + 1, 1000, 4096, 9000]))
    K = int(rng.choice([32, 96, 256, 2048]))
    if T * K > 4096 * 2048:
        K = 256
    # skewed (a few hot experts) or uniform expert choice, distinct per token
    p = None
    if seed % 2:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = rng.permutation(p / p.sum())
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    say(f"moe_route_quant sweep seed={seed} T={T} K={K} k={k} E={E} {'skewed' if p is not None else 'uniform'}")
    x = rand_bf16(rng, (T, K), 8)
    xq, xs, sr, eri, gl = mx.moe_route_quant(bf16_dev(x), i32_dev(ids), E)
    torch.cuda.synchronize()
    rq, rs, rsr, reri, rc = moe_ref.route_quant_ref(x, ids, E)
    assert np.array_equal(host(gl), rc)
    assert np.array_equal(host(sr), rsr)
    assert np.array_equal(host(eri), reri)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs), rs)


@pytest.mark.parametrize("seed", SEEDS)
def test_finalize_sweep(seed):
    rng = np.random.default_rng(3000 + seed)
    T = int(rng.choice([1, 3, 64, 333, 2048]))
    K = int(rng.choice([8, 72, 512, 1024, 2056, 4096]))
    k = int(rng.choice([1, 2, 6, 8]))
    M = T * k
    say(f"moe_finalize sweep seed={seed} T={T} K={K} k={k}")
    y = rand_bf16(rng, (M, K), 6)
    w = rng.random((T, k)).astype(np.float32)
    eri = rng.permutation(M).astype(np.int32)
    drop = rng.random(M) < 0.02                    # dropped assignments (invalid ids upstream)
    eri[drop] = -1
    out = mx.moe_finalize(bf16_dev(y), f32_dev(w), i32_dev(eri))
    torch.cuda.synchronize()
    w_eff = np.where(drop.reshape(T, k), np.float32(0.0), w)
    ref = moe_ref.finalize_ref(y, w_eff, np.where(drop, 0, eri))
    assert np.array_equal(bf16_host(out), ref)


@pytest.mark.parametrize("seed", list(range(6)))
def test_forward_sweep(seed):
    rng = np.random.default_rng(4000 + seed)
    # the Zipf bias needs more than its 16 top experts; hot/cold routing
    # leaves two experts unchosen
    routing = ["plain", "zipf", "hot_cold"][seed % 3]
    E = int(rng.choice({"plain": [4, 16, 64, 128], "zipf": [64, 128], "hot_cold": [16, 64]}[routing]))
    k = min(int(rng.choice([1, 2, 4, 8])), E)
    T = int(rng.choice([1, 5, 33, 200, 700]))
    K = int(rng.choice([256, 512, 768]))
    I = int(rng.choice([128, 256, 384]))
    outliers = bool(rng.integers(0, 2))
    cfg = custom_config(f"sweep{seed}", T, K, I, E, k, routing=routing, outliers=outliers)
    d = make_inputs(cfg, seed=seed)
    say(f"moe_mxfp8_forward sweep seed={seed} T={T} K={K} I={I} E={E} k={k} routing={routing} outliers={outliers}")
    w13q, w13s = mx.mx_quantize(bf16_dev(d["w13"]))
    w2q, w2s = mx.mx_quantize(bf16_dev(d["w2"]))
    # the oracle quantiser over the worker pool (the same bytes as the serial
    # routine, pinned in test_oracle_pool.py)
    r13q, r13s = (a.reshape(E, 2 * I, *a.shape[1:]) for a in oracle_pool.quantize_bf16(d["w13"].reshape(-1, K)))
    r2q, r2s = (a.reshape(E, K, *a.shape[1:]) for a in oracle_pool.quantize_bf16(d["w2"].reshape(-1, I)))
    assert np.array_equal(host(w13q), r13q) and np.array_equal(host(w13s), r13s)
    assert np.array_equal(host(w2q), r2q) and np.array_equal(host(w2s), r2s)
    ws = mx.forward_workspace(T, K, I, E, k)
    out = mx.moe_mxfp8_forward(bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"]), w13q, w13s, w2q, w2s,
                               workspace=ws)
    torch.cuda.synchronize()
    inter = {n: host(v) for n, v in mx.forward_intermediates(ws, T, K, I, E, k).items() if n != "y"}
    inter["y"] = bf16_host(mx.forward_intermediates(ws, T, K, I, E, k)["y"])
    check_layer_every_row(d, bf16_host(out), inter, r13q, r13s, r2q, r2s, "e4m3", TOL, 5e-2)
    # the same layer on tile-packed weights: the same bytes
    wp13, wp2 = mx.mx_pack_weights(w13q, mx.PACK_GEMM1), mx.mx_pack_weights(w2q, mx.PACK_GEMM2)
    out_p = mx.moe_mxfp8_forward_packed(bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"]), wp13, w13s,
                                        wp2, w2s)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out)
    # the same layer with the weights quantised to MXFP4 (e2m1) instead
    del wp13, wp2, out_p
    f13q, f13s = mx.mx_quantize_fp4(bf16_dev(d["w13"]))
    f2q, f2s = mx.mx_quantize_fp4(bf16_dev(d["w2"]))
    g13q, g13s = oracle_pool.quantize_bf16(d["w13"].reshape(-1, K), fp4=True)
    g2q, g2s = oracle_pool.quantize_bf16(d["w2"].reshape(-1, I), fp4=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(f13q).reshape(g13q.shape), g13q) and np.array_equal(host(f13s).reshape(g13s.shape), g13s)
    assert np.array_equal(host(f2q).reshape(g2q.shape), g2q) and np.array_equal(host(f2s).reshape(g2s.shape), g2s)
    out4 = mx.moe_w4a8_forward(bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"]), f13q, f13s, f2q, f2s,
                               workspace=ws)
    torch.cuda.synchronize()
    inter4 = {n: host(v) for n, v in mx.forward_intermediates(ws, T, K, I, E, k).items() if n != "y"}
    inter4["y"] = bf16_host(mx.forward_intermediates(ws, T, K, I, E, k)["y"])
    check_layer_every_row(d, bf16_host(out4), inter4, g13q.reshape(E, 2 * I, K // 2), g13s.reshape(E, 2 * I, -1, 2),
                          g2q.reshape(E, K, I // 2), g2s.reshape(E, K, -1, 2), "e2m1", TOL, 5e-2)


@pytest.mark.parametrize("seed", SEEDS)
def test_linear_sweep(seed):
    rng = np.random.default_rng(6000 + seed)
    T = int(rng.choice([1, 17, 255, 256, 257, 1000]))
    K = int(rng.choice([128, 256, 384, 512, 1024]))
    N = int(rng.choice([256, 512, 768, 1024]))
    say(f"mx_linear sweep seed={seed} T={T} K={K} N={N}")
    x = rand_bf16(rng, (T, K), 4)
    w = to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wq, ws = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(w))
    y = mx.mx_linear(bf16_dev(x), u8_dev(wq), u8_dev(ws))
    torch.cuda.synchronize()
    xq, xs = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(x))
    ref = moe_ref.gmm_mx_ref(xq, xs, wq[None], ws[None], np.array([T], np.int64), 1)
    err = bf16_rows_rel_err(bf16_host(y), ref)
    say(f"  max row rel err {err.max():.3g}")
    assert err.max() <= TOL


@pytest.mark.parametrize("seed", SEEDS)
def test_router_sweep(seed):
    rng = np.random.default_rng(5000 + seed)
    E = int(rng.choice([2, 8, 33, 64, 65, 128, 200, 256]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([1, 63, 64, 65, 1000, 3000]))
    K = int(rng.choice([64, 192, 1024, 2048]))
    renorm = bool(rng.integers(0, 2))
    kind = seed % 3
    bias = None
    if kind >= 1:
        bias = rng.standard_normal(E) * 0.5
        if kind == 2:                       # some experts never chosen, at least k left
            bias[rng.choice(E, size=(E - k) // 2, replace=False)] = -np.inf
    say(f"moe_router sweep seed={seed} T={T} K={K} E={E} k={k} renormalize={renorm} "
        f"bias={['none', 'finite', 'with -inf'][kind]}")
    x = rand_bf16(rng, (T, K), 2)
    gate = to_bf16_bits((rng.standard_normal((E, K)) * 0.02).astype(np.float32))
    ids, w = run_router(x, gate, bias, k, renorm)
    near, werr = check_router(ids, w, x, gate, bias, k, renorm)
    say(f"  tokens with a near-tie at the k-th place {near}, weight rel err {werr:.3g}")
