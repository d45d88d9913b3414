"""Tile-packed expert weights (mx_pack_weights and the *_packed GEMMs and
layer) on the GPU: the pack against the layout's definition written out
here with NumPy, and the packed GEMMs and layer against the row-major
entry points (identical bytes: the same MFMAs in the same order on the same
operands) and against the oracle, with the same bars as the row-major path."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_topk_amd as mx
from gpu_util import (bf16_dev, bf16_host, bf16_rows_rel_err, check_layer_every_row, explain_hq_mismatches,
                      f32_dev, guard_alloc, guards_intact, host, i32_dev, i64_dev, row_rel_err, say, u8_dev)
from oracle import moe_ref, mx_ref
from workloads import CONFIGS, custom_config, make_inputs

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(77)
TOL = 2e-2
E2E_TOL = 5e-2


def pack_by_definition(w, kind):
    """The tile-packed layout of include/mxmoe.h, element by element: block
    (e, nt, ks) holds 256 rows of 128 bytes, chunk c of block row r stored at
    position c ^ ((r // 2) % 8); block row r is weight row 256 nt + r (kind 0),
    or for kind 1 gate row 128 nt + 64 h + (r % 64) when r % 128 < 64 and up
    row I + 128 nt + 64 h + (r % 64) otherwise, h = r // 128."""
    E, N, Kd = w.shape
    nk, NT, I = Kd // 128, N // 256, N // 2
    out = np.empty((E, NT, nk, 256, 8, 16), np.uint8)
    for nt in range(NT):
        for r in range(256):
            if kind == 0:
                n = 256 * nt + r
            else:
                h, rr = r // 128, r % 128
                n = (0 if rr < 64 else I) + 128 * nt + 64 * h + rr % 64
            row = w[:, n, :].reshape(E, nk, 8, 16)
            for c in range(8):
                out[:, nt, :, r, c ^ ((r // 2) % 8), :] = row[:, :, c, :]
    return out.reshape(E, N, Kd)


@pytest.mark.parametrize("E,N,Kd,kind", [(3, 512, 384, 0), (2, 256, 1024, 1), (4, 768, 256, 1), (1, 256, 128, 0)])
def test_pack_matches_the_layout_definition(E, N, Kd, kind):
    w = RNG.integers(0, 256, size=(E, N, Kd), dtype=np.uint8)
    raw, out = guard_alloc(E * N * Kd, torch.uint8, fill=0x39)
    say(f"mx_pack_weights E={E} N={N} Kd={Kd} kind={kind}")
    mx.mx_pack_weights(u8_dev(w), kind, out=out.view(E, N, Kd))
    torch.cuda.synchronize()
    assert guards_intact(raw, E * N * Kd, fill=0x39)
    assert np.array_equal(host(out).reshape(E, N, Kd), pack_by_definition(w, kind))


def _operands(counts, Kd, N):
    E = len(counts)
    M = int(sum(counts))
    a = RNG.standard_normal((M, Kd)) * np.exp2(RNG.integers(-4, 4, (M, 1)))
    w = RNG.standard_normal((E * N, Kd)) * 0.05 * np.exp2(RNG.integers(-4, 4, (E * N, 1)))
    aq, as_ = mx_ref.mx_quantize_ref(a)
    wq, ws = mx_ref.mx_quantize_ref(w)
    return np.array(counts, np.int64), aq, as_, wq.reshape(E, N, Kd), ws.reshape(E, N, -1, 2)


# 256-row tiles with 4-stage scale groups, 256-row tiles with per-stage scales,
# and the 128-row three-slot tiles (few rows per expert)
CASES = {
    "ragged-256": ([0, 1, 127, 300, 257, 0, 5, 600], 512, 256),
    "per-stage-scales": ([70, 150, 400], 384, 512),
    "small-tiles": ([16, 17, 31, 0, 33, 2, 1] + [0] * 3, 768, 256),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gmm_mx_packed(name):
    counts, Kd, N = CASES[name]
    counts, aq, as_, wq, ws = _operands(counts, Kd, N)
    say(f"gmm_mx_packed {name} M={counts.sum()} N={N} Kd={Kd} E={len(counts)}")
    wd = u8_dev(wq)
    wp = mx.mx_pack_weights(wd, mx.PACK_GEMM2)
    y = mx.gmm_mx_packed(u8_dev(aq), u8_dev(as_), wp, u8_dev(ws), i64_dev(counts), 1)
    y0 = mx.gmm_mx(u8_dev(aq), u8_dev(as_), wd, u8_dev(ws), i64_dev(counts), 1)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(y), bf16_host(y0))
    ref = moe_ref.gmm_mx_ref(aq, as_, wq, ws, counts, 1)
    assert bf16_rows_rel_err(bf16_host(y), ref).max() <= TOL


@pytest.mark.parametrize("name", list(CASES))
def test_gmm_swiglu_mxquant_packed(name):
    counts, K, N = CASES[name]
    I = N // 2 if N >= 256 else 128
    counts, aq, as_, wq, ws = _operands(counts, K, 2 * I)
    say(f"gmm_swiglu_mxquant_packed {name} M={counts.sum()} K={K} I={I} E={len(counts)}")
    wd = u8_dev(wq)
    wp = mx.mx_pack_weights(wd, mx.PACK_GEMM1)
    hq, hs, h = mx.gmm_swiglu_mxquant_packed(u8_dev(aq), u8_dev(as_), wp, u8_dev(ws), i64_dev(counts), 1,
                                             h_debug=True)
    hq0, hs0 = mx.gmm_swiglu_mxquant(u8_dev(aq), u8_dev(as_), wd, u8_dev(ws), i64_dev(counts), 1)
    torch.cuda.synchronize()
    assert np.array_equal(host(hq), host(hq0)) and np.array_equal(host(hs), host(hs0))
    rq, rs, rh = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, wq, ws, counts, 1, I)
    assert row_rel_err(host(h), rh).max() <= 1e-3
    n_mis, n_bad = explain_hq_mismatches(host(hq), host(hs), rq, rh)
    assert n_bad == 0 and n_mis <= 0.01 * rq.size


def _packed_layer(d, wdev):
    cfg = d["cfg"]
    T, K, I, E, k = cfg.T, cfg.K, cfg.I, cfg.E, cfg.k
    w13p = mx.mx_pack_weights(wdev[0], mx.PACK_GEMM1)
    w2p = mx.mx_pack_weights(wdev[2], mx.PACK_GEMM2)
    ws = mx.forward_workspace(T, K, I, E, k)
    x, ids, w = bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"])
    say(f"moe_mxfp8_forward_packed {cfg.name} T={T} K={K} I={I} E={E} k={k}")
    out = mx.moe_mxfp8_forward_packed(x, ids, w, w13p, wdev[1], w2p, wdev[3], workspace=ws)
    torch.cuda.synchronize()
    inter = {n: host(v) for n, v in mx.forward_intermediates(ws, T, K, I, E, k).items() if n != "y"}
    inter["y"] = bf16_host(mx.forward_intermediates(ws, T, K, I, E, k)["y"])
    out0 = mx.moe_mxfp8_forward(x, ids, w, *wdev)
    torch.cuda.synchronize()
    return bf16_host(out), inter, bf16_host(out0)


@pytest.mark.parametrize("name", ["decode", "mid"])
def test_forward_packed_equals_row_major(name):
    """decode (128-row tiles) and mid at full size: the packed layer gives the
    row-major layer's bytes exactly."""
    d = make_inputs(CONFIGS[name])
    w13q, w13s = mx.mx_quantize(bf16_dev(d["w13"]))
    w2q, w2s = mx.mx_quantize(bf16_dev(d["w2"]))
    out, _, out0 = _packed_layer(d, [w13q, w13s, w2q, w2s])
    assert np.array_equal(out, out0)


@pytest.mark.timeout(900)
def test_forward_packed_prefill_every_row():
    """The 16K prefill layer with packed weights: every row of every stage
    against the oracle, and the row-major layer's output exactly."""
    d = make_inputs(CONFIGS["prefill"])
    wdev = [u8_dev(d[n]) for n in ("w13q", "w13s", "w2q", "w2s")]
    out, inter, out0 = _packed_layer(d, wdev)
    assert np.array_equal(out, out0)
    del wdev
    check_layer_every_row(d, out, inter, d["w13q"], d["w13s"], d["w2q"], d["w2s"], "e4m3", TOL, E2E_TOL)
