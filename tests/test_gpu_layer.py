"""Whole-layer parity: moe_mxfp8_forward (the call the benchmark times)
against the CPU oracle.

Small layers and the four full-size workloads (in the benchmark's launch
configuration) are compared on every row of every stage: routing indices,
group counts, the activation payload and scales and the weights' load-time
quantisation bit-exact; GEMM1's requant bytes exact or explained by the
requant rule; GEMM2 on identical operands within 2e-2 per row; finalize
bit-exact; the end-to-end output within the end-to-end bar."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_topk_amd as mx
import oracle_pool
from gpu_util import (bf16_dev, bf16_host, bf16_rows_rel_err, check_layer_every_row, explain_hq_mismatches, f32_dev,
                      guard_alloc, guards_intact, host, i32_dev, quantize_experts_ref, say, u8_dev)
from oracle import moe_ref, mx_ref
from workloads import CONFIGS, custom_config, make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2        # bf16 outputs vs the oracle on identical dequantised operands
E2E_TOL = 5e-2    # output vs the fully independent oracle (GEMM1 requant flips propagate)


def _device_weights(d):
    """Quantised weights on the GPU: online workloads are quantised by the
    library's mx_quantize (load time); the offline one ships bytes."""
    if d["cfg"].offline:
        return [u8_dev(d[n]) for n in ("w13q", "w13s", "w2q", "w2s")]
    w13q, w13s = mx.mx_quantize(bf16_dev(d["w13"]))
    w2q, w2s = mx.mx_quantize(bf16_dev(d["w2"]))
    return [w13q, w13s, w2q, w2s]


def _run(d, wdev):
    cfg = d["cfg"]
    T, K, I, E, k = cfg.T, cfg.K, cfg.I, cfg.E, cfg.k
    ws = mx.forward_workspace(T, K, I, E, k)
    say(f"moe_mxfp8_forward {cfg.name} T={T} K={K} I={I} E={E} k={k}")
    out = mx.moe_mxfp8_forward(bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"]), *wdev,
                               workspace=ws)
    torch.cuda.synchronize()
    inter = {n: host(v) for n, v in mx.forward_intermediates(ws, T, K, I, E, k).items() if n != "y"}
    inter["y"] = bf16_host(mx.forward_intermediates(ws, T, K, I, E, k)["y"])
    return bf16_host(out), inter


def _check_routing_and_xq(d, inter):
    cfg = d["cfg"]
    counts, sr, eri = moe_ref.route_ref_fast(d["topk_ids"], cfg.E)
    assert np.array_equal(inter["group_list"], counts)
    assert np.array_equal(inter["sorted_row"], sr)
    assert np.array_equal(inter["expanded_row_idx"], eri)
    qt, st = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(d["x"]))
    tok = sr.astype(np.int64) // cfg.k
    assert np.array_equal(inter["xq"], qt[tok])
    assert np.array_equal(inter["xs"], st[tok])
    return qt, st, eri


@pytest.mark.parametrize("shape", [
    ("tiny", None),
    ("several-tiles", (300, 512, 256, 12, 4)),
    ("sparse-experts", (129, 256, 128, 70, 3)),
    ("k1-ragged", (333, 256, 128, 3, 1)),
    # decode-sized: one row per expert on average (GEMM1 on 128-row tiles)
    ("decode-small", (16, 512, 256, 64, 4)),
    ("decode-i384", (8, 768, 384, 32, 8)),
])
def test_forward_small_full_compare(shape):
    name, dims = shape
    cfg = CONFIGS["tiny"] if dims is None else custom_config(name, *dims)
    d = make_inputs(cfg)
    wdev = _device_weights(d)
    out, inter = _run(d, wdev)
    _check_routing_and_xq(d, inter)
    w13q, w13s = quantize_experts_ref(d["w13"])
    w2q, w2s = quantize_experts_ref(d["w2"])
    assert np.array_equal(host(wdev[0]), w13q) and np.array_equal(host(wdev[1]), w13s)
    assert np.array_equal(host(wdev[2]), w2q) and np.array_equal(host(wdev[3]), w2s)
    ref = moe_ref.moe_forward_ref(d["x"], d["topk_ids"], d["topk_w"], w13q, w13s, w2q, w2s)
    n_mis, n_bad = explain_hq_mismatches(inter["hq"], inter["hs"], ref["hq"], ref["h"])
    say(f"  {cfg.name}: hq/hs mismatches {n_mis} of {ref['hq'].size} bytes, unexplained {n_bad}")
    assert n_bad == 0 and n_mis <= 0.01 * ref["hq"].size
    # GEMM2 against the oracle on identical dequantised operands (the GPU's hq/hs)
    y_same = moe_ref.gmm_mx_ref(inter["hq"], inter["hs"], w2q, w2s, inter["group_list"], 1)
    yerr = bf16_rows_rel_err(inter["y"], y_same)
    # finalize is exact given the same y
    assert np.array_equal(out, moe_ref.finalize_ref(inter["y"], d["topk_w"], inter["expanded_row_idx"]))
    e2e = bf16_rows_rel_err(out, ref["out"])
    say(f"  y max row rel err {yerr.max():.3g} (same operands); end-to-end out {e2e.max():.3g}")
    assert yerr.max() <= TOL
    assert e2e.max() <= E2E_TOL


def _weights_every_expert(d, wdev):
    """Online workloads: the GPU's load-time quantisation of every expert's
    w13 and w2 equals the oracle's, byte for byte.  Returns the oracle's
    bytes (offline: the shipped bytes), shaped [E, N, Kd] / [E, N, Kd/64, 2]."""
    cfg = d["cfg"]
    E, K, I = cfg.E, cfg.K, cfg.I
    if cfg.offline:
        return d["w13q"], d["w13s"], d["w2q"], d["w2s"]
    w13q, w13s = oracle_pool.quantize_bf16(d["w13"].reshape(E * 2 * I, K))
    w2q, w2s = oracle_pool.quantize_bf16(d["w2"].reshape(E * K, I))
    assert np.array_equal(host(wdev[0]).reshape(w13q.shape), w13q)
    assert np.array_equal(host(wdev[1]).reshape(w13s.shape), w13s)
    assert np.array_equal(host(wdev[2]).reshape(w2q.shape), w2q)
    assert np.array_equal(host(wdev[3]).reshape(w2s.shape), w2s)
    return (w13q.reshape(E, 2 * I, K), w13s.reshape(E, 2 * I, -1, 2), w2q.reshape(E, K, I),
            w2s.reshape(E, K, -1, 2))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "mid", "prefill", "wide"])
def test_forward_full_size_every_row(name):
    """The four full-size workloads in the benchmark's launch configuration,
    every row of every stage against the oracle (see check_layer_every_row),
    with guard bands around the output and the workspace."""
    cfg = CONFIGS[name]
    say(f"generating {name}")
    d = make_inputs(cfg)
    wdev = _device_weights(d)
    T, K, I, E, k = cfg.T, cfg.K, cfg.I, cfg.E, cfg.k
    need = mx.forward_workspace_size(T, K, I, E, k)
    raw_ws, ws = guard_alloc(need, torch.uint8, fill=0x3C)
    raw_out, out = guard_alloc(T * K, torch.bfloat16, fill=0x6B)
    say(f"moe_mxfp8_forward {name} T={T} K={K} I={I} E={E} k={k}")
    mx.moe_mxfp8_forward(bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"]), *wdev,
                         out=out.view(T, K), workspace=ws)
    torch.cuda.synchronize()
    assert guards_intact(raw_ws, need, fill=0x3C) and guards_intact(raw_out, T * K * 2, fill=0x6B)
    inter = {n: host(v) for n, v in mx.forward_intermediates(ws, T, K, I, E, k).items() if n != "y"}
    inter["y"] = bf16_host(mx.forward_intermediates(ws, T, K, I, E, k)["y"])
    out_h = bf16_host(out.view(T, K))
    say(f"  {name}: oracle weight quantisation, every expert")
    w13q, w13s, w2q, w2s = _weights_every_expert(d, wdev)
    del wdev
    check_layer_every_row(d, out_h, inter, w13q, w13s, w2q, w2s, "e4m3", TOL, E2E_TOL)


def test_forward_deterministic_and_stream_ordered():
    d = make_inputs(custom_config("det", 777, 256, 256, 16, 6))
    wdev = _device_weights(d)
    out1, inter1 = _run(d, wdev)
    out2, inter2 = _run(d, wdev)
    assert np.array_equal(out1, out2)
    for n in inter1:
        assert np.array_equal(inter1[n], inter2[n]), n
    # same result on a side stream made current
    s = torch.cuda.Stream()
    cfg = d["cfg"]
    with torch.cuda.stream(s):
        ws = mx.forward_workspace(cfg.T, cfg.K, cfg.I, cfg.E, cfg.k)
        say("moe_mxfp8_forward on a side stream")
        o = mx.moe_mxfp8_forward(bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"]), *wdev,
                                 workspace=ws)
    s.synchronize()
    assert np.array_equal(bf16_host(o), out1)


def test_explicit_stream_argument():
    """stream= names a stream that is not torch's current one: the binding's
    own allocations (outputs, workspaces) must belong to that stream, so
    work queued meanwhile on the current stream cannot be given the same
    memory while the kernels still use it."""
    d = make_inputs(custom_config("side", 513, 512, 256, 16, 8))
    cfg = d["cfg"]
    wdev = _device_weights(d)
    ref, inter = _run(d, wdev)
    x, ids, w = bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    say("layer and stand-alone entry points with stream= a side stream")
    # keep the current stream busy allocating and writing while the side stream runs
    outs = []
    for _ in range(3):
        o = mx.moe_mxfp8_forward(x, ids, w, *wdev, stream=s)
        junk = [torch.full((1 << 20,), 7, dtype=torch.uint8, device="cuda") for _ in range(8)]
        outs.append(o)
        del junk
    xq, xs, sr, eri, gl = mx.moe_route_quant(x, ids, cfg.E, stream=s)
    hq, hs = mx.gmm_swiglu_mxquant(xq, xs, wdev[0], wdev[1], gl, stream=s)
    y = mx.gmm_mx(hq, hs, wdev[2], wdev[3], gl, stream=s)
    o2 = mx.moe_finalize(y, w, eri, stream=s)
    s.synchronize()
    for o in outs + [o2]:
        assert np.array_equal(bf16_host(o), ref)
    assert np.array_equal(host(xq), inter["xq"]) and np.array_equal(host(hq), inter["hq"])


def test_forward_graph_replays():
    """The whole layer captured in a HIP graph and replayed on three new
    inputs (new tokens, routing and weights copied into the captured
    buffers), with eager forwards and synchronisations between replays:
    every replay equals the eager forward on the same inputs, bit for bit."""
    cfg = custom_config("graph", 513, 512, 256, 16, 8)
    T, K, I, E, k = cfg.T, cfg.K, cfg.I, cfg.E, cfg.k
    sets = [make_inputs(custom_config(f"graph{i}", T, K, I, E, k), seed=20 + i) for i in range(4)]
    wdev = _device_weights(sets[0])
    x, ids, w = bf16_dev(sets[0]["x"]), i32_dev(sets[0]["topk_ids"]), f32_dev(sets[0]["topk_w"])
    ws = mx.forward_workspace(T, K, I, E, k)
    out = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        mx.moe_mxfp8_forward(x, ids, w, *wdev, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mx.moe_mxfp8_forward(x, ids, w, *wdev, out=out, workspace=ws)
    for i in (1, 2, 3):
        d = sets[i]
        x.copy_(bf16_dev(d["x"]))
        ids.copy_(i32_dev(d["topk_ids"]))
        w.copy_(f32_dev(d["topk_w"]))
        say(f"moe_mxfp8_forward graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        got = bf16_host(out)
        eager_ws = mx.forward_workspace(T, K, I, E, k)
        eager = mx.moe_mxfp8_forward(bf16_dev(d["x"]), i32_dev(d["topk_ids"]), f32_dev(d["topk_w"]), *wdev,
                                     workspace=eager_ws)
        torch.cuda.synchronize()
        assert np.array_equal(got, bf16_host(eager)), i
