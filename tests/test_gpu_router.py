"""GPU router (moe_router) against the router oracle (reading R28).

The kernel sums the bf16 products in float32, the oracle in float64, so the
two may order two experts differently only when their logits lie within
the float32 accumulation error of each other.  The comparison therefore
checks, per token and output position j, that the expert the GPU put there
has an oracle logit within that error of the oracle's j-th largest logit
(which makes the selected set and its order equal wherever no near-tie
decides them), that the ids are distinct and in range, that the sets agree
exactly wherever the oracle's k-th and (k+1)-th logits are further apart than
twice the error, and that each weight equals the softmax probability (fp64,
from the oracle's logits, renormalised over the GPU's own selection) within
the error that the logit error allows."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_topk_amd as mx
from gpu_util import bf16_dev, check_router, f32_dev, host, run_router, say
from workloads import CONFIGS, custom_config, make_x, router_inputs, to_bf16_bits

pytestmark = pytest.mark.gpu

@pytest.mark.parametrize("name", ["tiny", "decode", "mid", "prefill", "wide"])
def test_router_workloads(name):
    cfg = CONFIGS[name]
    x = make_x(cfg)
    gate, bias, _ = router_inputs(cfg, x)
    say(f"moe_router {name} T={cfg.T} K={cfg.K} E={cfg.E} k={cfg.k}")
    ids, w = run_router(x, gate, bias, cfg.k)
    near, werr = check_router(ids, w, x, gate, bias, cfg.k, True)
    say(f"moe_router {name}: {near} near-tie tokens, max weight rel err {werr:.2e}")


@pytest.mark.parametrize("T,K,E,k,renorm", [
    (1, 64, 8, 1, True),          # one token, one chunk
    (65, 128, 40, 3, False),      # ragged token tile, E not a multiple of 32, plain softmax
    (100, 192, 96, 96, True),     # k = E, odd number of k chunks
    (130, 256, 256, 8, True),     # E at the limit
    (64, 320, 33, 5, False),
])
def test_router_shapes(T, K, E, k, renorm):
    cfg = custom_config(f"router{T}", T, K, 128, E, k)
    x = make_x(cfg)
    rng = np.random.default_rng(T + E)
    gate = to_bf16_bits((0.02 * rng.standard_normal((E, K))).astype(np.float32))
    bias = rng.standard_normal(E) if E % 2 else None
    say(f"moe_router shape T={T} K={K} E={E} k={k} renorm={renorm}")
    ids, w = run_router(x, gate, bias, k, renorm)
    check_router(ids, w, x, gate, bias, k, renorm)


def test_router_ties_and_minus_inf():
    """Equal logits pick lower ids first; -inf bias experts are never picked."""
    T, K, E, k = 96, 64, 16, 4
    x = to_bf16_bits(np.random.default_rng(7).standard_normal((T, K)).astype(np.float32))
    gate = to_bf16_bits(np.zeros((E, K), np.float32))       # all logits = bias
    bias = np.zeros(E)
    bias[[0, 5]] = -np.inf
    bias[[9, 12]] = 1.0
    say("moe_router ties / -inf")
    ids, w = run_router(x, gate, bias, k, True)
    assert (ids == np.array([9, 12, 1, 2])[None, :]).all()
    check_router(ids, w, x, gate, bias, k, True)


def test_router_empty_and_feeds_the_layer():
    """T = 0 is a no-op; the router's output drives moe_route_quant."""
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    say("moe_router T=0")
    ids, w = mx.moe_router(x, g, 2)
    torch.cuda.synchronize()
    assert ids.shape == (0, 2) and w.shape == (0, 2)
    cfg = CONFIGS["tiny"]
    xb = make_x(cfg)
    gate, bias, _ = router_inputs(cfg, xb)
    say("moe_router -> moe_route_quant")
    ids, w = mx.moe_router(bf16_dev(xb), bf16_dev(gate), cfg.k)
    xq, xs, sr, eri, gl = mx.moe_route_quant(bf16_dev(xb), ids, cfg.E)
    torch.cuda.synchronize()
    assert int(host(gl).sum()) == cfg.T * cfg.k


def test_router_guard_bands():
    """topk_ids and topk_w sit between 4 KB guard bands (ragged token count,
    a k that does not divide the wave); the bands stay intact."""
    from gpu_util import guard_alloc, guards_intact
    rng = np.random.default_rng(8)
    T, K, E, k = 1001, 512, 96, 6
    x = to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    gate = to_bf16_bits((rng.standard_normal((E, K)) * 0.02).astype(np.float32))
    raw_i, ids = guard_alloc(T * k, torch.int32, fill=0x2D)
    raw_w, w = guard_alloc(T * k, torch.float32, fill=0x4E)
    say(f"moe_router guard bands T={T} K={K} E={E} k={k}")
    mx.moe_router(bf16_dev(x), bf16_dev(gate), k, out=(ids.view(T, k), w.view(T, k)))
    torch.cuda.synchronize()
    assert guards_intact(raw_i, T * k * 4, fill=0x2D) and guards_intact(raw_w, T * k * 4, fill=0x4E)
    check_router(host(ids.view(T, k)), host(w.view(T, k)), x, gate, None, k, True)
