"""Dense MXFP8 linear (mx_linear) against the oracle: the oracle's MX
quantisation of x followed by its MX GEMM with one group (the dense case the
oracle pins against a direct float64 product).  Every row, small shapes and
the benchmark's 16384 x 4096 x 4096 shape."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_topk_amd as mx
import oracle_pool
from gpu_util import (bf16_dev, bf16_host, bf16_rows_rel_err, bf16_rows_rel_err_chunked, guard_alloc, guards_intact,
                      say, u8_dev)
from oracle import moe_ref, mx_ref
from workloads import dense_linear_inputs, normal_bf16, rng_for

pytestmark = pytest.mark.gpu

TOL = 2e-2


def oracle_rows(x_bits, wq, ws, rows):
    xq, xs = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(x_bits[rows]))
    return moe_ref.gmm_mx_ref(xq, xs, wq[None], ws[None], np.array([len(rows)], np.int64), 1)


@pytest.mark.parametrize("T,K,N,offline", [
    (1, 128, 256, False),
    (300, 384, 512, False),       # ragged m-tiles, 3 k stages
    (257, 256, 768, True),        # offline-style weight bytes
])
def test_linear_small(T, K, N, offline):
    if offline:
        x, wq, ws = dense_linear_inputs(T, K, N, seed=3)
    else:
        x = normal_bf16(rng_for(1, "x"), (T, K), 1.0)
        w = normal_bf16(rng_for(1, "w13"), (N, K), 0.02)
        wq, ws = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(w))
    say(f"mx_linear T={T} K={K} N={N} offline={offline}")
    y = mx.mx_linear(bf16_dev(x), u8_dev(wq), u8_dev(ws))
    torch.cuda.synchronize()
    ref = oracle_rows(x, wq, ws, np.arange(T))
    err = bf16_rows_rel_err(bf16_host(y), ref)
    say(f"mx_linear T={T}: max row rel err {err.max():.2e}")
    assert err.max() <= TOL


@pytest.mark.timeout(900)
def test_linear_large_every_row():
    """The benchmark's dense shape, every row, with guard bands around y."""
    T, K, N = 16384, 4096, 4096
    x, wq, ws = dense_linear_inputs(T, K, N)
    raw, y = guard_alloc(T * N, torch.bfloat16, fill=0x4D)
    say(f"mx_linear T={T} K={K} N={N}")
    mx.mx_linear(bf16_dev(x), u8_dev(wq), u8_dev(ws), out=y.view(T, N))
    torch.cuda.synchronize()
    assert guards_intact(raw, T * N * 2, fill=0x4D)
    xq, xs = oracle_pool.quantize_bf16(x)
    ref = oracle_pool.gemm2_y(xq, xs, wq[None], ws[None], np.array([T], np.int64), 1)
    err = bf16_rows_rel_err_chunked(bf16_host(y.view(T, N)), ref)
    say(f"mx_linear large: max row rel err {err.max():.2e} over {T} rows")
    assert err.max() <= TOL


def test_linear_empty():
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    y = mx.mx_linear(x, torch.zeros((256, 128), dtype=torch.uint8, device="cuda"),
                     torch.zeros((256, 2, 2), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (0, 256)
