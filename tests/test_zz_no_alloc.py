"""moe_route_quant_noalloc (routing scratch in the library's own device
array, no workspace) against moe_route_quant (caller workspace), through
the C ABI: all five outputs byte for byte, on consecutive calls whose sizes
shrink, so the second call runs over the scratch the first one left."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_topk_amd as mx
from gpu_util import bf16_dev, host, i32_dev, say
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(T, K, k, E, seed):
    rng = np.random.default_rng(seed)
    x = to_bf16_bits((rng.standard_normal((T, K)) * np.exp2(rng.integers(-8, 8, (T, 1)))).astype(np.float32))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    return bf16_dev(x), i32_dev(ids)


def _filled_outputs(T, K, k, E):
    M = T * k
    dev = "cuda"
    return (torch.full((M, K), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((M, K // 64, 2), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((M,), -7, dtype=torch.int32, device=dev),
            torch.full((M,), -7, dtype=torch.int32, device=dev),
            torch.full((E,), -7, dtype=torch.int64, device=dev))


@pytest.mark.parametrize("sizes", [
    # (T, K, k, E): many routing chunks, then fewer chunks and experts, then
    # one chunk (no scratch use), then many chunks again
    [(2049, 512, 8, 128), (301, 256, 4, 16), (20, 128, 8, 64), (777, 256, 6, 40)],
])
def test_noalloc_matches_workspace_entry_point(sizes):
    for i, (T, K, k, E) in enumerate(sizes):
        x, ids = _inputs(T, K, k, E, seed=100 + i)
        say(f"moe_route_quant_noalloc call {i}: T={T} K={K} k={k} E={E}")
        got = mx.moe_route_quant_noalloc(x, ids, E, out=_filled_outputs(T, K, k, E))
        ref = mx.moe_route_quant(x, ids, E)
        torch.cuda.synchronize()
        for name, r, g in zip(("xq", "xs", "sorted_row", "expanded_row_idx", "group_list"), ref, got):
            assert np.array_equal(host(r), host(g)), (i, name)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    # E = 1024, top-8: 32 tokens per routing chunk, 4 KB of counts per chunk,
    # plus the super-chunk offsets and flags: past 31712 tokens the scratch
    # needs more than the 4 MiB the library holds
    T, K, k, E = 31713, 32, 8, 1024
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    with pytest.raises(mx.MxError, match="routing scratch"):
        mx.moe_route_quant_noalloc(x, ids, E)
    # the largest batch that fits
    T = 31712
    x, ids = _inputs(T, K, k, E, seed=7)
    say(f"moe_route_quant_noalloc at its limit: T={T} k={k} E={E}")
    got = mx.moe_route_quant_noalloc(x, ids, E)
    ref = mx.moe_route_quant(x, ids, E)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert np.array_equal(host(r), host(g))


def test_noalloc_graph_replays():
    """Captured in a HIP graph (the callers this entry point is for), replayed
    on new inputs: every replay routes its own inputs."""
    from test_gpu_kernels import route_graph_replays
    E = 64
    route_graph_replays(lambda x, ids, outs: mx.moe_route_quant_noalloc(x, ids, E, out=outs), E=E, seed=11)
