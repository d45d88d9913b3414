"""Per-kernel parity of the HIP path against the CPU oracle, through the C ABI.

Bars: bit-exact for quantised bytes, scales and routing indices; bf16
outputs within a per-row max relative error of 2e-2; GEMM1's h within 1e-3
and its requant bytes bit-exact given the kernel's own h.
"""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_topk_amd as mx
from gpu_util import (bf16_dev, bf16_host, bf16_rows_rel_err, explain_hq_mismatches, f32_dev, guard_alloc,
                      guards_intact, host, i32_dev, i64_dev, row_rel_err, say, u8_dev)
from oracle import moe_ref, mx_ref
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(2024)
TOL = 2e-2


def _rand_bf16(shape, scale_spread=0):
    x = RNG.standard_normal(shape).astype(np.float32)
    if scale_spread:
        x *= np.exp2(RNG.integers(-scale_spread, scale_spread, shape[:-1] + (1,))).astype(np.float32)
    return to_bf16_bits(x)


def _adversarial_rows():
    """Blocks of 32 built to hit every branch of the quantiser."""
    rows = []
    z = np.zeros(32, np.float32)
    rows.append(z)                                            # all zero
    rows.append(-z)                                           # all -0
    rows.append(np.full(32, 1e-40, np.float32))               # subnormal block
    t = np.zeros(32, np.float32); t[0] = 256.0                # s = 0, exact ties below
    t[1:9] = [1.0625, 1.1875, -1.0625, 2.125, 0.0029296875, -0.0029296875, 448.0, 464.0]
    rows.append(t)
    sat = np.full(32, 1.0, np.float32); sat[0] = 1.99; sat[1] = -1.99   # top element saturates
    rows.append(sat)
    rows.append(np.full(32, 3.0e38, np.float32))              # largest scale
    tiny = np.full(32, 2.0 ** -126, np.float32); tiny[3] = -(2.0 ** -120)
    rows.append(tiny)
    mixed = (RNG.standard_normal(32) * np.exp2(RNG.integers(-40, 40, 32))).astype(np.float32)
    rows.append(mixed)
    return to_bf16_bits(np.concatenate(rows).reshape(1, -1))


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    bits = b[np.isfinite(f)].astype(np.uint16)
    RNG.shuffle(bits)
    n = (bits.size // 64) * 64
    return bits[:n].reshape(-1, 64)


@pytest.mark.parametrize("shape", [(1, 32), (7, 64), (33, 2048), (5, 4304), (3, 40), (130, 768), (2, 8),
                                   (9, 4128), (4, 2080)])
def test_mx_quantize_bitexact(shape):
    say(f"mx_quantize shape={shape}")
    x = _rand_bf16(shape, scale_spread=30)
    q, s = mx.mx_quantize(bf16_dev(x))
    torch.cuda.synchronize()
    qr, sr = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(x))
    assert np.array_equal(host(q), qr)
    assert np.array_equal(host(s), sr)


def test_mx_quantize_adversarial_and_all_bf16():
    for name, x in [("adversarial", _adversarial_rows()), ("all-bf16", _all_finite_bf16())]:
        say(f"mx_quantize {name} {x.shape}")
        q, s = mx.mx_quantize(bf16_dev(x))
        torch.cuda.synchronize()
        qr, sr = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(x))
        assert np.array_equal(host(q), qr), name
        assert np.array_equal(host(s), sr), name


def test_mx_quantize_strided_rows_and_3d():
    say("mx_quantize strided rows")
    wide = _rand_bf16((9, 512), scale_spread=8)
    xd = bf16_dev(wide)[:, 128:384]                     # row stride 512, 256 columns
    q, s = mx.mx_quantize(xd)
    torch.cuda.synchronize()
    qr, sr = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(wide[:, 128:384]))
    assert np.array_equal(host(q), qr) and np.array_equal(host(s), sr)
    say("mx_quantize 3-D expert weights")
    w = _rand_bf16((3, 64, 256))
    q, s = mx.mx_quantize(bf16_dev(w))
    torch.cuda.synchronize()
    qr, sr = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(w.reshape(-1, 256)))
    assert q.shape == (3, 64, 256) and s.shape == (3, 64, 4, 2)
    assert np.array_equal(host(q).reshape(-1, 256), qr) and np.array_equal(host(s).reshape(-1, 4, 2), sr)


def test_mx_quantize_guard_bands():
    say("mx_quantize guard bands")
    x = _rand_bf16((17, 96))
    rawq, q = guard_alloc(17 * 96, torch.uint8)
    raws, s = guard_alloc(17 * 2 * 2, torch.uint8)
    mx.mx_quantize(bf16_dev(x), q=q.view(17, 96), s=s.view(17, 2, 2))
    torch.cuda.synchronize()
    assert guards_intact(rawq, 17 * 96) and guards_intact(raws, 17 * 4)
    qr, sr = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(x))
    assert np.array_equal(host(q).reshape(17, 96), qr) and np.array_equal(host(s).reshape(17, 2, 2), sr)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def _distinct_ids(T, k, E, p=None):
    return np.stack([RNG.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


ROUTE_CASES = {
    "small": (40, 256, 4, 12, None),
    "ragged-many-chunks": (301, 512, 8, 64, None),
    "k1": (257, 128, 1, 5, None),
    "one-hot-expert": (200, 256, 4, 16, "hot"),
    "sparse-experts": (100, 96, 2, 128, "sparse"),
    "E1": (33, 64, 1, 1, None),
    "k-eq-E": (50, 64, 6, 6, None),
    "big-k": (70, 64, 32, 40, None),
    # T*k <= 256 is one routing chunk (no leader workgroups): the boundary on
    # both sides, and the largest expert count in one chunk
    "one-chunk-full": (32, 256, 8, 128, None),
    "two-chunks-min": (33, 256, 8, 128, None),
    "one-chunk-E1024": (16, 64, 8, 1024, None),
    "one-chunk-hot": (60, 128, 4, 9, "hot"),
    # leaders owning several chunks each (157 chunks over 32 leaders), in
    # batches of 3 chunks (E = 1024 fills the LDS counts); 79 chunks of 256
    # single-expert assignments, the last one ragged
    "leader-batches-E1024": (5000, 64, 8, 1024, None),
    "leaders-k1": (20000, 32, 1, 7, None),
}


def _route_ids(T, k, E, kind):
    if kind == "hot":
        ids = _distinct_ids(T, k - 1, E - 1) + 1
        return np.concatenate([np.zeros((T, 1), np.int32), ids], axis=1)     # every token picks expert 0
    if kind == "sparse":
        used = RNG.choice(E, size=5, replace=False)
        return np.stack([RNG.choice(used, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    return _distinct_ids(T, k, E)


@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_route_quant_bitexact(name):
    T, K, k, E, kind = ROUTE_CASES[name]
    say(f"moe_route_quant {name} T={T} K={K} k={k} E={E}")
    x = _rand_bf16((T, K), scale_spread=10)
    ids = _route_ids(T, k, E, kind)
    xq, xs, sr, eri, gl = mx.moe_route_quant(bf16_dev(x), i32_dev(ids), E)
    torch.cuda.synchronize()
    rq, rs, rsr, reri, rc = moe_ref.route_quant_ref(x, ids, E)
    assert np.array_equal(host(gl), rc)
    assert np.array_equal(host(sr), rsr)
    assert np.array_equal(host(eri), reri)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs), rs)


@pytest.mark.parametrize("limit", [0, 1, 3])
@pytest.mark.parametrize("name", ["ragged-many-chunks", "hot-many-chunks", "leader-batches-E1024", "leaders-k1"])
def test_route_quant_wait_paths(name, limit):
    """A routing workgroup that stops waiting for the published counts counts
    them from topk_ids itself.  Limit 0 puts every workgroup on that path;
    1 and 3 polls leave some on each path.  Output bit-exact either way."""
    T, K, k, E, kind = ROUTE_CASES.get(name) or (1500, 128, 8, 64, "hot")
    say(f"moe_route_quant {name} T={T} K={K} k={k} E={E} wait limit {limit}")
    x = _rand_bf16((T, K), scale_spread=10)
    ids = _route_ids(T, k, E, kind)
    prev = mx.route_set_wait_limit(limit)
    try:
        xq, xs, sr, eri, gl = mx.moe_route_quant(bf16_dev(x), i32_dev(ids), E)
        torch.cuda.synchronize()
    finally:
        mx.route_set_wait_limit(prev)
    rq, rs, rsr, reri, rc = moe_ref.route_quant_ref(x, ids, E)
    assert np.array_equal(host(gl), rc)
    assert np.array_equal(host(sr), rsr)
    assert np.array_equal(host(eri), reri)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xs), rs)


def test_route_quant_reused_workspace():
    """Consecutive calls on one workspace: the second call's flags, counts and
    offsets replace the first's (its tags differ), never mix with them."""
    T, K, k, E = 3000, 64, 8, 96
    ws = torch.empty(mx.route_workspace_size(T, k, E), dtype=torch.uint8, device="cuda")
    for i, kind in enumerate([None, "hot", None]):
        say(f"moe_route_quant reused workspace, call {i}")
        x = _rand_bf16((T, K))
        ids = _route_ids(T, k, E, kind)
        xq, xs, sr, eri, gl = mx.moe_route_quant(bf16_dev(x), i32_dev(ids), E, workspace=ws)
        torch.cuda.synchronize()
        rq, rs, rsr, reri, rc = moe_ref.route_quant_ref(x, ids, E)
        assert np.array_equal(host(gl), rc)
        assert np.array_equal(host(sr), rsr)
        assert np.array_equal(host(eri), reri)
        assert np.array_equal(host(xq), rq)
        assert np.array_equal(host(xs), rs)


def route_graph_replays(call, T=2049, K=256, k=8, E=64, seed=5):
    """Captures `call(x, ids, outs)` (one routing call on the current stream)
    in a HIP graph, then replays it on three new inputs copied into the
    captured buffers, with eager routing calls and synchronisations between
    the replays; every replay and every eager call is checked against the
    oracle.  The inputs change between replays, so a replay that accepted an
    earlier replay's published counts would place rows wrongly."""
    rng = np.random.default_rng(seed)
    M = T * k
    sets = []
    for i in range(4):
        x = to_bf16_bits((rng.standard_normal((T, K)) * np.exp2(rng.integers(-6, 6, (T, 1)))).astype(np.float32))
        ids = np.stack([rng.choice(E, size=k, replace=False,
                                   p=None if i % 2 == 0 else np.r_[[0.3], np.full(E - 1, 0.7 / (E - 1))])
                        for _ in range(T)]).astype(np.int32)
        sets.append((x, ids))
    x_buf, ids_buf = bf16_dev(sets[0][0]), i32_dev(sets[0][1])

    def new_outs():
        return (torch.empty((M, K), dtype=torch.uint8, device="cuda"),
                torch.empty((M, K // 64, 2), dtype=torch.uint8, device="cuda"),
                torch.empty(M, dtype=torch.int32, device="cuda"), torch.empty(M, dtype=torch.int32, device="cuda"),
                torch.empty(E, dtype=torch.int64, device="cuda"))

    def check(outs, x, ids, what):
        ref = moe_ref.route_quant_ref(x, ids, E)
        for name, g, r in zip(("xq", "xs", "sorted_row", "expanded_row_idx", "group_list"), outs, ref):
            assert np.array_equal(host(g), r), (what, name)

    outs = new_outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        call(x_buf, ids_buf, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    check(outs, *sets[0], "warm-up")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x_buf, ids_buf, outs)
    for i in (1, 2, 3):
        x_buf.copy_(bf16_dev(sets[i][0]))
        ids_buf.copy_(i32_dev(sets[i][1]))
        say(f"graph replay {i}")
        graph.replay()
        torch.cuda.synchronize()
        check(outs, *sets[i], f"replay {i}")
        eager = new_outs()
        call(bf16_dev(sets[i - 1][0]), i32_dev(sets[i - 1][1]), eager)
        torch.cuda.synchronize()
        check(eager, *sets[i - 1], f"eager call after replay {i}")


def test_route_quant_graph_replays():
    T, k, E = 2049, 8, 64
    ws = torch.empty(mx.route_workspace_size(T, k, E), dtype=torch.uint8, device="cuda")
    route_graph_replays(lambda x, ids, outs: mx.moe_route_quant(x, ids, E, out=outs, workspace=ws), T=T, k=k, E=E)


def test_route_quant_empty_batch():
    say("moe_route_quant T=0")
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    gl = torch.full((8,), 7, dtype=torch.int64, device="cuda")
    out = (torch.empty((0, 128), dtype=torch.uint8, device="cuda"),
           torch.empty((0, 2, 2), dtype=torch.uint8, device="cuda"),
           torch.empty(0, dtype=torch.int32, device="cuda"), torch.empty(0, dtype=torch.int32, device="cuda"), gl)
    mx.moe_route_quant(x, ids, 8, out=out)
    torch.cuda.synchronize()
    assert host(gl).tolist() == [0] * 8


def test_route_quant_invalid_ids_are_dropped():
    T, K, k, E = 64, 128, 4, 10
    say("moe_route_quant invalid ids")
    x = _rand_bf16((T, K))
    ids = _distinct_ids(T, k, E)
    ids[3, 1] = -1
    ids[10, 0] = E
    ids[50, 3] = 1 << 20
    xq, xs, sr, eri, gl = mx.moe_route_quant(bf16_dev(x), i32_dev(ids), E)
    torch.cuda.synchronize()
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    assert np.array_equal(host(gl), np.bincount(flat[valid], minlength=E))
    order = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
    nv = order.size
    assert np.array_equal(host(sr)[:nv], order)
    e = host(eri)
    assert np.all(e[~valid] == -1)
    assert np.array_equal(e[order], np.arange(nv))
    qt, st = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(x))
    assert np.array_equal(host(xq)[:nv], qt[order // k])
    assert np.array_equal(host(xs)[:nv], st[order // k])


# --------------------------------------------------------------------------
# grouped GEMMs
# --------------------------------------------------------------------------

def _mx_operands(M, Kd, E, N, spread=4):
    a = RNG.standard_normal((M, Kd)) * np.exp2(RNG.integers(-spread, spread, (M, 1)))
    w = RNG.standard_normal((E * N, Kd)) * 0.05 * np.exp2(RNG.integers(-spread, spread, (E * N, 1)))
    aq, as_ = mx_ref.mx_quantize_ref(a)
    wq, ws = mx_ref.mx_quantize_ref(w)
    return aq, as_, wq.reshape(E, N, Kd), ws.reshape(E, N, -1, 2)


# The library picks 128-token tiles (three-slot ring) when Kd >= 384 and the
# experts average at most 64 rows (M <= 64 E), else 256-token tiles: here
# the *-128, *-3stage, *-4stage, decode-*, few-rows-* and many-tiles cases
# (empty experts appended where needed) take the 128-row kernel, the rest the
# 256-row one.
GMM_CASES = {
    "ragged": ([0, 1, 127, 128, 129, 255, 256, 257, 300, 0, 5], 256, 256),
    "single-expert": ([515], 384, 256),
    "tiny-rows": ([1, 1, 1, 2], 128, 512),
    "wide-k": ([64, 200, 33], 1024, 256),
    "multi-tile-n": ([700, 20], 256, 768),
    # tail tiles whose valid rows end at or just past a wave's 32- or
    # 64-token boundary (waves skip MFMAs / token DMA); K = 512 runs the
    # 4-stage scale groups
    "tail-boundaries": ([64, 65, 192, 193, 32, 33, 128, 1], 512, 256),
    # the same tails with one large expert: 256-row tiles, 4-stage scale groups
    "tail-boundaries-256": ([64, 65, 192, 193, 32, 33, 128, 1, 2000], 512, 256),
    # the same tails on 128-row tiles
    "tail-boundaries-128": ([64, 65, 192, 193, 32, 33, 128, 1] + [0] * 4, 512, 256),
    # 128-row tiles with the fewest k stages (3) and tails at 16/32/128 rows
    "small-tiles-3stage": ([16, 17, 31, 32, 33, 127, 128, 129, 0, 255, 1] + [0] * 2, 384, 512),
    # decode-shaped: many experts of 0-4 rows, 6 k stages
    "decode-like": ([2, 3, 0, 1, 2, 2, 0, 4] * 8, 768, 256),
    # 512 tiles, two per CU: the ring carries across tile boundaries
    "decode-many-tiles": ([2, 3, 1, 1, 2, 2, 5, 4] * 16, 384, 1024),
    # 128-row tiles with 4 k stages (one scale group per tile): tails at
    # 16/32/128 rows; 1024 tiles.  decode-many-tiles-4stage runs two tiles per
    # CU, so the second tile reads the expert tables after the scale ring's
    # second buffer has been written (waves 6 and 7, which have no scale
    # rows, must not write past that buffer)
    "small-tiles-4stage": ([16, 17, 31, 32, 33, 127, 128, 129, 0, 255, 1] + [0] * 2, 512, 512),
    "decode-many-tiles-4stage": ([2, 3, 1, 1, 2, 2, 5, 4] * 16, 512, 1024),
    # 128-row tiles, 512 of them (two per CU): the ring carries across tiles
    "few-rows-many-tiles": ([6, 7, 5, 9, 6, 8, 10, 5] * 16, 384, 1024),
    "few-rows-many-tiles-4stage": ([6, 7, 5, 9, 6, 8, 10, 5] * 16, 512, 1024),
    # mostly empty experts beside a few of 32-70 rows (256-row tiles, K = 256)
    "sparse-ragged": ([70, 33, 32, 1, 2] + [0] * 40, 256, 256),
    # 128-row tiles, 1024 of them (four per CU), 3 k stages
    "many-tiles": ([2, 3, 1, 1, 2, 2, 5, 4] * 16, 384, 2048),
}


@pytest.mark.parametrize("name", list(GMM_CASES))
@pytest.mark.parametrize("gl_type", [1, 0])
def test_gmm_mx_parity(name, gl_type):
    counts, Kd, N = GMM_CASES[name]
    counts = np.array(counts, np.int64)
    M, E = int(counts.sum()), len(counts)
    say(f"gmm_mx {name} gl_type={gl_type} M={M} Kd={Kd} N={N} E={E}")
    aq, as_, wq, ws = _mx_operands(M, Kd, E, N)
    gl = counts if gl_type == 1 else np.cumsum(counts)
    y = mx.gmm_mx(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(gl), gl_type)
    torch.cuda.synchronize()
    ref = moe_ref.gmm_mx_ref(aq, as_, wq, ws, gl, gl_type)
    err = bf16_rows_rel_err(bf16_host(y), ref)
    say(f"  max row rel err {err.max():.3g}")
    assert err.max() <= TOL


def test_gmm_mx_exact_cases():
    say("gmm_mx all-ones and single-nonzero")
    M, K, N, E = 300, 256, 256, 3
    aq = np.full((M, K), 0x38, np.uint8)
    as_ = np.full((M, K // 64, 2), 127, np.uint8)
    wq = np.full((E, N, K), 0x38, np.uint8)
    ws = np.full((E, N, K // 64, 2), 127, np.uint8)
    y = mx.gmm_mx(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev([100, 0, 200]), 1)
    torch.cuda.synchronize()
    assert np.all(mx_ref.bf16_to_f64(bf16_host(y)) == K)
    aq = np.zeros((M, K), np.uint8)
    aq[np.arange(M), np.arange(M) % K] = 0x40          # 2.0 at a moving k
    as_ = np.full((M, K // 64, 2), 127, np.uint8)
    as_[:, 0, 0] = 129
    wq = np.zeros((E, N, K), np.uint8)
    wq[:, :, :] = 0xB8                                 # -1.0 everywhere
    y = mx.gmm_mx(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev([100, 0, 200]), 1)
    torch.cuda.synchronize()
    ref = mx_ref.bf16_to_f64(moe_ref.gmm_mx_ref(aq, as_, wq, ws, np.array([100, 0, 200]), 1))
    assert np.array_equal(mx_ref.bf16_to_f64(bf16_host(y)), ref)


def test_gmm_mx_bf16_rounding_is_rne():
    """Exact fp32 sums that need rounding to bf16 (including exact ties) must
    round to nearest even, as the oracle does."""
    say("gmm_mx bf16 rounding")
    rng = np.random.default_rng(11)
    M, K, N, E = 256, 128, 256, 1
    aq = np.zeros((M, K), np.uint8)
    # 256 + small terms: the sum needs more than bf16's 8 significant bits
    aq[:, 0] = 0x78                                        # 256
    small = np.array([0x38, 0x30, 0x28, 0x20, 0x3C, 0x34, 0x00], np.uint8)   # 1, .5, .25, .125, 1.5, .75, 0
    for j in range(1, 4):
        aq[:, j] = rng.choice(small, M)
    as_ = np.full((M, K // 64, 2), 127, np.uint8)
    wq = np.zeros((E, N, K), np.uint8)
    wq[0, :, :4] = np.where(rng.random((N, 4)) < 0.5, 0x38, 0xB8)   # +-1
    wq[0, :, 0] = 0x38
    ws = np.full((E, N, K // 64, 2), 127, np.uint8)
    y = mx.gmm_mx(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev([M]), 1)
    torch.cuda.synchronize()
    ref = moe_ref.gmm_mx_ref(aq, as_, wq, ws, np.array([M]), 1)
    assert np.array_equal(bf16_host(y), ref)


def test_gmm_mx_guard_bands_and_untouched_rows():
    counts = np.array([0, 129, 0, 70], np.int64)
    M, Kd, N, E = 250, 128, 256, 4                     # 51 rows owned by no expert
    say("gmm_mx guard bands")
    aq, as_, wq, ws = _mx_operands(M, Kd, E, N)
    raw, y = guard_alloc(M * N, torch.bfloat16, fill=0x5A)
    mx.gmm_mx(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(counts), 1, out=y.view(M, N))
    torch.cuda.synchronize()
    assert guards_intact(raw, M * N * 2, fill=0x5A)
    yh = bf16_host(y.view(M, N))
    assert np.all(yh[199:] == 0x5A5A)                  # rows past the last expert untouched


# (128-row tiles: single, tail-boundaries-128, *-3stage, *-4stage, decode-*,
# few-rows-*, many-tiles)
GMM1_CASES = {
    "ragged": ([3, 0, 128, 129, 1, 260, 256, 511], 256, 128),
    "wide-i": ([70, 150], 128, 384),
    "single": ([1], 512, 128),
    "tail-boundaries": ([64, 65, 192, 193, 32, 33, 1], 512, 128),
    "tail-boundaries-256": ([64, 65, 192, 193, 32, 33, 1, 1500], 512, 128),
    "tail-boundaries-128": ([64, 65, 192, 193, 32, 33, 1] + [0] * 3, 512, 128),
    "small-tiles-3stage": ([16, 17, 31, 32, 33, 127, 128, 129, 0, 255, 1] + [0] * 2, 384, 256),
    "decode-like": ([2, 3, 0, 1, 2, 2, 0, 4] * 8, 2048, 128),
    # 512 tiles, two per CU: the ring carries across tile boundaries
    "decode-many-tiles": ([2, 3, 1, 1, 2, 2, 5, 4] * 16, 384, 512),
    "small-tiles-4stage": ([16, 17, 31, 32, 33, 127, 128, 129, 0, 255, 1] + [0] * 2, 512, 256),
    "decode-many-tiles-4stage": ([2, 3, 1, 1, 2, 2, 5, 4] * 16, 512, 512),
    "few-rows-many-tiles": ([6, 7, 5, 9, 6, 8, 10, 5] * 16, 384, 512),
    "few-rows-many-tiles-4stage": ([6, 7, 5, 9, 6, 8, 10, 5] * 16, 512, 512),
    "sparse-ragged": ([70, 33, 32, 1, 2] + [0] * 40, 256, 128),
    # 1024 tiles (four per CU), 4 k stages
    "many-tiles": ([2, 3, 1, 1, 2, 2, 5, 4] * 16, 512, 1024),
}


@pytest.mark.parametrize("name", list(GMM1_CASES))
def test_gmm_swiglu_mxquant_parity(name):
    counts, K, I = GMM1_CASES[name]
    counts = np.array(counts, np.int64)
    M, E = int(counts.sum()), len(counts)
    say(f"gmm_swiglu_mxquant {name} M={M} K={K} I={I} E={E}")
    aq, as_, wq, ws = _mx_operands(M, K, E, 2 * I)
    hq, hs, h = mx.gmm_swiglu_mxquant(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(counts), 1,
                                      h_debug=True)
    torch.cuda.synchronize()
    rq, rs, rh = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, wq, ws, counts, 1, I)
    hk = host(h)
    herr = row_rel_err(hk, rh)
    say(f"  h max row rel err {herr.max():.3g}")
    assert herr.max() <= 1e-3
    # requant bytes are exact given the kernel's own h
    kq, ks = mx_ref.mx_quantize_ref(hk.astype(np.float64))
    assert np.array_equal(host(hq), kq)
    assert np.array_equal(host(hs), ks)
    n_mis, n_bad = explain_hq_mismatches(host(hq), host(hs), rq, rh)
    say(f"  {name}: hq/hs mismatches vs oracle {n_mis} of {rq.size}, unexplained {n_bad}")
    assert n_bad == 0 and n_mis <= 0.01 * rq.size
    # cumulative group list gives the same bytes
    hq0, hs0 = mx.gmm_swiglu_mxquant(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(np.cumsum(counts)), 0)
    torch.cuda.synchronize()
    assert np.array_equal(host(hq0), host(hq)) and np.array_equal(host(hs0), host(hs))


def _checkpoint_bytes(rng, shape):
    """Random e4m3 weight bytes (NaN codes 0x7F/0xFF moved to 0x7E/0xFE) and
    scale bytes in 118..121, as a pre-quantised checkpoint ships them."""
    n = int(np.prod(shape))
    q = np.frombuffer(rng.bytes(n), np.uint8).copy()
    q[(q & 0x7F) == 0x7F] &= 0xFE
    s = rng.integers(118, 122, size=shape[:-1] + (shape[-1] // 64, 2), dtype=np.uint8)
    return q.reshape(shape), s


@pytest.mark.parametrize("kd", [256, 384, 512])
@pytest.mark.parametrize("rows", [(0, 4), (4, 13)])
def test_gmm_max_experts(kd, rows):
    """Both GEMMs at the largest expert count the kernels take (1024), with
    0-3 and 4-12 rows per expert: Kd = 256 runs the 256-row tiles, Kd = 384
    and 512 the 128-row tiles with the three-slot ring (3 and 4 k stages)."""
    rng = np.random.default_rng(1024 + kd + rows[0])
    E, N, I = 1024, 256, 128
    counts = rng.integers(rows[0], rows[1], E).astype(np.int64)
    M = int(counts.sum())
    say(f"gmm_mx / gmm_swiglu_mxquant E={E} M={M} Kd={kd}")
    aq, as_ = mx_ref.mx_quantize_ref(rng.standard_normal((M, kd)))
    wq, ws = _checkpoint_bytes(rng, (E, N, kd))
    y = mx.gmm_mx(u8_dev(aq), u8_dev(as_), u8_dev(wq), u8_dev(ws), i64_dev(counts), 1)
    torch.cuda.synchronize()
    err = bf16_rows_rel_err(bf16_host(y), moe_ref.gmm_mx_ref(aq, as_, wq, ws, counts, 1))
    say(f"  gmm_mx max row rel err {err.max():.3g}")
    assert err.max() <= TOL
    w13q, w13s = _checkpoint_bytes(rng, (E, 2 * I, kd))
    hq, hs, h = mx.gmm_swiglu_mxquant(u8_dev(aq), u8_dev(as_), u8_dev(w13q), u8_dev(w13s), i64_dev(counts), 1,
                                      h_debug=True)
    torch.cuda.synchronize()
    rq, rs, rh = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, w13q, w13s, counts, 1, I)
    hk = host(h)
    herr = row_rel_err(hk, rh)
    say(f"  gmm_swiglu_mxquant h max row rel err {herr.max():.3g}")
    assert herr.max() <= 1e-3
    kq, ks = mx_ref.mx_quantize_ref(hk.astype(np.float64))
    assert np.array_equal(host(hq), kq) and np.array_equal(host(hs), ks)


def _offset_u8_dev(a, offset=4):
    """uint8 device copy whose data pointer is 4 bytes past a 256-byte
    aligned allocation: 4-byte aligned, not 16-byte aligned."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    buf = torch.zeros(a.size + 64, dtype=torch.uint8, device="cuda")
    v = buf[offset:offset + a.size]
    v.copy_(torch.from_numpy(a.reshape(-1)).to("cuda"))
    assert v.data_ptr() % 16 == offset
    return v.view(a.shape)


def test_gmm_scales_not_16_byte_aligned():
    """Scale tensors that are 4- but not 16-byte aligned take the per-stage
    scale loads even where the k stages divide into groups of 4; both GEMMs
    still match the oracle."""
    counts = np.array([100, 0, 300, 45], np.int64)
    M, E, K, I, N = int(counts.sum()), len(counts), 512, 128, 256
    say(f"gemms with 4-byte-aligned scales M={M} K={K}")
    aq, as_, wq, ws = _mx_operands(M, K, E, N)
    y = mx.gmm_mx(u8_dev(aq), _offset_u8_dev(as_), u8_dev(wq), _offset_u8_dev(ws), i64_dev(counts), 1)
    torch.cuda.synchronize()
    err = bf16_rows_rel_err(bf16_host(y), moe_ref.gmm_mx_ref(aq, as_, wq, ws, counts, 1))
    say(f"  gmm_mx max row rel err {err.max():.3g}")
    assert err.max() <= TOL
    aq, as_, wq, ws = _mx_operands(M, K, E, 2 * I)
    hq, hs, h = mx.gmm_swiglu_mxquant(u8_dev(aq), _offset_u8_dev(as_), u8_dev(wq), _offset_u8_dev(ws),
                                      i64_dev(counts), 1, h_debug=True)
    torch.cuda.synchronize()
    rq, rs, rh = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, wq, ws, counts, 1, I)
    hk = host(h)
    assert row_rel_err(hk, rh).max() <= 1e-3
    kq, ks = mx_ref.mx_quantize_ref(hk.astype(np.float64))
    assert np.array_equal(host(hq), kq) and np.array_equal(host(hs), ks)


def test_gmm_swiglu_gate_up_closed_form():
    """gate row outputs 2, up row outputs 3 -> h = silu(2) * 3 everywhere."""
    K, I, E, M = 128, 128, 2, 40
    say("gmm_swiglu_mxquant closed form")
    aq = np.zeros((M, K), np.uint8); aq[:, 0] = 0x38
    as_ = np.full((M, K // 64, 2), 127, np.uint8)
    w = np.zeros((E, 2 * I, K), np.uint8)
    w[:, :I, 0] = 0x40
    w[:, I:, 0] = 0x44
    ws = np.full((E, 2 * I, K // 64, 2), 127, np.uint8)
    hq, hs, h = mx.gmm_swiglu_mxquant(u8_dev(aq), u8_dev(as_), u8_dev(w), u8_dev(ws), i64_dev([15, 25]), 1,
                                      h_debug=True)
    torch.cuda.synchronize()
    expect = 2.0 / (1 + np.exp(-2.0)) * 3.0
    assert np.allclose(host(h), expect, rtol=2e-6)
    rq, rs, _ = moe_ref.gmm_swiglu_mxquant_ref(aq, as_, w, ws, np.array([15, 25]), 1, I)
    assert np.array_equal(host(hq), rq) and np.array_equal(host(hs), rs)


# --------------------------------------------------------------------------
# finalize
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(64, 256, 2), (33, 2048, 8), (5, 4096, 1), (17, 128, 12)])
def test_finalize_bitexact(shape):
    T, K, k = shape
    say(f"moe_finalize T={T} K={K} k={k}")
    M = T * k
    y = _rand_bf16((M, K), scale_spread=6)
    w = RNG.random((T, k)).astype(np.float32)
    eri = RNG.permutation(M).astype(np.int32)
    out = mx.moe_finalize(bf16_dev(y), f32_dev(w), i32_dev(eri))
    torch.cuda.synchronize()
    ref = moe_ref.finalize_ref(y, w, eri)
    assert np.array_equal(bf16_host(out), ref)


def test_finalize_skips_invalid_rows():
    T, K, k = 20, 64, 3
    say("moe_finalize invalid rows")
    M = T * k
    y = _rand_bf16((M, K))
    w = RNG.random((T, k)).astype(np.float32)
    eri = RNG.permutation(M).astype(np.int32)
    eri[[4, 9, 30]] = -1
    eri[40] = M + 5
    out = mx.moe_finalize(bf16_dev(y), f32_dev(w), i32_dev(eri))
    torch.cuda.synchronize()
    w2 = w.copy().reshape(-1)
    bad = (eri < 0) | (eri >= M)
    w2[bad] = 0.0
    eri2 = np.where(bad, 0, eri)
    ref = moe_ref.finalize_ref(y, w2.reshape(T, k), eri2)
    assert np.array_equal(bf16_host(out), ref)


# --------------------------------------------------------------------------
# guard bands around every output of the layer's entry points
# --------------------------------------------------------------------------

def _guarded(shape, dtype, fill):
    n = int(np.prod(shape))
    raw, t = guard_alloc(n, dtype, fill=fill)
    return raw, t.view(shape), n * torch.empty((), dtype=dtype).element_size()


def test_every_output_guard_bands():
    """Each output buffer of moe_route_quant, gmm_swiglu_mxquant and
    moe_finalize sits between 4 KB guard bands of a fill byte; after the calls
    (on ragged shapes, several routing chunks, tail tiles) the bands are
    intact and the outputs still match the oracle."""
    T, K, k, E, I = 301, 512, 8, 64, 256
    M = T * k
    x = _rand_bf16((T, K), scale_spread=6)
    ids = _distinct_ids(T, k, E)
    outs = [_guarded((M, K), torch.uint8, 0x11), _guarded((M, K // 64, 2), torch.uint8, 0x22),
            _guarded((M,), torch.int32, 0x33), _guarded((M,), torch.int32, 0x44), _guarded((E,), torch.int64, 0x55)]
    say(f"guard bands: moe_route_quant T={T} K={K} k={k} E={E}")
    mx.moe_route_quant(bf16_dev(x), i32_dev(ids), E, out=tuple(o[1] for o in outs))
    torch.cuda.synchronize()
    for (raw, t, nb), fill in zip(outs, (0x11, 0x22, 0x33, 0x44, 0x55)):
        assert guards_intact(raw, nb, fill=fill)
    rq, rs, rsr, reri, rc = moe_ref.route_quant_ref(x, ids, E)
    xq, xs, sr, eri, gl = (o[1] for o in outs)
    assert np.array_equal(host(xq), rq) and np.array_equal(host(xs), rs) and np.array_equal(host(gl), rc)
    assert np.array_equal(host(sr), rsr) and np.array_equal(host(eri), reri)

    w13 = (RNG.standard_normal((E * 2 * I, K)) * 0.05)
    w13q, w13s = mx_ref.mx_quantize_ref(w13)
    w13q, w13s = w13q.reshape(E, 2 * I, K), w13s.reshape(E, 2 * I, -1, 2)
    hq_g, hs_g = _guarded((M, I), torch.uint8, 0x66), _guarded((M, I // 64, 2), torch.uint8, 0x77)
    say(f"guard bands: gmm_swiglu_mxquant M={M} K={K} I={I} E={E}")
    mx.gmm_swiglu_mxquant(xq, xs, u8_dev(w13q), u8_dev(w13s), gl, 1, out=(hq_g[1], hs_g[1]))
    torch.cuda.synchronize()
    assert guards_intact(hq_g[0], hq_g[2], fill=0x66) and guards_intact(hs_g[0], hs_g[2], fill=0x77)
    rhq, rhs, rh = moe_ref.gmm_swiglu_mxquant_ref(rq, rs, w13q, w13s, rc, 1, I)
    n_mis, n_bad = explain_hq_mismatches(host(hq_g[1]), host(hs_g[1]), rhq, rh)
    assert n_bad == 0 and n_mis <= 0.01 * rhq.size

    y = _rand_bf16((M, K), scale_spread=4)
    w = RNG.random((T, k)).astype(np.float32)
    out_g = _guarded((T, K), torch.bfloat16, 0x5A)
    say(f"guard bands: moe_finalize T={T} K={K} k={k}")
    mx.moe_finalize(bf16_dev(y), f32_dev(w), eri, out=out_g[1])
    torch.cuda.synchronize()
    assert guards_intact(out_g[0], out_g[2], fill=0x5A)
    assert np.array_equal(bf16_host(out_g[1]), moe_ref.finalize_ref(y, w, reri))
