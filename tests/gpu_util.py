"""Helpers shared by the GPU parity tests (host <-> device marshalling and
the comparison rules).  Imported only by tests marked ``gpu``."""

import os
import sys

import numpy as np
import torch

from oracle import mx_ref
from oracle.moe_ref import router_ref
from oracle.mx_ref import bf16_to_f64


def say(msg):
    """Name the case before each GPU step, flushed, so a failing run says which.
    With MXMOE_CASE_LOG set, the line is also appended to that file (passing
    tests' measured errors are otherwise not shown)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()
    path = os.environ.get("MXMOE_CASE_LOG")
    if path:
        with open(path, "a") as f:
            f.write(msg + "\n")


def dev():
    return torch.device("cuda:0")


def bf16_dev(bits):
    """uint16 bf16 bit patterns (NumPy) -> torch.bfloat16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def bf16_host(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def i64_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(dev())


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def host(t):
    return t.detach().cpu().numpy()


def row_rel_err(got, ref):
    """Per-row max|got - ref| / max|ref| (the 2e-2 output rule); a row whose
    reference is all zero must be all zero.  Returns the per-row errors."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def bf16_rows_rel_err(got_bits, ref_bits):
    return row_rel_err(mx_ref.bf16_to_f64(got_bits), mx_ref.bf16_to_f64(ref_bits))


def quantize_experts_ref(w_bits):
    """Oracle MX quantisation of bf16 expert weights [E, N, Kd] (host)."""
    E, N, Kd = w_bits.shape
    q, s = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(w_bits.reshape(E * N, Kd)))
    return q.reshape(E, N, Kd), s.reshape(E, N, -1, 2)


class LazyExpertQuant:
    """Per-expert oracle quantisation on first use (full-size workloads touch
    only the experts of the sampled tokens)."""

    def __init__(self, w_bits):
        self.w = w_bits
        self.shape = w_bits.shape
        self.cache = {}

    def get(self, e):
        if e not in self.cache:
            q, s = mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(self.w[e]))
            self.cache[e] = (q, s)
        return self.cache[e]


class FixedExperts:
    """Already-quantised expert weights with the LazyExpertQuant interface."""

    def __init__(self, q, s):
        self.q, self.s = q, s
        self.shape = q.shape

    def get(self, e):
        return self.q[e], self.s[e]


def guard_alloc(n, dtype, guard=4096, fill=0xA5):
    """A tensor of n elements with guard bands either side filled with `fill`."""
    esize = torch.empty((), dtype=dtype).element_size()
    gb = guard // esize
    raw = torch.full(((n + 2 * gb) * esize,), fill, dtype=torch.uint8, device=dev())
    return raw, raw[guard:guard + n * esize].view(dtype)


def guards_intact(raw, n_bytes, guard=4096, fill=0xA5):
    h = raw.cpu().numpy()
    return bool(np.all(h[:guard] == fill) and np.all(h[guard + n_bytes:] == fill))


def explain_hq_mismatches(hq, hs, hq_ref, h_ref, rtol=1e-3):
    """GEMM1's requant bytes may differ from the oracle's where the kernel's
    float32 h (MFMA accumulation) and the oracle's (float64 accumulation)
    round differently: near an e4m3 rounding midpoint, across a power-of-two
    block amax, or on elements much smaller than their row, whose absolute
    error is set by the row.  A GPU byte is accepted when it is the correct
    rounding of some h' within rtol * max|h_ref row| of the oracle's h:
        |deq(gpu) - h_ref| <= rtol * rowmax + half the e4m3 spacing at deq(gpu)
    (the spacing in the block's own scale), or the byte is the saturated
    code +-448 * 2^s and h_ref lies at or beyond that value.  Returns (number of bytes that
    differ from the oracle's, number not accepted)."""
    M, I = hq.shape
    nb = I // 32
    sb = hs.reshape(M, -1)[:, :nb].astype(np.int64)
    scale = np.repeat(np.exp2(sb - 127.0), 32, axis=1)
    q = hq.astype(np.int64)
    deq = mx_ref.e4m3_decode(q) * scale
    ef = (q >> 3) & 0xF
    spacing = np.where(ef == 0, 2.0 ** -9, np.exp2(ef - 10.0)) * scale
    h = np.asarray(h_ref, np.float64)
    atol = rtol * np.abs(h).max(axis=1, keepdims=True)
    ok = np.abs(deq - h) <= atol + 0.5 * spacing * (1 + 1e-9)
    # saturation: the largest code stands for every h' at or beyond 448 * 2^s
    sat = ((q & 0x7F) == 0x7E) & (np.sign(deq) * h >= np.abs(deq) - atol)
    ok |= sat
    return int(np.sum(hq != hq_ref)), int(np.sum(~ok))


def explain_hq_mismatches_rows(hq, hs, hq_ref, h_ref, rows=8192):
    """explain_hq_mismatches over row chunks (full-size matrices)."""
    n_mis = n_bad = 0
    for a in range(0, hq.shape[0], rows):
        m, b = explain_hq_mismatches(hq[a:a + rows], hs[a:a + rows], hq_ref[a:a + rows], h_ref[a:a + rows])
        n_mis += m
        n_bad += b
    return n_mis, n_bad


def bf16_rows_rel_err_chunked(got_bits, ref_bits, rows=8192):
    return np.concatenate([bf16_rows_rel_err(got_bits[a:a + rows], ref_bits[a:a + rows])
                           for a in range(0, got_bits.shape[0], rows)] or [np.zeros(0)])


def check_layer_every_row(d, out, inter, w13q, w13s, w2q, w2s, w_format, tol, e2e_tol):
    """Every row of every stage of one layer call against the oracle.

    * routing maps, group counts, xq and xs: bit-exact;
    * GEMM1: the oracle's h from the oracle's own xq/xs; the GPU's hq/hs
      bytes must equal the oracle's or be explained by the requant rule;
    * GEMM2 on identical operands (the GPU's hq/hs): every row within
      ``tol`` (per-row max relative error);
    * finalize of the GPU's y: bit-exact, every token;
    * end to end, every token: the oracle's chain (its own hq/hs into its
      GEMM2; rows whose hq/hs bytes equal the GPU's give y exactly as on
      identical operands, so only the others are recomputed), then its
      finalize, within ``e2e_tol``.
    Returns a dict of the measured figures."""
    import oracle_pool
    from oracle import moe_ref

    cfg = d["cfg"]
    K, I, k = cfg.K, cfg.I, cfg.k
    counts, sr, eri = moe_ref.route_ref_fast(d["topk_ids"], cfg.E)
    assert np.array_equal(inter["group_list"], counts)
    assert np.array_equal(inter["sorted_row"], sr)
    assert np.array_equal(inter["expanded_row_idx"], eri)
    say(f"  {cfg.name}: oracle routing quant")
    qt, st = oracle_pool.quantize_bf16(d["x"])
    tok = sr.astype(np.int64) // k
    xq, xs = qt[tok], st[tok]
    assert np.array_equal(inter["xq"], xq)
    assert np.array_equal(inter["xs"], xs)
    M = xq.shape[0]

    say(f"  {cfg.name}: oracle GEMM1 over {M} rows")
    h_ref = oracle_pool.gemm1_h(xq, xs, w13q, w13s, counts, 1, I, w_format)
    hq_ref, hs_ref = oracle_pool.quantize_f32(h_ref)
    n_mis, n_bad = explain_hq_mismatches_rows(inter["hq"], inter["hs"], hq_ref, h_ref)
    say(f"  {cfg.name}: hq/hs bytes differing from the oracle {n_mis} of {hq_ref.size}, unexplained {n_bad}")
    assert n_bad == 0 and n_mis <= 0.01 * hq_ref.size

    say(f"  {cfg.name}: oracle GEMM2 on the GPU's hq/hs")
    y_same = oracle_pool.gemm2_y(inter["hq"], inter["hs"], w2q, w2s, counts, 1, w_format)
    yerr = bf16_rows_rel_err_chunked(inter["y"], y_same)
    assert np.array_equal(out, moe_ref.finalize_ref(inter["y"], d["topk_w"], inter["expanded_row_idx"]))

    diff = np.nonzero((inter["hq"] != hq_ref).any(axis=1) |
                      (inter["hs"].reshape(M, -1) != hs_ref.reshape(M, -1)).any(axis=1))[0]
    y_ref = y_same.copy()
    say(f"  {cfg.name}: oracle GEMM2 on its own hq/hs ({diff.size} rows differ)")
    oracle_pool.gemm2_y(hq_ref, hs_ref, w2q, w2s, counts, 1, w_format, only_rows=diff, out=y_ref)
    out_ref = moe_ref.finalize_ref(y_ref, d["topk_w"], eri)
    e2e = bf16_rows_rel_err_chunked(out, out_ref)
    say(f"  {cfg.name}: y max row rel err {yerr.max():.3g} over {M} rows (identical operands); "
        f"{diff.size} rows with a requant difference; end-to-end out {e2e.max():.3g} over {out.shape[0]} tokens")
    assert yerr.max() <= tol
    assert e2e.max() <= e2e_tol
    return dict(y_err=float(yerr.max()), e2e=float(e2e.max()), hq_mismatch=n_mis, rows_requant_diff=int(diff.size))


# --------------------------------------------------------------------------
# the GPU router against the router oracle
# --------------------------------------------------------------------------

U32 = 2.0 ** -24   # float32 unit roundoff


def check_router(ids, w, x_bits, gate_bits, bias, k, renormalize):
    T, K = x_bits.shape
    E = gate_bits.shape[0]
    ids_o, _, L = router_ref(x_bits, gate_bits, bias, k, renormalize)
    xd, gd = bf16_to_f64(x_bits), bf16_to_f64(gate_bits)
    # |float32 sum - exact| <= K u sum|x g| (any summation order), plus the bias add
    mag = np.abs(xd) @ np.abs(gd).T
    fin = np.where(np.isfinite(L), np.abs(L), 0.0)
    delta = (K * U32 * mag + U32 * fin).max(axis=1) + 1e-30          # per token
    assert ids.shape == (T, k) and w.shape == (T, k)
    assert ((ids >= 0) & (ids < E)).all()
    assert all(len(set(r)) == k for r in ids.tolist()), "repeated expert in a token's selection"
    srt = -np.sort(-L, axis=1)
    got = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    both_inf = np.isneginf(got) & np.isneginf(srt[:, :k])
    diff = np.where(both_inf, 0.0, np.abs(got - srt[:, :k]))
    bad = np.argwhere(diff > 2 * delta[:, None])
    assert bad.size == 0, f"token {bad[0][0]} position {bad[0][1]}: logit off by {diff[tuple(bad[0])]}"
    if k < E:
        clear = (srt[:, k - 1] - srt[:, k]) > 2 * delta
    else:
        clear = np.ones(T, bool)
    same = np.sort(ids, axis=1) == np.sort(ids_o, axis=1)
    assert same[clear].all(), "selection differs where no near-tie decides it"
    # weights: softmax of the oracle logits over all experts / the GPU's selection
    z = L - L.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    pw = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        pw = pw / pw.sum(axis=1, keepdims=True)
    rtol = 4 * delta[:, None] + 1e-5
    err = np.abs(w - pw) / np.maximum(pw, 1e-30)
    assert (err <= rtol).all(), f"weight rel err {err.max():.3g}"
    return int((~clear).sum()), float(err.max())


def run_router(x_bits, gate_bits, bias, k, renormalize=True):
    import mxfp8_block_scaled_topk_amd as mx
    xb, gb = bf16_dev(x_bits), bf16_dev(gate_bits)
    bd = None if bias is None else f32_dev(np.asarray(bias, np.float32))
    ids, w = mx.moe_router(xb, gb, k, bias=bd, renormalize=renormalize)
    torch.cuda.synchronize()
    return host(ids), host(w)
