"""MoE expert-layer oracle (test infrastructure only).

The chain follows the fused-experts description in "[WIP] Fix offline W8A8
MXFP8 quantization for Qwen3.5 on Ascend NPU" (sglang PR 32266, first commit
message: routing, activation quant, swiglu-quant grouped GEMM, grouped GEMM,
finalize routing) and the forward notes of "Quantization on Ascend", MXFP8 for
LLM MoE models (routing with fused MX activation quant; GEMM1 fuses gate/up,
SwiGLU and requant and wants a cumulative group list; GEMM2 takes counts).

Readings of what the pages leave open (numbered as in the design notes):

* R9   dropless routing, no capacity; inside one expert, rows keep the order
       of the flat assignment index i = t*k + j (a stable counting sort).
* R10  both maps are produced: sorted_row[p] = i and expanded_row_idx[i] = p.
* R13  w13 rows [0, I) are the gate projection, rows [I, 2I) the up projection.
* R14  SwiGLU is silu(gate) * up with silu(g) = g / (1 + exp(-g)), no clamp.
* R15  GEMM1's requant reads the float32 SwiGLU result (no bf16 rounding).
* R16  an MX dot product is the sum over 32-blocks of
       2^(sa + sb) * (sum of the block's e4m3 products).  Each block sum is
       exact in float64 (see ``_mx_dot``); the block terms are added in float64
       in ascending block order and the total is rounded once to float32.
* R17  GEMM2's output is the float32 accumulator rounded to bf16 (RNE).
* R18  finalize: out[t] = bf16(sum over j ascending of fp32(w[t,j] * y)),
       each multiply and add rounded to float32; no bias or residual.
* R19  group_list is int64; type 0 = cumulative (inclusive), 1 = counts.
* R28  the router (upstream of the layer): logits = x . Wg^T (+ a per-expert
       bias) from the bf16 operands, softmax over the E experts, the k
       experts with the largest logits in descending order (equal logits:
       lower expert id first), weights = their softmax probabilities,
       optionally renormalised to sum to 1.

bf16 tensors are carried as uint16 bit patterns.
"""

import numpy as np

from .mx_ref import (
    BLOCK,
    e2m1_decode,
    e4m3_decode,
    e8m0_decode,
    f32_to_bf16,
    bf16_to_f64,
    fp4_unpack,
    mx_quantize_ref,
    scales_flat,
)

# e4m3 code -> value, without the block scale; NaN codes are never produced
_E4M3_VALUES = e4m3_decode(np.arange(256))
# e2m1 code -> value (codes 0..15)
_E2M1_VALUES = e2m1_decode(np.arange(16))


def weight_values(wq, w_format):
    """Weight payload -> element values without the block scale: "e4m3"
    bytes [..., Kd], or "e2m1" packed bytes [..., Kd/2] (W4A8, R29-R30)."""
    if w_format == "e4m3":
        return _E4M3_VALUES[np.asarray(wq)]
    assert w_format == "e2m1", w_format
    return _E2M1_VALUES[fp4_unpack(wq)]


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def route_ref(topk_ids, E):
    """Stable counting sort of the T*k assignments by expert (R9, R10).

    Returns (counts int64 [E], sorted_row int32 [M], expanded_row_idx int32 [M]).
    Flat index i = t*k + j; position p of i is offsets[e_i] + the number of
    earlier flat indices with the same expert.  Ids must lie in [0, E).
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    assert np.all((ids >= 0) & (ids < E)), "expert id out of range"
    M = ids.size
    counts = np.bincount(ids, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)[:-1]])
    sorted_row = np.empty(M, np.int64)
    expanded_row_idx = np.empty(M, np.int64)
    fill = offsets.copy()
    for i in range(M):            # plain loop: the definition, one assignment at a time
        e = ids[i]
        p = fill[e]
        fill[e] += 1
        sorted_row[p] = i
        expanded_row_idx[i] = p
    return counts, sorted_row.astype(np.int32), expanded_row_idx.astype(np.int32)


def route_ref_fast(topk_ids, E):
    """Same result as ``route_ref`` via a stable argsort (for large M).

    A stable sort by expert keeps flat-index order inside each expert, which
    is exactly the counting-sort order; tests pin it to ``route_ref``.
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    assert np.all((ids >= 0) & (ids < E)), "expert id out of range"
    counts = np.bincount(ids, minlength=E).astype(np.int64)
    sorted_row = np.argsort(ids, kind="stable")
    expanded_row_idx = np.empty_like(sorted_row)
    expanded_row_idx[sorted_row] = np.arange(ids.size)
    return counts, sorted_row.astype(np.int32), expanded_row_idx.astype(np.int32)


def route_quant_ref(x_bf16, topk_ids, E):
    """Routing with fused MX activation quant.

    Every expanded row p carries the MX quantisation of its token's row
    x[sorted_row[p] // k].  The fused and two-step forms are the same bytes
    ("[WIP] Fix offline W8A8 MXFP8 ...", commit adding the fused routing
    quant: byte-identical to route-then-quant).

    Returns (xq uint8 [M, K], xs uint8 [M, ceil(K/64), 2], sorted_row,
    expanded_row_idx, counts).
    """
    x = bf16_to_f64(x_bf16)
    T, K = x.shape
    k = np.asarray(topk_ids).shape[1]
    counts, sorted_row, expanded_row_idx = (
        route_ref(topk_ids, E) if T * k <= 4096 else route_ref_fast(topk_ids, E))
    q_tok, s_tok = mx_quantize_ref(x)            # quantise each token once
    tok = sorted_row.astype(np.int64) // k
    return q_tok[tok], s_tok[tok], sorted_row, expanded_row_idx, counts


def group_bounds(group_list, group_list_type, M):
    """Row range [start_e, end_e) of every expert from a group list (R19).

    Type 1 = per-expert counts, type 0 = inclusive cumulative counts
    ("PR #30768 report", key source excerpt: the fused GEMM1 wants the
    cumulative form and the dispatcher hands out counts).
    """
    gl = np.asarray(group_list).astype(np.int64)
    if group_list_type == 1:
        ends = np.cumsum(gl)
    elif group_list_type == 0:
        ends = gl.copy()
    else:
        raise ValueError("group_list_type must be 0 (cumulative) or 1 (count)")
    starts = np.concatenate([[0], ends[:-1]])
    assert np.all(ends >= starts) and ends[-1] <= M
    return starts, ends


# --------------------------------------------------------------------------
# grouped GEMMs
# --------------------------------------------------------------------------

def _mx_dot(aq, as_flat, wq, ws_flat, w_format="e4m3"):
    """float32 result of the MX dot products of rows of A with rows of W (R16).

    aq [n, Kd] e4m3 codes; wq [N, Kd] e4m3 codes, or [N, Kd/2] packed e2m1
    (W4A8); as_flat [n, nb], ws_flat [N, nb] scale bytes, nb = Kd/32.  For
    each block b the element products are summed exactly: every e4m3 value is
    an integer multiple of 2^-9 below 2^9 (an e2m1 value a multiple of 2^-1 up
    to 6), so products are multiples of 2^-18 below 2^18 and a 32-term sum
    fits in 41 bits of a float64 mantissa, whatever the order.  Block sums are
    scaled by 2^(sa + sb) (exact) and added in ascending block order in
    float64; the total is rounded once to float32.  Returns float32 [n, N].
    """
    n, Kd = aq.shape
    N = wq.shape[0]
    assert Kd % BLOCK == 0, "GEMM operands need whole 32-blocks"
    nb = Kd // BLOCK
    av = _E4M3_VALUES[aq].reshape(n, nb, BLOCK)
    wv = weight_values(wq, w_format).reshape(N, nb, BLOCK)
    sa = e8m0_decode(as_flat[:, :nb])            # [n, nb]
    sw = e8m0_decode(ws_flat[:, :nb])            # [N, nb]
    acc = np.zeros((n, N))
    for b in range(nb):
        part = av[:, b, :] @ wv[:, b, :].T       # exact block sums
        acc += part * sa[:, b:b + 1] * sw[:, b][None, :]
    return acc.astype(np.float32)


def silu_mul_ref(g, u):
    """SwiGLU (R14): fp32(g * sigmoid(g) * u), evaluated in float64."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    return (g / (1.0 + np.exp(-g)) * u).astype(np.float32)


def gmm_swiglu_mxquant_ref(aq, as_, w13q, w13s, group_list, group_list_type, I, w_format="e4m3"):
    """GEMM1 with SwiGLU and MX requant fused, per expert.

    For expert e and its rows: acc = A . W13_e^T (R16), gate = acc[:, :I],
    up = acc[:, I:] (R13), h = silu(gate) * up (R14), then MX quantise h along
    I (R15).  Returns (hq uint8 [M, I], hs uint8 [M, ceil(I/64), 2],
    h float32 [M, I]).  Rows past the last expert's end are left zero.
    """
    M, K = aq.shape
    E = w13q.shape[0]
    assert w13q.shape == (E, 2 * I, K if w_format == "e4m3" else K // 2)
    starts, ends = group_bounds(group_list, group_list_type, M)
    as_flat = scales_flat(as_, K)
    h = np.zeros((M, I), np.float32)
    for e in range(E):
        r0, r1 = starts[e], ends[e]
        if r1 == r0:
            continue
        acc = _mx_dot(aq[r0:r1], as_flat[r0:r1], w13q[e], scales_flat(w13s[e], K), w_format)
        h[r0:r1] = silu_mul_ref(acc[:, :I], acc[:, I:])
    hq, hs = mx_quantize_ref(h.astype(np.float64))
    return hq, hs, h


def gmm_mx_ref(aq, as_, wq, ws, group_list, group_list_type, w_format="e4m3"):
    """Grouped MX GEMM with bf16 output (GEMM2), per expert.

    y[rows of e] = bf16(A_e . W_e^T) (R16, R17).  wq [E, N, Kd] e4m3, or
    [E, N, Kd/2] packed e2m1 (W4A8).
    Returns bf16 bits uint16 [M, N].
    """
    M, Kd = aq.shape
    E, N, _ = wq.shape
    starts, ends = group_bounds(group_list, group_list_type, M)
    as_flat = scales_flat(as_, Kd)
    y = np.zeros((M, N), np.float32)
    for e in range(E):
        r0, r1 = starts[e], ends[e]
        if r1 == r0:
            continue
        y[r0:r1] = _mx_dot(aq[r0:r1], as_flat[r0:r1], wq[e], scales_flat(ws[e], Kd), w_format)
    return f32_to_bf16(y)


# --------------------------------------------------------------------------
# finalize
# --------------------------------------------------------------------------

def finalize_ref(y_bf16, topk_w, expanded_row_idx):
    """Weighted un-permute and sum (R18).

    out[t] = bf16( sum_{j=0..k-1} fp32(w[t,j] * y[expanded_row_idx[t*k+j]]) ),
    accumulated in float32 in ascending j.  Returns bf16 bits uint16 [T, K].
    """
    w = np.asarray(topk_w, np.float32)
    T, k = w.shape
    y = bf16_to_f64(y_bf16).astype(np.float32)
    idx = np.asarray(expanded_row_idx).reshape(T, k)
    acc = np.zeros((T, y.shape[1]), np.float32)
    for j in range(k):
        acc = acc + w[:, j:j + 1] * y[idx[:, j]]   # float32 ops, each rounded
    return f32_to_bf16(acc)


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

def moe_forward_ref(x_bf16, topk_ids, topk_w, w13q, w13s, w2q, w2s, w_format="e4m3"):
    """Route+quant -> GEMM1+SwiGLU+requant -> GEMM2 -> finalize.  Weights
    are e4m3, or packed e2m1 for the W4A8 path (activations MXFP8 either way).

    Returns a dict with every intermediate (xq, xs, sorted_row,
    expanded_row_idx, counts, hq, hs, h, y) and the output ``out`` (bf16 bits).
    """
    E, twoI = w13q.shape[:2]
    K = np.asarray(x_bf16).shape[1]
    I = twoI // 2
    xq, xs, sorted_row, eri, counts = route_quant_ref(x_bf16, topk_ids, E)
    hq, hs, h = gmm_swiglu_mxquant_ref(xq, xs, w13q, w13s, counts, 1, I, w_format)
    y = gmm_mx_ref(hq, hs, w2q, w2s, counts, 1, w_format)
    out = finalize_ref(y, topk_w, eri)
    return dict(xq=xq, xs=xs, sorted_row=sorted_row, expanded_row_idx=eri,
                counts=counts, hq=hq, hs=hs, h=h, y=y, out=out)


def moe_token_ref(x_row_bf16, ids_row, w_row, w13q, w13s, w2q, w2s, w_format="e4m3"):
    """One token through the layer with no permutation (brute force).

    For each of the token's k experts: MX-quantise the token row, GEMM1 row
    with that expert, SwiGLU, requant, GEMM2 row, then the weighted sum in
    ascending j.  Uses the same per-row operations as the permuted pipeline,
    so it must reproduce it exactly (the pipeline's batching and permutation
    change no arithmetic).  Returns (out bf16 bits [K], per-j dict list).
    """
    E, twoI = w13q.shape[:2]
    K = np.asarray(x_row_bf16).size
    I = twoI // 2
    x = bf16_to_f64(np.asarray(x_row_bf16).reshape(1, K))
    xq, xs = mx_quantize_ref(x)
    per = []
    ys = []
    for j, e in enumerate(np.asarray(ids_row).tolist()):
        acc = _mx_dot(xq, scales_flat(xs, K), w13q[e], scales_flat(w13s[e], K), w_format)
        h = silu_mul_ref(acc[:, :I], acc[:, I:])
        hq, hs = mx_quantize_ref(h.astype(np.float64))
        yv = _mx_dot(hq, scales_flat(hs, I), w2q[e], scales_flat(w2s[e], I), w_format)
        yb = f32_to_bf16(yv)
        ys.append(yb[0])
        per.append(dict(expert=e, xq=xq[0], xs=xs[0], h=h[0], hq=hq[0], hs=hs[0], y=yb[0]))
    w = np.asarray(w_row, np.float32).reshape(1, -1)
    out = finalize_ref(np.stack(ys), w, np.arange(len(ys)).reshape(1, -1))
    return out[0], per


def moe_dense_bruteforce_ref(x_bf16, topk_ids, topk_w, w13q, w13s, w2q, w2s, w_format="e4m3"):
    """Every token through ``moe_token_ref``; tiny inputs only."""
    T = np.asarray(x_bf16).shape[0]
    return np.stack([
        moe_token_ref(x_bf16[t], topk_ids[t], topk_w[t], w13q, w13s, w2q, w2s, w_format)[0]
        for t in range(T)])


def moe_unquantized_ref(x_bf16, topk_ids, topk_w, w13_bf16, w2_bf16):
    """The same layer with no MX quantisation at all (float64 throughout).

    A sanity reference for the size of the quantisation error, not a parity
    target: out[t] = sum_j w[t,j] * (silu(x W1^T) * (x W3^T)) W2^T.
    """
    x = bf16_to_f64(x_bf16)
    T, K = x.shape
    w13 = bf16_to_f64(w13_bf16.reshape(-1, K)).reshape(w13_bf16.shape)
    w2 = bf16_to_f64(w2_bf16.reshape(-1, w2_bf16.shape[-1])).reshape(w2_bf16.shape)
    I = w13.shape[1] // 2
    out = np.zeros((T, K))
    ids = np.asarray(topk_ids)
    for t in range(T):
        for j, e in enumerate(ids[t]):
            a = w13[e] @ x[t]
            h = a[:I] / (1.0 + np.exp(-a[:I])) * a[I:]
            out[t] += float(topk_w[t, j]) * (w2[e] @ h)
    return out


# --------------------------------------------------------------------------
# router (upstream of the layer: produces the top-k ids and weights)
# --------------------------------------------------------------------------

def router_ref(x_bf16, gate_bf16, bias=None, k=8, renormalize=True):
    """Top-k softmax router over a bf16 gate linear ("Quantization on Ascend",
    MXFP8 for LLM MoE models, implementation notes: the router gate is a
    plain linear layer kept in bf16 on the online path), reading R28.

    Everything in float64: logits = x . Wg^T (+ bias), p = softmax(logits);
    the k largest logits in descending order, equal logits taken lower id
    first (a stable sort); weights p[ids], divided by their sum when
    ``renormalize``.  Returns (ids int32 [T,k], weights float32 [T,k],
    logits float64 [T,E]).
    """
    x = bf16_to_f64(np.asarray(x_bf16))
    g = bf16_to_f64(np.asarray(gate_bf16))
    logits = x @ g.T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float64)[None, :]
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32), logits
