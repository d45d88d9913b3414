"""The oracle's row-wise work spread over CPU worker processes, for parity at
the full workload sizes (test infrastructure; imported only by tests).

Every function here calls the oracle's own routines (``moe_ref._mx_dot``,
``moe_ref.silu_mul_ref``, ``mx_ref.mx_quantize_ref``) on chunks of rows and
stitches the chunks back together.  Those routines compute each output row
from its own input row, the expert's weights and a fixed order of
operations (each 32-block's products summed exactly, blocks added in
ascending order, one rounding to float32; the quantiser works block by
block), so the stitched result is the bytes the oracle gives on the whole
matrix; ``test_oracle_pool.py`` pins that on the CPU.

The workers are forked once, by ``start`` (called when the test session is
configured, or at the start of the benchmark), before the process touches
the GPU, so no worker holds GPU state; they then wait for work.  Each
worker runs single-threaded BLAS (the thin 32-wide block products run
faster that way than on a shared thread pool).
"""

import multiprocessing as mp
import os

import numpy as np

from oracle import moe_ref, mx_ref

_POOL = None


def n_workers():
    # the GPU machine gives one GPU's tests 16 CPU threads
    return max(1, min(16, os.cpu_count() or 1))


def start():
    """Fork the workers now (call before the GPU is initialised)."""
    global _POOL
    if _POOL is None:
        _POOL = mp.get_context("fork").Pool(n_workers(), initializer=_init_worker)
    return _POOL


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def pool():
    return start()


def shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


# ---------------------------------------------------------------------------
# worker bodies (module level so the pool can pickle them)
# ---------------------------------------------------------------------------

def _w_gemm1(args):
    aq, as_flat, wq, ws_flat, I, w_format = args
    acc = moe_ref._mx_dot(aq, as_flat, wq, ws_flat, w_format)
    return moe_ref.silu_mul_ref(acc[:, :I], acc[:, I:])


def _w_gemm2(args):
    aq, as_flat, wq, ws_flat, w_format = args
    return mx_ref.f32_to_bf16(moe_ref._mx_dot(aq, as_flat, wq, ws_flat, w_format))


def _w_quant_f32(v):
    return mx_ref.mx_quantize_ref(np.asarray(v, np.float64))


def _w_quant_bf16(bits):
    return mx_ref.mx_quantize_ref(mx_ref.bf16_to_f64(bits))


def _w_quant_fp4_bf16(bits):
    return mx_ref.mxfp4_quantize_ref(mx_ref.bf16_to_f64(bits))


# ---------------------------------------------------------------------------
# parent side
# ---------------------------------------------------------------------------

def _chunks(n, rows):
    return [(r, min(r + rows, n)) for r in range(0, n, rows)]


def _expert_tasks(starts, ends, rows, only_rows=None):
    """(expert, row0, row1) pieces of every expert's row range; with
    ``only_rows`` (sorted row indices) the pieces hold just those rows."""
    out = []
    for e, (r0, r1) in enumerate(zip(starts.tolist(), ends.tolist())):
        if r1 <= r0:
            continue
        if only_rows is None:
            for a, b in _chunks(r1 - r0, rows):
                out.append((e, np.arange(r0 + a, r0 + b)))
        else:
            sel = only_rows[(only_rows >= r0) & (only_rows < r1)]
            out += [(e, sel[i:i + rows]) for i in range(0, sel.size, rows)]
    return out


def gemm1_h(aq, as_, w13q, w13s, group_list, group_list_type, I, w_format="e4m3", rows=1024):
    """h [M, I] float32, equal to ``gmm_swiglu_mxquant_ref(...)[2]``."""
    M, K = aq.shape
    starts, ends = moe_ref.group_bounds(group_list, group_list_type, M)
    as_flat = mx_ref.scales_flat(as_, K)
    tasks = _expert_tasks(starts, ends, rows)
    args = [(aq[r], as_flat[r], w13q[e], mx_ref.scales_flat(w13s[e], K), I, w_format) for e, r in tasks]
    h = np.zeros((M, I), np.float32)
    for (e, r), part in zip(tasks, pool().imap(_w_gemm1, args)):
        h[r] = part
    return h


def gemm2_y(aq, as_, wq, ws, group_list, group_list_type, w_format="e4m3", rows=1024, only_rows=None,
            out=None):
    """y [M, N] bf16 bits, equal to ``gmm_mx_ref(...)``; with ``only_rows``
    just those rows are computed (into ``out`` when given, else zeros)."""
    M, Kd = aq.shape
    N = wq.shape[1]
    starts, ends = moe_ref.group_bounds(group_list, group_list_type, M)
    as_flat = mx_ref.scales_flat(as_, Kd)
    tasks = _expert_tasks(starts, ends, rows, only_rows)
    args = [(aq[r], as_flat[r], wq[e], mx_ref.scales_flat(ws[e], Kd), w_format) for e, r in tasks]
    y = np.zeros((M, N), np.uint16) if out is None else out
    for (e, r), part in zip(tasks, pool().imap(_w_gemm2, args)):
        y[r] = part
    return y


def quantize_f32(v, rows=4096):
    """mx_quantize_ref of float32 rows [R, Kd] -> (q [R, Kd], s [R, ceil(Kd/64), 2])."""
    R, Kd = v.shape
    q = np.empty((R, Kd), np.uint8)
    s = np.empty((R, -(-Kd // 64), 2), np.uint8)
    parts = _chunks(R, rows)
    for (a, b), (qq, ss) in zip(parts, pool().imap(_w_quant_f32, [v[a:b] for a, b in parts])):
        q[a:b], s[a:b] = qq, ss
    return q, s


def quantize_bf16(bits, rows=2048, fp4=False):
    """mx_quantize_ref (or mxfp4_quantize_ref) of bf16 rows [R, Kd]."""
    R, Kd = bits.shape
    q = np.empty((R, Kd // 2 if fp4 else Kd), np.uint8)
    s = np.empty((R, -(-Kd // 64), 2), np.uint8)
    parts = _chunks(R, rows)
    fn = _w_quant_fp4_bf16 if fp4 else _w_quant_bf16
    for (a, b), (qq, ss) in zip(parts, pool().imap(fn, [bits[a:b] for a, b in parts])):
        q[a:b], s[a:b] = qq, ss
    return q, s


def _w_finalize(args):
    y_rows, w, k = args
    n = w.shape[0]
    return moe_ref.finalize_ref(y_rows, w, np.arange(n * k).reshape(n, k))


def route_quant(x_bits, topk_ids, E, rows=2048):
    """Equal to ``moe_ref.route_quant_ref``: the stable routing maps, and
    every expanded row's MX quantisation of its token (each token quantised
    once, by row chunks in the workers, then gathered)."""
    ids = np.asarray(topk_ids)
    k = ids.shape[1]
    counts, sorted_row, eri = moe_ref.route_ref_fast(ids, E)
    q_tok, s_tok = quantize_bf16(x_bits, rows)
    tok = sorted_row.astype(np.int64) // k
    return q_tok[tok], s_tok[tok], sorted_row, eri, counts


def finalize(y_bits, topk_w, expanded_row_idx, tokens=1024):
    """Equal to ``moe_ref.finalize_ref``: each chunk of tokens gets its own
    k rows of y (gathered here in token order) and the oracle's finalize
    runs on them in a worker."""
    w = np.asarray(topk_w, np.float32)
    T, k = w.shape
    idx = np.asarray(expanded_row_idx).reshape(T, k)
    parts = _chunks(T, tokens)
    args = [(y_bits[idx[a:b].reshape(-1)], w[a:b], k) for a, b in parts]
    out = np.empty((T, y_bits.shape[1]), np.uint16)
    for (a, b), part in zip(parts, pool().imap(_w_finalize, args)):
        out[a:b] = part
    return out
