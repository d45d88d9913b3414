"""Python binding of libmxmoe.so, the MXFP8 block-scaled top-k MoE expert
layer for AMD MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch tensors on the GPU (torch supplies device memory and the
current stream); outputs are allocated here when not passed in.  Any non-OK
status from the library raises ``MxError`` with the library's message.

Formats (see include/mxmoe.h): e4m3 payloads and e8m0 scales are uint8
tensors; scales use the pair-split layout [rows, ceil(cols/64), 2]; bf16
tensors are torch.bfloat16; group lists are int64 (type 1 = counts,
type 0 = inclusive cumulative counts).
"""

import ctypes
import functools
import inspect
import os

import torch

__all__ = [
    "MxError", "lib_path", "load", "mx_quantize", "moe_route_quant", "gmm_swiglu_mxquant",
    "gmm_mx", "moe_finalize", "moe_mxfp8_forward", "forward_workspace", "forward_intermediates",
    "route_workspace_size", "forward_workspace_size", "last_error", "moe_router", "mx_linear",
    "linear_workspace_size", "mx_quantize_fp4", "moe_route_quant_noalloc", "mx_pack_weights", "route_set_wait_limit",
    "gmm_swiglu_mxquant_packed", "gmm_mx_packed", "moe_mxfp8_forward_packed", "gmm_mx_w4a8", "gmm_swiglu_mxquant_w4a8", "moe_w4a8_forward",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

MX_OK = 0
GROUP_CUMULATIVE = 0
GROUP_COUNT = 1


class MxError(RuntimeError):
    """A non-OK status from libmxmoe."""


def lib_path():
    return os.path.join(_HERE, "libmxmoe.so")


def load():
    """Load libmxmoe.so (built by ``python -m mxfp8_block_scaled_topk_amd.build``).

    There is no fallback: a missing library is an error."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise MxError(f"{path} is missing; build it with `python -m mxfp8_block_scaled_topk_amd.build`")
    lib = ctypes.CDLL(path)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "mx_quantize": (I32, [P, I64, I64, I64, P, P, P]),
        "mx_quantize_fp4": (I32, [P, I64, I64, I64, P, P, P]),
        "moe_route_quant_workspace_size": (SZ, [I64, I64, I64]),
        "moe_route_quant": (I32, [P, P, I64, I64, I64, I64, P, P, P, P, P, P, SZ, P]),
        "moe_route_quant_noalloc": (I32, [P, P, I64, I64, I64, I64, P, P, P, P, P, P]),
        "moe_route_quant_set_wait_limit": (I64, [I64]),
        "gmm_swiglu_mxquant": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P, P, P]),
        "gmm_mx": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P]),
        "gmm_mx_w4a8": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P]),
        "gmm_swiglu_mxquant_w4a8": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P, P, P]),
        "moe_w4a8_forward": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
        "moe_finalize": (I32, [P, P, P, I64, I64, I64, I64, P, P]),
        "moe_mxfp8_forward_workspace_size": (SZ, [I64, I64, I64, I64, I64]),
        "moe_mxfp8_forward": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
        "moe_mxfp8_forward_workspace_layout": (I32, [I64, I64, I64, I64, I64, P]),
        "moe_router": (I32, [P, P, P, I64, I64, I64, I64, I32, P, P, P]),
        "mx_linear_workspace_size": (SZ, [I64, I64]),
        "mx_linear": (I32, [P, P, P, I64, I64, I64, P, P, SZ, P]),
        "mx_pack_weights": (I32, [P, I64, I64, I64, I32, P, P]),
        "gmm_swiglu_mxquant_packed": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P, P, P]),
        "gmm_mx_packed": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P]),
        "moe_mxfp8_forward_packed": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
        "mx_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def last_error():
    return load().mx_last_error().decode()


def _check(rc, what):
    if rc != MX_OK:
        raise MxError(f"{what}: status {rc}: {last_error()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _stream_scoped(fn):
    """Run ``fn`` with its ``stream`` argument (when given) as torch's current
    stream.  Every tensor the binding allocates for the call (outputs left to
    it, internal workspaces) then comes from that stream's pool of the caching
    allocator: freed on return, such a workspace is reused only by later work
    on the same stream, which runs after the kernels that used it.  Allocated
    on another stream instead, it could be handed to work on that stream while
    the kernels still read or write it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kw):
        s = sig.bind(*args, **kw).arguments.get("stream")
        if s is None:
            return fn(*args, **kw)
        with torch.cuda.stream(s):
            return fn(*args, **kw)
    return wrapper


# Argument checks.  The library receives raw pointers and sizes, so every
# tensor is checked here for dtype, exact shape, contiguity and device before
# the call: a tensor smaller than its sizes say would be read or written out
# of bounds on the GPU.  Shape checks come first and residency on the GPU
# last, so that shape errors are reported the same way on any device.

def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _need_shape(t, shape, name, dtype, device):
    """t: a contiguous `dtype` tensor of exactly `shape` on `device`."""
    _need(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _need_workspace(ws, nbytes, device, name="workspace"):
    _need(ws, torch.uint8, name, 1)
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ws.device != device:
        raise ValueError(f"{name} must be on {device}, got {ws.device}")
    if ws.numel() < nbytes:
        raise ValueError(f"{name} has {ws.numel()} bytes, {nbytes} needed")


def _need_gpu(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")


def _pairs(n):
    return -(-n // 64)


@_stream_scoped
def mx_quantize(x, q=None, s=None, stream=None):
    """MX-quantise the last dim of a bf16 tensor [..., Kd] (rows may be strided
    with unit inner stride).  Returns (q uint8 [..., Kd], s uint8 [..., ceil(Kd/64), 2])."""
    _need(x, torch.bfloat16, "x")
    kd = x.shape[-1]
    lead = tuple(x.shape[:-1])
    x2 = x.reshape(-1, kd) if x.dim() != 2 else x
    if x2.stride(-1) != 1:
        raise ValueError("x must have unit stride along the last dim")
    rows = x2.shape[0]
    if q is None:
        q = torch.empty(lead + (kd,), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(lead + (_pairs(kd), 2), dtype=torch.uint8, device=x.device)
    _need_shape(q, lead + (kd,), "q", torch.uint8, x.device)
    _need_shape(s, lead + (_pairs(kd), 2), "s", torch.uint8, x.device)
    ld = x2.stride(0) if rows > 1 else kd
    _need_gpu(x, "x")
    rc = load().mx_quantize(_ptr(x2), rows, kd, ld, _ptr(q), _ptr(s), _stream(stream))
    _check(rc, "mx_quantize")
    return q, s


def route_workspace_size(T, k, E):
    return int(load().moe_route_quant_workspace_size(T, k, E))


def route_set_wait_limit(polls):
    """Polls a routing workgroup makes for the published expert counts before
    counting them itself (process-wide; 0 = always count). Returns the
    previous value."""
    return int(load().moe_route_quant_set_wait_limit(int(polls)))


@_stream_scoped
def moe_route_quant(x, topk_ids, E, out=None, workspace=None, stream=None):
    """Routing with fused MX activation quant.

    Returns (xq [M,K] u8, xs [M,K/64,2] u8, sorted_row [M] i32,
    expanded_row_idx [M] i32, group_list [E] i64 counts)."""
    _need(x, torch.bfloat16, "x", 2); _need(topk_ids, torch.int32, "topk_ids", 2)
    T, K = x.shape
    k = topk_ids.shape[1]
    M = T * k
    dev = x.device
    _need_shape(x, (T, K), "x", torch.bfloat16, dev)
    _need_shape(topk_ids, (T, k), "topk_ids", torch.int32, dev)
    if out is None:
        out = (torch.empty((M, K), dtype=torch.uint8, device=dev),
               torch.empty((M, _pairs(K), 2), dtype=torch.uint8, device=dev),
               torch.empty(M, dtype=torch.int32, device=dev),
               torch.empty(M, dtype=torch.int32, device=dev),
               torch.empty(E, dtype=torch.int64, device=dev))
    xq, xs, sr, eri, gl = out
    _need_shape(xq, (M, K), "xq", torch.uint8, dev)
    _need_shape(xs, (M, _pairs(K), 2), "xs", torch.uint8, dev)
    _need_shape(sr, (M,), "sorted_row", torch.int32, dev)
    _need_shape(eri, (M,), "expanded_row_idx", torch.int32, dev)
    _need_shape(gl, (E,), "group_list", torch.int64, dev)
    need = route_workspace_size(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need_workspace(workspace, need, dev)
    _need_gpu(x, "x")
    rc = load().moe_route_quant(_ptr(x), _ptr(topk_ids), T, K, k, E, _ptr(xq), _ptr(xs), _ptr(sr), _ptr(eri),
                                _ptr(gl), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "moe_route_quant")
    return xq, xs, sr, eri, gl


@_stream_scoped
def moe_route_quant_noalloc(x, topk_ids, E, out=None, stream=None):
    """moe_route_quant with the routing scratch held by the library (no
    workspace; the C call allocates nothing).  The caller may pass the
    outputs preallocated in ``out`` (then this call allocates nothing either).
    Returns (xq, xs, sorted_row, expanded_row_idx, group_list)."""
    _need(x, torch.bfloat16, "x", 2); _need(topk_ids, torch.int32, "topk_ids", 2)
    T, K = x.shape
    k = topk_ids.shape[1]
    M = T * k
    dev = x.device
    _need_shape(x, (T, K), "x", torch.bfloat16, dev)
    _need_shape(topk_ids, (T, k), "topk_ids", torch.int32, dev)
    if out is None:
        out = (torch.empty((M, K), dtype=torch.uint8, device=dev),
               torch.empty((M, _pairs(K), 2), dtype=torch.uint8, device=dev),
               torch.empty(M, dtype=torch.int32, device=dev),
               torch.empty(M, dtype=torch.int32, device=dev),
               torch.empty(E, dtype=torch.int64, device=dev))
    xq, xs, sr, eri, gl = out
    _need_shape(xq, (M, K), "xq", torch.uint8, dev)
    _need_shape(xs, (M, _pairs(K), 2), "xs", torch.uint8, dev)
    _need_shape(sr, (M,), "sorted_row", torch.int32, dev)
    _need_shape(eri, (M,), "expanded_row_idx", torch.int32, dev)
    _need_shape(gl, (E,), "group_list", torch.int64, dev)
    _need_gpu(x, "x")
    rc = load().moe_route_quant_noalloc(_ptr(x), _ptr(topk_ids), T, K, k, E, _ptr(xq), _ptr(xs), _ptr(sr), _ptr(eri),
                                        _ptr(gl), _stream(stream))
    _check(rc, "moe_route_quant_noalloc")
    return xq, xs, sr, eri, gl


@_stream_scoped
def gmm_swiglu_mxquant(a, a_s, w13, w13_s, group_list, group_list_type=GROUP_COUNT, out=None,
                       h_debug=False, stream=None, _w4=False, _packed=False):
    """GEMM1 + SwiGLU + MX requant.  Returns (hq, hs) or (hq, hs, h) with h_debug."""
    _need(a, torch.uint8, "a", 2); _need(w13, torch.uint8, "w13", 3)
    M, K = a.shape
    E, twoI, Kw = w13.shape
    Kb = K // 2 if _w4 else K           # weight payload bytes per row
    if Kw != Kb or twoI % 2:
        raise ValueError(f"w13 must be [E, 2I, {Kb}], got {tuple(w13.shape)}")
    I = twoI // 2
    dev = a.device
    _need_shape(a, (M, K), "a", torch.uint8, dev)
    _need_shape(a_s, (M, _pairs(K), 2), "a_s", torch.uint8, dev)
    _need_shape(w13, (E, twoI, Kb), "w13", torch.uint8, dev)
    _need_shape(w13_s, (E, twoI, _pairs(K), 2), "w13_s", torch.uint8, dev)
    _need_shape(group_list, (E,), "group_list", torch.int64, dev)
    if out is None:
        out = (torch.empty((M, I), dtype=torch.uint8, device=dev),
               torch.empty((M, _pairs(I), 2), dtype=torch.uint8, device=dev))
    hq, hs = out
    _need_shape(hq, (M, I), "hq", torch.uint8, dev)
    _need_shape(hs, (M, _pairs(I), 2), "hs", torch.uint8, dev)
    h = torch.empty((M, I), dtype=torch.float32, device=dev) if h_debug else None
    _need_gpu(a, "a")
    name = "gmm_swiglu_mxquant_w4a8" if _w4 else "gmm_swiglu_mxquant_packed" if _packed else "gmm_swiglu_mxquant"
    rc = getattr(load(), name)(_ptr(a), _ptr(a_s), _ptr(w13), _ptr(w13_s), _ptr(group_list), group_list_type, M, K,
                               I, E, _ptr(hq), _ptr(hs), _ptr(h), _stream(stream))
    _check(rc, name)
    return (hq, hs, h) if h_debug else (hq, hs)


@_stream_scoped
def gmm_mx(a, a_s, w, w_s, group_list, group_list_type=GROUP_COUNT, out=None, stream=None, _w4=False,
           _packed=False):
    """Grouped MX GEMM, bf16 output [M, N]."""
    _need(a, torch.uint8, "a", 2); _need(w, torch.uint8, "w", 3)
    M, Kd = a.shape
    E, N, Kw = w.shape
    Kb = Kd // 2 if _w4 else Kd
    if Kw != Kb:
        raise ValueError(f"w must be [E, N, {Kb}], got {tuple(w.shape)}")
    dev = a.device
    _need_shape(a, (M, Kd), "a", torch.uint8, dev)
    _need_shape(a_s, (M, _pairs(Kd), 2), "a_s", torch.uint8, dev)
    _need_shape(w, (E, N, Kb), "w", torch.uint8, dev)
    _need_shape(w_s, (E, N, _pairs(Kd), 2), "w_s", torch.uint8, dev)
    _need_shape(group_list, (E,), "group_list", torch.int64, dev)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _need_shape(out, (M, N), "out", torch.bfloat16, dev)
    _need_gpu(a, "a")
    name = "gmm_mx_w4a8" if _w4 else "gmm_mx_packed" if _packed else "gmm_mx"
    rc = getattr(load(), name)(_ptr(a), _ptr(a_s), _ptr(w), _ptr(w_s), _ptr(group_list), group_list_type, M, N, Kd,
                               E, _ptr(out), _stream(stream))
    _check(rc, name)
    return out


@_stream_scoped
def moe_finalize(y, topk_w, expanded_row_idx, out=None, stream=None):
    """Weighted un-permute and sum: out [T, K] bf16."""
    _need(y, torch.bfloat16, "y", 2); _need(topk_w, torch.float32, "topk_w", 2)
    _need(expanded_row_idx, torch.int32, "expanded_row_idx")
    M, K = y.shape
    T, k = topk_w.shape
    dev = y.device
    _need_shape(y, (M, K), "y", torch.bfloat16, dev)
    _need_shape(topk_w, (T, k), "topk_w", torch.float32, dev)
    if expanded_row_idx.numel() != T * k:
        raise ValueError(f"expanded_row_idx must hold T*k = {T * k} entries, got {expanded_row_idx.numel()}")
    _need_shape(expanded_row_idx, tuple(expanded_row_idx.shape), "expanded_row_idx", torch.int32, dev)
    if out is None:
        out = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    _need_shape(out, (T, K), "out", torch.bfloat16, dev)
    _need_gpu(y, "y")
    rc = load().moe_finalize(_ptr(y), _ptr(topk_w), _ptr(expanded_row_idx), T, K, k, M, _ptr(out),
                             _stream(stream))
    _check(rc, "moe_finalize")
    return out


def forward_workspace_size(T, K, I, E, k):
    return int(load().moe_mxfp8_forward_workspace_size(T, K, I, E, k))


def forward_workspace(T, K, I, E, k, device="cuda"):
    return torch.empty(max(forward_workspace_size(T, K, I, E, k), 256), dtype=torch.uint8, device=device)


@_stream_scoped
def moe_mxfp8_forward(x, topk_ids, topk_w, w13, w13_s, w2, w2_s, out=None, workspace=None, stream=None,
                      _w4=False, _packed=False):
    """The whole layer.  x [T,K] bf16, topk_ids [T,k] i32, topk_w [T,k] f32,
    w13 [E,2I,K] u8 + w13_s [E,2I,K/64,2], w2 [E,K,I] u8 + w2_s [E,K,I/64,2].
    Returns out [T,K] bf16."""
    _need(x, torch.bfloat16, "x", 2); _need(topk_ids, torch.int32, "topk_ids", 2)
    _need(w13, torch.uint8, "w13", 3)
    T, K = x.shape
    k = topk_ids.shape[1]
    E, twoI, Kw = w13.shape
    Kb = K // 2 if _w4 else K
    if Kw != Kb or twoI % 2:
        raise ValueError(f"w13 must be [E, 2I, {Kb}], got {tuple(w13.shape)}")
    I = twoI // 2
    dev = x.device
    _need_shape(x, (T, K), "x", torch.bfloat16, dev)
    _need_shape(topk_ids, (T, k), "topk_ids", torch.int32, dev)
    _need_shape(topk_w, (T, k), "topk_w", torch.float32, dev)
    _need_shape(w13, (E, twoI, Kb), "w13", torch.uint8, dev)
    _need_shape(w13_s, (E, twoI, _pairs(K), 2), "w13_s", torch.uint8, dev)
    _need_shape(w2, (E, K, I // 2 if _w4 else I), "w2", torch.uint8, dev)
    _need_shape(w2_s, (E, K, _pairs(I), 2), "w2_s", torch.uint8, dev)
    if out is None:
        out = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    _need_shape(out, (T, K), "out", torch.bfloat16, dev)
    need = forward_workspace_size(T, K, I, E, k)
    if workspace is None:
        workspace = forward_workspace(T, K, I, E, k, dev)
    _need_workspace(workspace, need, dev)
    _need_gpu(x, "x")
    name = "moe_w4a8_forward" if _w4 else "moe_mxfp8_forward_packed" if _packed else "moe_mxfp8_forward"
    rc = getattr(load(), name)(_ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w13), _ptr(w13_s), _ptr(w2), _ptr(w2_s),
                               T, K, I, E, k, _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, name)
    return out


def forward_intermediates(workspace, T, K, I, E, k):
    """Views of the intermediates a forward call left in its workspace:
    dict(xq, xs, sorted_row, expanded_row_idx, group_list, hq, hs, y)."""
    offs = (ctypes.c_size_t * 8)()
    _check(load().moe_mxfp8_forward_workspace_layout(T, K, I, E, k, offs), "workspace_layout")
    M = T * k

    def view(i, n, dtype):
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return workspace[offs[i]:offs[i] + nbytes].view(dtype)

    return dict(
        xq=view(0, M * K, torch.uint8).view(M, K),
        xs=view(1, M * _pairs(K) * 2, torch.uint8).view(M, _pairs(K), 2),
        sorted_row=view(2, M, torch.int32),
        expanded_row_idx=view(3, M, torch.int32),
        group_list=view(4, E, torch.int64),
        hq=view(5, M * I, torch.uint8).view(M, I),
        hs=view(6, M * _pairs(I) * 2, torch.uint8).view(M, _pairs(I), 2),
        y=view(7, M * K, torch.bfloat16).view(M, K),
    )


@_stream_scoped
def moe_router(x, gate, k, bias=None, renormalize=True, out=None, stream=None):
    """Top-k softmax router: x [T,K] bf16, gate [E,K] bf16, optional bias [E]
    fp32.  Returns (topk_ids [T,k] int32, topk_w [T,k] float32)."""
    _need(x, torch.bfloat16, "x", 2); _need(gate, torch.bfloat16, "gate", 2)
    T, K = x.shape
    E = gate.shape[0]
    dev = x.device
    _need_shape(x, (T, K), "x", torch.bfloat16, dev)
    _need_shape(gate, (E, K), "gate", torch.bfloat16, dev)
    if bias is not None:
        _need_shape(bias, (E,), "bias", torch.float32, dev)
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev))
    ids, w = out
    _need_shape(ids, (T, k), "topk_ids", torch.int32, dev)
    _need_shape(w, (T, k), "topk_w", torch.float32, dev)
    _need_gpu(x, "x")
    rc = load().moe_router(_ptr(x), _ptr(gate), _ptr(bias), T, K, E, k, 1 if renormalize else 0, _ptr(ids), _ptr(w),
                           _stream(stream))
    _check(rc, "moe_router")
    return ids, w


def linear_workspace_size(T, K):
    return int(load().mx_linear_workspace_size(T, K))


@_stream_scoped
def mx_linear(x, w, w_s, out=None, workspace=None, stream=None):
    """Dense MXFP8 linear: x [T,K] bf16, w [N,K] e4m3 bytes, w_s [N,K/64,2]
    e8m0 bytes (as mx_quantize makes them).  Returns y [T,N] bf16."""
    _need(x, torch.bfloat16, "x", 2); _need(w, torch.uint8, "w", 2)
    T, K = x.shape
    N = w.shape[0]
    dev = x.device
    _need_shape(x, (T, K), "x", torch.bfloat16, dev)
    _need_shape(w, (N, K), "w", torch.uint8, dev)
    _need_shape(w_s, (N, _pairs(K), 2), "w_s", torch.uint8, dev)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    _need_shape(out, (T, N), "out", torch.bfloat16, dev)
    need = linear_workspace_size(T, K)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need_workspace(workspace, need, dev)
    _need_gpu(x, "x")
    if workspace.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")
    rc = load().mx_linear(_ptr(x), _ptr(w), _ptr(w_s), T, K, N, _ptr(out), _ptr(workspace), workspace.numel(),
                          _stream(stream))
    _check(rc, "mx_linear")
    return out


@_stream_scoped
def mx_quantize_fp4(x, q=None, s=None, stream=None):
    """MXFP4-quantise the last dim of a bf16 tensor [..., Kd] (Kd % 32 == 0).
    Returns (q uint8 [..., Kd/2] packed e2m1, s uint8 [..., ceil(Kd/64), 2])."""
    _need(x, torch.bfloat16, "x")
    kd = x.shape[-1]
    lead = tuple(x.shape[:-1])
    x2 = x.reshape(-1, kd) if x.dim() != 2 else x
    if x2.stride(-1) != 1:
        raise ValueError("x must have unit stride along the last dim")
    if kd % 2:
        raise ValueError("Kd must be even (two codes per byte)")
    rows = x2.shape[0]
    if q is None:
        q = torch.empty(lead + (kd // 2,), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(lead + (_pairs(kd), 2), dtype=torch.uint8, device=x.device)
    _need_shape(q, lead + (kd // 2,), "q", torch.uint8, x.device)
    _need_shape(s, lead + (_pairs(kd), 2), "s", torch.uint8, x.device)
    ld = x2.stride(0) if rows > 1 else kd
    _need_gpu(x, "x")
    rc = load().mx_quantize_fp4(_ptr(x2), rows, kd, ld, _ptr(q), _ptr(s), _stream(stream))
    _check(rc, "mx_quantize_fp4")
    return q, s


@_stream_scoped
def gmm_swiglu_mxquant_w4a8(a, a_s, w13, w13_s, group_list, group_list_type=GROUP_COUNT, out=None,
                            h_debug=False, stream=None):
    """GEMM1 + SwiGLU + MX requant with MXFP4 weights: w13 [E, 2I, K/2] packed
    e2m1 + w13_s [E, 2I, K/64, 2].  Returns (hq, hs) (MXFP8) or (hq, hs, h)."""
    return gmm_swiglu_mxquant(a, a_s, w13, w13_s, group_list, group_list_type, out, h_debug, stream, _w4=True)


@_stream_scoped
def gmm_mx_w4a8(a, a_s, w, w_s, group_list, group_list_type=GROUP_COUNT, out=None, stream=None):
    """Grouped MX GEMM with MXFP4 weights (w [E, N, Kd/2] packed e2m1), bf16 [M, N]."""
    return gmm_mx(a, a_s, w, w_s, group_list, group_list_type, out, stream, _w4=True)


@_stream_scoped
def moe_w4a8_forward(x, topk_ids, topk_w, w13, w13_s, w2, w2_s, out=None, workspace=None, stream=None):
    """The layer with MXFP4 expert weights: w13 [E,2I,K/2], w2 [E,K,I/2] packed e2m1."""
    return moe_mxfp8_forward(x, topk_ids, topk_w, w13, w13_s, w2, w2_s, out, workspace, stream, _w4=True)


PACK_GEMM2 = 0   # mx_pack_weights kind: plain weight rows (w2, the dense linear)
PACK_GEMM1 = 1   # mx_pack_weights kind: w13, gate rows then up rows


@_stream_scoped
def mx_pack_weights(w, kind, out=None, stream=None):
    """e4m3 expert weights w [E, N, Kd] uint8 -> the tile-packed layout the
    *_packed GEMMs read (same shape and size; see include/mxmoe.h).
    kind: PACK_GEMM1 for w13 [E, 2I, K], PACK_GEMM2 for w2 [E, K, I]."""
    _need(w, torch.uint8, "w", 3)
    E, N, Kd = w.shape
    if out is None:
        out = torch.empty_like(w)
    _need_shape(w, (E, N, Kd), "w", torch.uint8, w.device)
    _need_shape(out, (E, N, Kd), "out", torch.uint8, w.device)
    _need_gpu(w, "w")
    rc = load().mx_pack_weights(_ptr(w), E, N, Kd, int(kind), _ptr(out), _stream(stream))
    _check(rc, "mx_pack_weights")
    return out


def gmm_swiglu_mxquant_packed(a, a_s, w13_packed, w13_s, group_list, group_list_type=GROUP_COUNT, out=None,
                              h_debug=False, stream=None):
    """gmm_swiglu_mxquant with w13 tile-packed (mx_pack_weights, PACK_GEMM1)."""
    return gmm_swiglu_mxquant(a, a_s, w13_packed, w13_s, group_list, group_list_type, out, h_debug, stream,
                              _packed=True)


def gmm_mx_packed(a, a_s, w_packed, w_s, group_list, group_list_type=GROUP_COUNT, out=None, stream=None):
    """gmm_mx with w tile-packed (mx_pack_weights, PACK_GEMM2)."""
    return gmm_mx(a, a_s, w_packed, w_s, group_list, group_list_type, out, stream, _packed=True)


def moe_mxfp8_forward_packed(x, topk_ids, topk_w, w13_packed, w13_s, w2_packed, w2_s, out=None, workspace=None,
                             stream=None):
    """moe_mxfp8_forward with w13 and w2 tile-packed by mx_pack_weights."""
    return moe_mxfp8_forward(x, topk_ids, topk_w, w13_packed, w13_s, w2_packed, w2_s, out, workspace, stream,
                             _packed=True)
