"""C ABI checks that need no GPU: the library loads, exports every function
include/mxmoe.h declares, and rejects bad arguments on the host with the
documented status codes before anything is enqueued."""

import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_topk_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxmoe.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.lib_path()):
        pytest.fail("libmxmoe.so is not built (run python -m mxfp8_block_scaled_topk_amd.build)")
    return mx.load()


def test_header_declares_the_six_entry_points():
    names = declared_functions()
    for n in ["mx_quantize", "moe_route_quant", "gmm_swiglu_mxquant", "gmm_mx", "moe_finalize",
              "moe_mxfp8_forward", "mx_last_error"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in mxmoe.h but not exported"


def test_workspace_queries(lib):
    assert mx.route_workspace_size(16384, 8, 128) > 0
    ws = mx.forward_workspace_size(16384, 2048, 768, 128, 8)
    M = 16384 * 8
    assert ws >= M * 2048 + M * 768 + M * 2048 * 2       # xq + hq + y at least
    assert mx.forward_workspace_size(-1, 2048, 768, 128, 8) == 0
    offs = (ctypes.c_size_t * 8)()
    assert lib.moe_mxfp8_forward_workspace_layout(64, 256, 128, 8, 2, offs) == OK
    assert list(offs) == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lib.moe_mxfp8_forward_workspace_layout(64, 256, 128, 8, 2, None) == INVALID


def test_mx_quantize_validation(lib):
    assert lib.mx_quantize(None, 4, 64, 64, FAKE, FAKE, None) == INVALID
    assert "null" in mx.last_error()
    assert lib.mx_quantize(FAKE, 4, 0, 64, FAKE, FAKE, None) == INVALID
    assert lib.mx_quantize(FAKE, 4, 64, 32, FAKE, FAKE, None) == INVALID   # ld < kd
    assert lib.mx_quantize(FAKE, -1, 64, 64, FAKE, FAKE, None) == INVALID


def test_route_validation(lib):
    f = lib.moe_route_quant
    args = lambda T, K, k, E, ws=1 << 20: f(FAKE, FAKE, T, K, k, E, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert args(64, 256, 9, 8) == INVALID          # k > E
    assert args(64, 256, 0, 8) == INVALID
    assert args(64, 100, 2, 8) == UNSUPPORTED      # K % 32
    assert args(64, 256, 2, 2048) == UNSUPPORTED   # E > 1024
    assert args(64, 256, 300, 400) == UNSUPPORTED  # k > 256
    assert args(300, 256, 2, 8, ws=0) == WORKSPACE   # 600 assignments: 3 routing chunks
    assert "workspace" in mx.last_error()
    assert f(None, FAKE, 64, 256, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == INVALID



def test_route_noalloc_validation(lib):
    """The allocation-free routing entry point checks the same arguments and
    rejects sizes whose routing scratch exceeds the 4 MiB it holds, all on
    the host (no GPU is touched)."""
    f = lib.moe_route_quant_noalloc
    args = lambda T, K, k, E: f(FAKE, FAKE, T, K, k, E, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert args(64, 256, 9, 8) == INVALID
    assert args(64, 100, 2, 8) == UNSUPPORTED
    assert args(64, 256, 2, 2048) == UNSUPPORTED
    assert f(None, FAKE, 64, 256, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 64, 256, 2, 8, FAKE, FAKE, FAKE, FAKE, None, None) == INVALID
    # E = 1024, top-8: 4 KB of counts per 32-token routing chunk, plus the
    # control block, the super-chunk totals (128 KB) and flags: 991 chunks fit in 4 MiB
    assert mx.route_workspace_size(31712, 8, 1024) <= 4 << 20 < mx.route_workspace_size(31713, 8, 1024)
    assert args(31713, 256, 8, 1024) == UNSUPPORTED
    assert "routing scratch" in mx.last_error()
    assert mx.route_workspace_size(261056, 8, 128) <= 4 << 20 < mx.route_workspace_size(261057, 8, 128)


def test_pack_validation(lib):
    f = lib.mx_pack_weights
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p]
    other = ctypes.c_void_p(0x10000000)
    assert f(None, 2, 256, 128, 0, other, None) == INVALID
    assert f(FAKE, 0, 256, 128, 0, other, None) == INVALID
    assert f(FAKE, 2, 256, 128, 2, other, None) == INVALID          # kind
    assert f(FAKE, 2, 200, 128, 0, other, None) == UNSUPPORTED      # N % 256
    assert f(FAKE, 2, 256, 100, 1, other, None) == UNSUPPORTED      # Kd % 128
    assert f(FAKE, 2000, 256, 128, 0, other, None) == UNSUPPORTED   # E > 1024
    assert f(FAKE, 2, 256, 128, 0, ctypes.c_void_p(0x1000 + 256 * 128), None) == INVALID   # overlap
    assert "overlap" in mx.last_error()
    assert f(ctypes.c_void_p(0x1008), 2, 256, 128, 0, other, None) == UNSUPPORTED          # alignment

def test_gmm_validation(lib):
    g = lib.gmm_mx
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, 256, 128, 4, FAKE, None) == INVALID   # bad type
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16, 128, 128, 4, FAKE, None) == UNSUPPORTED  # N % 256
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16, 256, 96, 4, FAKE, None) == UNSUPPORTED   # Kd % 128
    assert g(FAKE, FAKE, FAKE, FAKE, None, 1, 16, 256, 128, 4, FAKE, None) == INVALID     # null group list
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16, 256, 128, 0, FAKE, None) == INVALID     # E = 0
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16, 256, 128, 1025, FAKE, None) == UNSUPPORTED  # E > 1024
    s = lib.gmm_swiglu_mxquant
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16, 128, 64, 4, FAKE, FAKE, None, None) == UNSUPPORTED  # I % 128
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16, 128, 128, 1025, FAKE, FAKE, None, None) == UNSUPPORTED  # E > 1024
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 5, 16, 128, 128, 4, FAKE, FAKE, None, None) == INVALID
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 16, 128, 128, 4, None, FAKE, None, None) == INVALID


def test_finalize_validation(lib):
    f = lib.moe_finalize
    assert f(FAKE, FAKE, FAKE, 4, 100, 2, 8, FAKE, None) == UNSUPPORTED   # K % 8
    assert f(FAKE, FAKE, FAKE, 4, 128, 0, 8, FAKE, None) == INVALID
    assert f(FAKE, None, FAKE, 4, 128, 2, 8, FAKE, None) == INVALID


def test_forward_validation(lib):
    f = lib.moe_mxfp8_forward
    call = lambda T, K, I, E, k, ws=1 << 30: f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, T, K, I, E, k, FAKE, FAKE,
                                               ws, None)
    assert call(64, 256, 96, 8, 2) == UNSUPPORTED      # I % 128
    assert call(64, 384, 128, 8, 2) == UNSUPPORTED     # K % 256
    assert call(64, 200, 128, 8, 2) == UNSUPPORTED     # K % 32
    assert call(64, 256, 128, 8, 9) == INVALID         # k > E
    assert call(64, 256, 128, 8, 2, ws=16) == WORKSPACE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 256, 128, 8, 2, FAKE, None, 1 << 30, None) == INVALID


def test_error_text_is_thread_local(lib):
    import threading
    lib.mx_quantize(None, 4, 64, 64, FAKE, FAKE, None)
    seen = {}

    def other():
        seen["msg"] = mx.last_error()

    t = threading.Thread(target=other)
    t.start(); t.join()
    assert seen["msg"] == "no error"
    assert "null" in mx.last_error()


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mx, "_LIB", None)
    monkeypatch.setattr(mx, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(mx.MxError):
        mx.load()


# The binding checks every tensor's dtype, shape, contiguity and device before
# it calls the library (the library sees only pointers and sizes), with shape
# errors ahead of the GPU-residency check, so CPU tensors exercise them here.

def _u8(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.uint8)


def _gemm_args(M=16, K=128, N=256, E=4):
    import torch
    return dict(a=_u8(M, K), a_s=_u8(M, K // 64, 2), w=_u8(E, N, K), w_s=_u8(E, N, K // 64, 2),
                gl=torch.zeros(E, dtype=torch.int64))


def _raises(fn, pattern):
    with pytest.raises((ValueError, TypeError), match=pattern):
        fn()


def test_binding_gmm_shape_checks(lib):
    import torch
    g = _gemm_args()
    call = lambda **kw: mx.gmm_mx(*[kw.get(n, g[n]) for n in ("a", "a_s", "w", "w_s", "gl")],
                                  out=kw.get("out"))
    _raises(lambda: call(), "on the GPU")                                   # shapes fine, not on the GPU
    _raises(lambda: call(a_s=_u8(16, 1, 2)), "a_s must have shape")        # wrong scale columns
    _raises(lambda: call(a_s=_u8(8, 2, 2)), "a_s must have shape")         # wrong scale rows
    _raises(lambda: call(w=_u8(4, 256, 64)), "w must be")                  # K of w != K of a
    _raises(lambda: call(w_s=_u8(4, 128, 2, 2)), "w_s must have shape")
    _raises(lambda: call(gl=torch.zeros(3, dtype=torch.int64)), "group_list must have shape")
    _raises(lambda: call(gl=torch.zeros(4, dtype=torch.int32)), "group_list must be torch.int64")
    _raises(lambda: call(out=torch.empty(16, 128, dtype=torch.bfloat16)), "out must have shape")
    _raises(lambda: call(out=torch.empty(16, 256, dtype=torch.float32)), "out must be torch.bfloat16")
    _raises(lambda: call(a=_u8(16, 256)[:, ::2]), "a must be contiguous")


def test_binding_gmm_swiglu_shape_checks(lib):
    import torch
    g = _gemm_args(N=512)
    call = lambda **kw: mx.gmm_swiglu_mxquant(*[kw.get(n, g[n]) for n in ("a", "a_s", "w", "w_s", "gl")],
                                              out=kw.get("out"))
    _raises(lambda: call(), "on the GPU")
    _raises(lambda: call(w=_u8(4, 511, 128)), "w13 must be")               # odd 2I
    _raises(lambda: call(w_s=_u8(4, 512, 1, 2)), "w13_s must have shape")
    _raises(lambda: call(out=(_u8(16, 256), _u8(16, 4, 2))), "on the GPU")          # I = 256: correct
    _raises(lambda: call(out=(_u8(16, 128), _u8(16, 4, 2))), "hq must have shape")
    _raises(lambda: call(out=(_u8(16, 256), _u8(16, 3, 2))), "hs must have shape")
    _raises(lambda: call(out=(_u8(16, 512)[:, ::2], _u8(16, 4, 2))), "hq must be contiguous")


def test_binding_route_finalize_forward_shape_checks(lib):
    import torch
    T, K, k, E, I = 8, 256, 2, 4, 128
    x = torch.zeros(T, K, dtype=torch.bfloat16)
    ids = torch.zeros(T, k, dtype=torch.int32)
    _raises(lambda: mx.moe_route_quant(x, ids, E), "on the GPU")
    _raises(lambda: mx.moe_route_quant(x, ids, E, out=(_u8(T * k, K), _u8(T * k, 3, 2), ids.flatten(),
                                                       ids.flatten(), torch.zeros(E, dtype=torch.int64))),
            "xs must have shape")
    # 300 tokens x top-2: three routing chunks, so a workspace is needed
    x3, ids3 = torch.zeros(300, K, dtype=torch.bfloat16), torch.zeros(300, k, dtype=torch.int32)
    _raises(lambda: mx.moe_route_quant(x3, ids3, E, workspace=_u8(1)), "workspace has 1 bytes")
    y = torch.zeros(T * k, K, dtype=torch.bfloat16)
    tw = torch.zeros(T, k, dtype=torch.float32)
    _raises(lambda: mx.moe_finalize(y, tw, ids.flatten()), "on the GPU")
    _raises(lambda: mx.moe_finalize(y, tw, ids.flatten()[:-1]), "expanded_row_idx must hold")
    _raises(lambda: mx.moe_finalize(y, tw, ids.flatten(), out=torch.zeros(T, K // 2, dtype=torch.bfloat16)),
            "out must have shape")
    w13, w13_s = _u8(E, 2 * I, K), _u8(E, 2 * I, K // 64, 2)
    w2, w2_s = _u8(E, K, I), _u8(E, K, I // 64, 2)
    fwd = lambda **kw: mx.moe_mxfp8_forward(kw.get("x", x), kw.get("ids", ids), kw.get("tw", tw), w13, w13_s,
                                            kw.get("w2", w2), kw.get("w2_s", w2_s), workspace=kw.get("ws"))
    _raises(lambda: fwd(), "on the GPU")
    _raises(lambda: fwd(tw=torch.zeros(T, k + 1)), "topk_w must have shape")
    _raises(lambda: fwd(w2=_u8(E, K, 2 * I)), "w2 must have shape")
    _raises(lambda: fwd(w2_s=_u8(E, K, 4, 2)), "w2_s must have shape")
    _raises(lambda: fwd(ws=_u8(64)), "workspace has 64 bytes")


def test_binding_mx_quantize_output_checks(lib):
    import torch
    x = torch.zeros(4, 100, dtype=torch.bfloat16)
    _raises(lambda: mx.mx_quantize(x), "on the GPU")
    _raises(lambda: mx.mx_quantize(x, s=_u8(4, 1, 2)), "s must have shape")   # ceil(100/64) = 2 pairs
    _raises(lambda: mx.mx_quantize(x, q=_u8(4, 64)), "q must have shape")


def test_router_validation(lib):
    f = lib.moe_router
    call = lambda T, K, E, k: f(FAKE, FAKE, None, T, K, E, k, 1, FAKE, FAKE, None)
    assert call(64, 128, 8, 9) == INVALID        # k > E
    assert call(64, 128, 8, 0) == INVALID
    assert call(-1, 128, 8, 2) == INVALID
    assert call(64, 100, 8, 2) == UNSUPPORTED    # K % 64
    assert call(64, 128, 300, 2) == UNSUPPORTED  # E > 256
    assert f(None, FAKE, None, 64, 128, 8, 2, 1, FAKE, FAKE, None) == INVALID
    assert f(ctypes.c_void_p(0x1008), FAKE, None, 64, 128, 8, 2, 1, FAKE, FAKE, None) == UNSUPPORTED
    assert "aligned" in mx.last_error()


def test_binding_router_shape_checks(lib):
    import torch
    x = torch.zeros(10, 128, dtype=torch.bfloat16)
    g = torch.zeros(8, 128, dtype=torch.bfloat16)
    _raises(lambda: mx.moe_router(x, g, 2), "on the GPU")
    _raises(lambda: mx.moe_router(x, torch.zeros(8, 64, dtype=torch.bfloat16), 2), "gate must have shape")
    _raises(lambda: mx.moe_router(x, g, 2, bias=torch.zeros(7)), "bias must have shape")
    _raises(lambda: mx.moe_router(x, g, 2, bias=torch.zeros(8, dtype=torch.float64)), "bias must be torch.float32")
    _raises(lambda: mx.moe_router(x, g, 2, out=(torch.zeros(10, 3, dtype=torch.int32), torch.zeros(10, 2))),
            "topk_ids must have shape")


def test_linear_validation(lib):
    f = lib.mx_linear
    call = lambda T, K, N, ws=1 << 30: f(FAKE, FAKE, FAKE, T, K, N, FAKE, FAKE, ws, None)
    assert call(64, 96, 256) == UNSUPPORTED      # K % 128
    assert call(64, 128, 128) == UNSUPPORTED     # N % 256
    assert call(64, 128, 0) == INVALID
    assert call(-1, 128, 256) == INVALID
    assert call(64, 128, 256, ws=16) == WORKSPACE
    assert f(FAKE, None, FAKE, 64, 128, 256, FAKE, FAKE, 1 << 30, None) == INVALID
    assert mx.linear_workspace_size(64, 128) >= 64 * 128 + 64 * 4   # xq, xs
    assert mx.linear_workspace_size(-1, 128) == 0


def test_binding_linear_shape_checks(lib):
    import torch
    x = torch.zeros(10, 128, dtype=torch.bfloat16)
    w, ws = _u8(256, 128), _u8(256, 2, 2)
    _raises(lambda: mx.mx_linear(x, w, ws), "on the GPU")
    _raises(lambda: mx.mx_linear(x, _u8(256, 64), ws), "w must have shape")
    _raises(lambda: mx.mx_linear(x, w, _u8(256, 1, 2)), "w_s must have shape")
    _raises(lambda: mx.mx_linear(x, w, ws, out=torch.zeros(10, 128, dtype=torch.bfloat16)), "out must have shape")
