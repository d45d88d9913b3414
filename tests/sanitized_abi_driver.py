"""Runs inside a process that preloads the sanitizer runtime and loads the
host-sanitised libmxmoe (see sanitized_build.py): calls every entry point
and size query with arguments its host checks must reject -- null pointers,
zero and negative sizes, sizes at and past every limit, int64 extremes --
and checks the returned status.  Nothing reaches the GPU: every call fails
validation first.  A sanitizer finding aborts the process."""

import ctypes
import sys
import threading

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
F = ctypes.c_void_p(0x1000)        # never dereferenced
BIG = [1 << 31, (1 << 31) + 7, 1 << 40, 1 << 62, (1 << 63) - 1]
NEG = [-1, -(1 << 31), -(1 << 63)]

lib = ctypes.CDLL(sys.argv[1])
SIG = {
    "mx_quantize": (I32, [P, I64, I64, I64, P, P, P]),
    "mx_quantize_fp4": (I32, [P, I64, I64, I64, P, P, P]),
    "moe_route_quant_workspace_size": (SZ, [I64, I64, I64]),
    "moe_route_quant": (I32, [P, P, I64, I64, I64, I64, P, P, P, P, P, P, SZ, P]),
    "moe_route_quant_noalloc": (I32, [P, P, I64, I64, I64, I64, P, P, P, P, P, P]),
    "gmm_swiglu_mxquant": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P, P, P]),
    "gmm_swiglu_mxquant_w4a8": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P, P, P]),
    "gmm_mx": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P]),
    "gmm_mx_w4a8": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P]),
    "moe_finalize": (I32, [P, P, P, I64, I64, I64, I64, P, P]),
    "moe_mxfp8_forward_workspace_size": (SZ, [I64, I64, I64, I64, I64]),
    "moe_mxfp8_forward_workspace_layout": (I32, [I64, I64, I64, I64, I64, P]),
    "moe_mxfp8_forward": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
    "moe_w4a8_forward": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
    "moe_router": (I32, [P, P, P, I64, I64, I64, I64, I32, P, P, P]),
    "mx_linear_workspace_size": (SZ, [I64, I64]),
    "mx_linear": (I32, [P, P, P, I64, I64, I64, P, P, SZ, P]),
    "mx_pack_weights": (I32, [P, I64, I64, I64, I32, P, P]),
    "gmm_mx_packed": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P]),
    "gmm_swiglu_mxquant_packed": (I32, [P, P, P, P, P, I32, I64, I64, I64, I64, P, P, P, P]),
    "moe_mxfp8_forward_packed": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P, SZ, P]),
    "mx_last_error": (ctypes.c_char_p, []),
}
for name, (res, args) in SIG.items():
    fn = getattr(lib, name)
    fn.restype, fn.argtypes = res, args

n = 0


def expect(got, want, what):
    global n
    n += 1
    if isinstance(want, tuple):
        ok = got in want
    else:
        ok = got == want
    if not ok:
        sys.exit(f"{what}: got {got}, want {want} ({lib.mx_last_error()!r})")


def err():
    return lib.mx_last_error().decode()


# ---- quantisers -----------------------------------------------------------
for fn in (lib.mx_quantize, lib.mx_quantize_fp4):
    expect(fn(None, 4, 64, 64, F, F, None), INVALID, "quant null x")
    expect(fn(F, 4, 64, 64, None, F, None), INVALID, "quant null q")
    for v in NEG:
        expect(fn(F, v, 64, 64, F, F, None), INVALID, f"quant rows {v}")
        expect(fn(F, 4, v, 64, F, F, None), INVALID, f"quant kd {v}")
        expect(fn(F, 4, 64, v, F, F, None), INVALID, f"quant ld {v}")
    expect(fn(F, 4, 64, 32, F, F, None), INVALID, "quant ld < kd")
    for v in BIG:
        expect(fn(F, v, 64, 64, F, F, None), UNSUPPORTED, f"quant rows {v}")
        expect(fn(F, 4, 64, v, F, F, None), UNSUPPORTED, f"quant ld {v}")
        expect(fn(F, 4, v, v, F, F, None), UNSUPPORTED, f"quant kd=ld {v}")
expect(lib.mx_quantize_fp4(F, 4, 48, 48, F, F, None), UNSUPPORTED, "fp4 kd % 32")

# ---- routing ------------------------------------------------------------
for fn, ws in ((lib.moe_route_quant, True), (lib.moe_route_quant_noalloc, False)):
    def call(T, K, k, E, wsb=1 << 40, x=F, gl=F):
        if ws:
            return fn(x, F, T, K, k, E, F, F, F, F, gl, F, wsb, None)
        return fn(x, F, T, K, k, E, F, F, F, F, gl, None)
    expect(call(64, 256, 9, 8), INVALID, "route k > E")
    expect(call(64, 256, 0, 8), INVALID, "route k = 0")
    expect(call(64, 256, 2, 0), INVALID, "route E = 0")
    expect(call(64, 0, 2, 8), INVALID, "route K = 0")
    expect(call(64, 256, 2, 8, x=None), INVALID, "route null x")
    expect(call(64, 256, 2, 8, gl=None), INVALID, "route null group_list")
    for v in NEG:
        expect(call(v, 256, 2, 8), INVALID, f"route T {v}")
        expect(call(64, v, 2, 8), INVALID, f"route K {v}")
        expect(call(64, 256, v, 8), INVALID, f"route k {v}")
        expect(call(64, 256, 2, v), INVALID, f"route E {v}")
    for v in BIG:
        expect(call(v, 256, 2, 8), UNSUPPORTED, f"route T {v}")
        expect(call(64, v, 2, 8), UNSUPPORTED, f"route K {v}")
        expect(call(64, 256, 2, v), UNSUPPORTED, f"route E {v}")
        expect(call(64, 256, v, v), UNSUPPORTED, f"route k=E {v}")
    expect(call(64, 100, 2, 8), UNSUPPORTED, "route K % 32")
    expect(call(64, 256, 300, 400), UNSUPPORTED, "route k > 256")
    expect(call((1 << 31) // 8, 256, 8, 16), UNSUPPORTED, "route T*k = 2^31")
    expect(call((1 << 27) // 8 + 1, 256, 8, 16), UNSUPPORTED, "route T*k above 2^27")
    if ws:
        expect(call(300, 256, 2, 8, wsb=0), WORKSPACE, "route workspace 0")
    else:
        expect(call(32768, 256, 8, 1024), UNSUPPORTED, "noalloc past its scratch")
        assert "routing scratch" in err()
q = lib.moe_route_quant_workspace_size
expect(q(300, 2, 8) > 0, True, "route ws query valid")
expect(q(128, 2, 8), 0, "route ws query one chunk")
for v in NEG + BIG:
    expect(q(v, 2, 8), 0, f"route ws query T {v}")
    expect(q(64, v, 8), 0, f"route ws query k {v}")
    expect(q(64, 2, v), 0, f"route ws query E {v}")

# ---- grouped GEMMs --------------------------------------------------------
for fn in (lib.gmm_mx, lib.gmm_mx_w4a8, lib.gmm_mx_packed):
    def call(M, N, Kd, E, t=1, gl=F, a=F):
        return fn(a, F, F, F, gl, t, M, N, Kd, E, F, None)
    expect(call(64, 256, 256, 4, t=2), INVALID, "gmm group_list_type 2")
    expect(call(64, 256, 256, 4, t=-1), INVALID, "gmm group_list_type -1")
    expect(call(64, 256, 256, 4, gl=None), INVALID, "gmm null group list")
    expect(call(64, 256, 256, 4, a=None), INVALID, "gmm null a")
    expect(call(64, 0, 256, 4), INVALID, "gmm N = 0")
    for v in NEG:
        expect(call(v, 256, 256, 4), INVALID, f"gmm M {v}")
        expect(call(64, v, 256, 4), INVALID, f"gmm N {v}")
        expect(call(64, 256, v, 4), INVALID, f"gmm Kd {v}")
        expect(call(64, 256, 256, v), INVALID, f"gmm E {v}")
    for v in BIG:
        expect(call(v, 256, 256, 4), UNSUPPORTED, f"gmm M {v}")
        expect(call(64, v, 256, 4), UNSUPPORTED, f"gmm N {v}")
        expect(call(64, 256, v, 4), UNSUPPORTED, f"gmm Kd {v}")
        expect(call(64, 256, v // 128 * 128, 4), UNSUPPORTED, f"gmm Kd {v} rounded")
        expect(call(64, 256, 256, v), UNSUPPORTED, f"gmm E {v}")
    expect(call(64, 256, 200, 4), UNSUPPORTED, "gmm Kd % 128")
    expect(call(64, 200, 256, 4), UNSUPPORTED, "gmm N % 256")
    expect(call(64, 256, 256, 1025), UNSUPPORTED, "gmm E > 1024")
    expect(call(64, 256, (1 << 20) + 128, 4), UNSUPPORTED, "gmm Kd past 2^20")
for fn in (lib.gmm_swiglu_mxquant, lib.gmm_swiglu_mxquant_w4a8, lib.gmm_swiglu_mxquant_packed):
    def call(M, K, I, E, t=1, hq=F):
        return fn(F, F, F, F, F, t, M, K, I, E, hq, F, None, None)
    expect(call(64, 256, 128, 4, hq=None), INVALID, "gmm1 null hq")
    expect(call(64, 256, 0, 4), INVALID, "gmm1 I = 0")
    for v in NEG:
        expect(call(64, 256, v, 4), INVALID, f"gmm1 I {v}")
    for v in BIG:
        expect(call(64, 256, v, 4), UNSUPPORTED, f"gmm1 I {v}")
        expect(call(64, 256, v // 128 * 128, 4), UNSUPPORTED, f"gmm1 I {v} rounded")
        expect(call(v, 256, 128, 4), UNSUPPORTED, f"gmm1 M {v}")
    expect(call(64, 256, 100, 4), UNSUPPORTED, "gmm1 I % 128")

# ---- finalize -------------------------------------------------------------
fz = lib.moe_finalize
expect(fz(F, None, F, 4, 64, 2, 8, F, None), INVALID, "finalize null w")
for v in NEG:
    expect(fz(F, F, F, v, 64, 2, 8, F, None), INVALID, f"finalize T {v}")
    expect(fz(F, F, F, 4, v, 2, 8, F, None), INVALID, f"finalize K {v}")
    expect(fz(F, F, F, 4, 64, v, 8, F, None), INVALID, f"finalize k {v}")
    expect(fz(F, F, F, 4, 64, 2, v, F, None), INVALID, f"finalize M {v}")
for v in BIG:
    expect(fz(F, F, F, v, 64, 2, 8, F, None), UNSUPPORTED, f"finalize T {v}")
    expect(fz(F, F, F, 4, v // 8 * 8, 2, 8, F, None), UNSUPPORTED, f"finalize K {v}")
    expect(fz(F, F, F, 4, 64, v, 8, F, None), UNSUPPORTED, f"finalize k {v}")
    expect(fz(F, F, F, 4, 64, 2, v, F, None), UNSUPPORTED, f"finalize M {v}")
expect(fz(F, F, F, 4, 60, 2, 8, F, None), UNSUPPORTED, "finalize K % 8")

# ---- forward --------------------------------------------------------------
for fn in (lib.moe_mxfp8_forward, lib.moe_w4a8_forward, lib.moe_mxfp8_forward_packed):
    def call(T, K, I, E, k, wsb=1 << 40, ws=F, out=F):
        return fn(F, F, F, F, F, F, F, T, K, I, E, k, out, ws, wsb, None)
    expect(call(64, 256, 128, 8, 2, ws=None), INVALID, "forward null workspace")
    expect(call(64, 256, 128, 8, 2, out=None), INVALID, "forward null out")
    expect(call(64, 256, 128, 8, 2, wsb=0), WORKSPACE, "forward workspace 0")
    expect(call(64, 256, 128, 8, 9), INVALID, "forward k > E")
    for v in NEG:
        for i in range(5):
            a = [64, 256, 128, 8, 2]
            a[i] = v
            expect(call(*a), INVALID, f"forward arg {i} = {v}")
    for v in BIG:
        for i in range(5):
            a = [64, 256, 128, 8, 2]
            a[i] = v
            expect(call(*a), (INVALID, UNSUPPORTED), f"forward arg {i} = {v}")
    expect(call(64, 128, 128, 8, 2), UNSUPPORTED, "forward K % 256")
    expect(call(64, 256, 64, 8, 2), UNSUPPORTED, "forward I % 128")
fq = lib.moe_mxfp8_forward_workspace_size
expect(fq(64, 256, 128, 8, 2) > 0, True, "forward ws query valid")
offs = (ctypes.c_size_t * 8)()
for v in NEG + BIG:
    for i in range(5):
        a = [64, 256, 128, 8, 2]
        a[i] = v
        expect(fq(*a), 0, f"forward ws query arg {i} = {v}")
        expect(lib.moe_mxfp8_forward_workspace_layout(*a, offs), (INVALID, UNSUPPORTED), f"layout arg {i} = {v}")

# ---- weight packing ---------------------------------------------------------
pk = lib.mx_pack_weights
G = ctypes.c_void_p(0x10000000)
expect(pk(None, 2, 256, 128, 0, G, None), INVALID, "pack null w")
expect(pk(F, 2, 256, 128, 3, G, None), INVALID, "pack kind")
for v in NEG:
    expect(pk(F, v, 256, 128, 0, G, None), INVALID, f"pack E {v}")
    expect(pk(F, 2, v, 128, 0, G, None), INVALID, f"pack N {v}")
    expect(pk(F, 2, 256, v, 0, G, None), INVALID, f"pack Kd {v}")
for v in BIG:
    expect(pk(F, v, 256, 128, 0, G, None), UNSUPPORTED, f"pack E {v}")
    expect(pk(F, 2, v // 256 * 256, 128, 1, G, None), UNSUPPORTED, f"pack N {v}")
    expect(pk(F, 2, 256, v // 128 * 128, 0, G, None), UNSUPPORTED, f"pack Kd {v}")
expect(pk(F, 2, 256, 128, 0, ctypes.c_void_p(0x1000 + 64), None), INVALID, "pack overlap")

# ---- router ---------------------------------------------------------------
rt = lib.moe_router
expect(rt(None, F, None, 64, 256, 8, 2, 1, F, F, None), INVALID, "router null x")
expect(rt(F, F, None, 64, 256, 8, 9, 1, F, F, None), INVALID, "router k > E")
for v in NEG:
    expect(rt(F, F, None, v, 256, 8, 2, 1, F, F, None), INVALID, f"router T {v}")
    expect(rt(F, F, None, 64, v, 8, 2, 1, F, F, None), INVALID, f"router K {v}")
for v in BIG:
    expect(rt(F, F, None, v, 256, 8, 2, 1, F, F, None), UNSUPPORTED, f"router T {v}")
    expect(rt(F, F, None, 64, v // 64 * 64, 8, 2, 1, F, F, None), UNSUPPORTED, f"router K {v}")
    expect(rt(F, F, None, 64, 256, v, 2, 1, F, F, None), UNSUPPORTED, f"router E {v}")

# ---- dense linear -----------------------------------------------------------
ln = lib.mx_linear
expect(ln(F, F, F, 64, 256, 256, F, None, 1 << 40, None), INVALID, "linear null workspace")
expect(ln(F, F, F, 64, 256, 256, F, F, 0, None), WORKSPACE, "linear workspace 0")
for v in NEG:
    expect(ln(F, F, F, v, 256, 256, F, F, 1 << 40, None), INVALID, f"linear T {v}")
    expect(ln(F, F, F, 64, 256, v, F, F, 1 << 40, None), INVALID, f"linear N {v}")
for v in BIG:
    expect(ln(F, F, F, v, 256, 256, F, F, 1 << 40, None), UNSUPPORTED, f"linear T {v}")
    expect(ln(F, F, F, 64, v // 128 * 128, 256, F, F, 1 << 40, None), UNSUPPORTED, f"linear K {v}")
    expect(ln(F, F, F, 64, 256, v // 256 * 256, F, F, 1 << 40, None), UNSUPPORTED, f"linear N {v}")
lq = lib.mx_linear_workspace_size
expect(lq(64, 256) > 0, True, "linear ws query valid")
for v in NEG + BIG:
    expect(lq(v, 256), 0, f"linear ws query T {v}")
    expect(lq(64, v), 0, f"linear ws query K {v}")

# ---- error text is per thread ------------------------------------------------
seen = {}


def worker(i):
    for _ in range(200):
        lib.mx_quantize(F, 4, 64, 32 - i, F, F, None)
        seen[i] = err()


threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
for t in threads:
    t.start()
for t in threads:
    t.join()
for i in range(4):
    assert f"ld={32 - i}" in seen[i], seen[i]

print(f"OK {n} checks")
