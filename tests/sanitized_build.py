"""Host-sanitised build of libmxmoe.so for the CPU tests (not the product).

Every source is compiled as in the product build, with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (device code is built as
usual), and linked by clang++ against the HIP runtime with the shared
sanitizer runtime.  A process that loads the result must preload that
runtime (``asan_runtime()``).  The library lands in _build/san/ and is
rebuilt when a source is newer than it.
"""

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from mxfp8_block_scaled_topk_amd import build as product  # noqa: E402

OUT = os.path.join(ROOT, "_build", "san")
LIB = os.path.join(OUT, "libmxmoe_san.so")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
# host-only sanitiser flags for hipcc (each directly after -Xarch_host)
HOST_SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer -Xarch_host -g").split()


def asan_runtime():
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = hits[0] if hits else ""
    return path


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    flags = [f for f in product.CFLAGS if f != "-O3"] + ["-O1"] + HOST_SAN
    r = subprocess.run([product.HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build():
    srcs = sorted(glob.glob(os.path.join(product.CSRC, "*.hip")))
    deps = srcs + glob.glob(os.path.join(product.CSRC, "*.h")) + [os.path.join(ROOT, "include", "mxmoe.h")]
    if os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(d) for d in deps):
        return LIB
    os.makedirs(OUT, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    link = [CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", *objs,
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", LIB + ".tmp"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())
