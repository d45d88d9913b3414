"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): a host-sanitised build of the library
(tests/sanitized_build.py) runs tests/sanitized_abi_driver.py, which calls
every entry point and size query with arguments it must reject, in a child
process that preloads the sanitizer runtime.  Any sanitizer finding (an
out-of-bounds access, a signed overflow in size arithmetic, ...) aborts the
child and fails the test."""

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(600)
def test_validation_layer_is_clean_under_sanitizers():
    import sanitized_build
    rt = sanitized_build.asan_runtime()
    if not rt:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = sanitized_build.build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitized_abi_driver.py"), lib], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    assert r.stdout.startswith("OK "), r.stdout
