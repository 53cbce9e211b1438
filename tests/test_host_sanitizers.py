"""libvc's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of the library is compiled as the product build compiles it, with
the sanitizers on the host pass only (device code is built as usual), and
linked into a separate shared library in a temporary directory; a C driver
(tests/sanitize/host_checks.c) then calls every entry point with malformed,
null, empty and extreme arguments -- sizes near 2^31, counts whose sums
overflow 32 bits, out-of-range enumerators -- and checks that each call is
refused before any GPU work with a status and a message, or, for the pure
host functions, that it returns the right value.  Any sanitizer report
(overflow, invalid enum load, out-of-bounds access, leak) fails the test.
No GPU is needed: the calls that would reach a device never get past the
host checks, and the one that asks the runtime for streams (creating a
staging object) must fail cleanly without a device.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from lossless_speculative_decoding_vc_amd import build as vcbuild

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "sanitize", "host_checks.c")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

# sanitizers on the host pass only: each flag is scoped with -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
DRIVER_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _clang():
    for cand in (os.path.join(os.path.dirname(os.path.realpath(vcbuild.hipcc())), "..", "llvm", "bin", "clang"),
                 "/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            return os.path.realpath(cand)
    return None


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    try:
        hipcc = vcbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    clang = _clang()
    if clang is None:
        pytest.skip("clang not available")
    out = tmp_path_factory.mktemp("vc_san")

    def compile_one(src):
        obj = str(out / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc, *vcbuild.CFLAGS, "-g", *HOST_SAN, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, f"sanitized compile of {src} failed:\n{r.stderr[-4000:]}"
        return obj

    srcs = vcbuild.sources()
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4, 8)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(out / "libvc_san.so")
    r = subprocess.run([hipcc, f"--offload-arch={vcbuild.ARCH}", "-shared", "-fPIC", *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, "sanitized link failed:\n" + r.stderr[-4000:]
    exe = str(out / "host_checks")
    r = subprocess.run([clang, "-g", "-O1", "-Wall", "-Werror", *DRIVER_SAN, f"-I{INCLUDE}", DRIVER, "-o", exe,
                        f"-L{out}", "-lvc_san", f"-Wl,-rpath,{out}"], capture_output=True, text=True)
    assert r.returncode == 0, "driver build failed:\n" + r.stderr[-4000:]
    return exe


def test_host_code_under_sanitizers(sanitized_driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""   # the staging object must fail for want of a device
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=120)
    report = r.stdout + r.stderr
    assert "runtime error" not in report and "Sanitizer" not in report, report[-6000:]
    assert r.returncode == 0, report[-6000:]
    assert "host checks passed" in r.stdout
