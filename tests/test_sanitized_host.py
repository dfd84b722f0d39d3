"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

`lamp_api.cpp` (argument checks, size arithmetic, workspace bookkeeping,
error paths) is compiled with both sanitizers on its host side only (every
-fsanitize flag sits behind -Xarch_host; device code is built as usual), the
quantisation, decode and statistics sources as usual, and the attention
kernel's two launchers as stubs.  A child process with the sanitizer
runtime preloaded loads that library through ctypes and drives every entry
point with invalid arguments (zero, negative and INT_MAX sizes, products
past 2^31, null and misaligned pointers, bad flags, NaN parameters) and with
valid ones, which end in a HIP error on this host without a GPU.  Any
sanitizer report, crash or undocumented return code fails the test.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_attention_lamp_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
RUNTIMES = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

BASE = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and RUNTIMES),
                                reason="hipcc or the sanitizer runtime is not installed")


def _compile(args):
    src, obj, extra = args
    r = subprocess.run([HIPCC, *BASE, *extra, "-x", "hip", "-c", src, "-o", obj],
                       capture_output=True, text=True)
    return src, r.returncode, r.stderr


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitized")
    jobs = [(os.path.join(CSRC, "lamp_api.cpp"), str(d / "api.o"), HOST_SAN)]
    for name in ("quant.hip", "decode.hip", "stats.hip"):
        jobs.append((os.path.join(CSRC, name), str(d / (name + ".o")), ["-fno-honor-nans"]))
    jobs.append((os.path.join(HERE, "attn_stub.hip"), str(d / "attn_stub.o"), []))
    with ThreadPoolExecutor(4) as ex:
        for src, rc, err in ex.map(_compile, jobs):
            noise = "is not a recognized feature"
            assert rc == 0, f"{src}:\n" + "\n".join(l for l in err.splitlines() if noise not in l)
    lib = str(d / "liblamp_sanitized.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[j[1] for j in jobs],
                        "-Xarch_host", "-shared-libsan", "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


def test_entry_points_under_sanitizers(sanitized_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = RUNTIMES[-1]
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    env["HIP_VISIBLE_DEVICES"] = ""          # host path only, also where a GPU exists
    r = subprocess.run([sys.executable, os.path.join(HERE, "drive_abi.py"), sanitized_lib],
                       capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "driven: all entry points" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
