"""Build liblamp.so (the gfx950 HIP kernels and the C ABI of include/lamp.h) in-tree.

    python -m mixed_precision_attention_lamp_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Every source is compiled to
an object in parallel, then linked into ``mixed_precision_attention_lamp_amd/
liblamp.so`` (replaced atomically).
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblamp.so")
# A second library for the LDS-race test: the same sources with every copy
# into LDS waited for where it is issued (and decode's stores fenced by a
# barrier); its outputs must equal liblamp.so's bit for bit.
LIB_SYNC = os.path.join(PKG, "liblamp_sync.so")
SOURCES = ["quant.hip", "attn.hip", "decode.hip", "stats.hip", "lamp_api.cpp"]
SYNC_SOURCES = ["attn.hip", "decode.hip"]
# Device sources: inputs are finite (documented in lamp.h), so max/min need no
# NaN quieting.  Not for lamp_api.cpp, whose argument checks test for NaN.
DEVICE_FLAGS = {"quant.hip": ["-fno-honor-nans"], "attn.hip": ["-fno-honor-nans"],
                "decode.hip": ["-fno-honor-nans"], "stats.hip": ["-fno-honor-nans"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src, obj, extra=()):
    cmd = [HIPCC, *FLAGS, *DEVICE_FLAGS.get(src, []), *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    return r.returncode, " ".join(cmd), err


def _link(objs, out, tmp):
    out_tmp = os.path.join(tmp, os.path.basename(out))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    shutil.copyfile(out_tmp, out + ".tmp")
    os.replace(out + ".tmp", out)


def build(verbose=False):
    """Compile every source and link liblamp.so and liblamp_sync.so; raises
    RuntimeError on failure."""
    tmp = tempfile.mkdtemp(prefix="lamp_build_")
    try:
        objs = {s: os.path.join(tmp, s + ".o") for s in SOURCES}
        sync_objs = {s: os.path.join(tmp, s + ".sync.o") for s in SYNC_SOURCES}
        jobs = [(s, objs[s], ()) for s in SOURCES] + [(s, sync_objs[s], ("-DLAMP_EXTRA_SYNC",))
                                                      for s in SYNC_SOURCES]
        with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            results = list(ex.map(lambda j: _compile(*j), jobs))
        for rc, cmd, err in results:
            if verbose or rc != 0:
                print(cmd, file=sys.stderr)
                if err.strip():
                    print(err, file=sys.stderr)
            if rc != 0:
                raise RuntimeError(f"hipcc failed: {cmd}\n{err}")
        _link([objs[s] for s in SOURCES], LIB, tmp)
        _link([sync_objs.get(s, objs[s]) for s in SOURCES], LIB_SYNC, tmp)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
