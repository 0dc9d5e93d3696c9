"""Build libkvdec.so (gfx950 code objects + the C-ABI host layer) in-tree.

hipcc cross-compiles for gfx950 without a GPU present.  Packed-FP32 VALU
forms are disabled for device code (the compiler otherwise forms
v_pk_{add,mul,fma}_f32 from plain float code).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "kvdec_kernels.hip"), os.path.join(CSRC, "kvdec_api.cpp")]
HEADERS = [os.path.join(CSRC, "kvdec_internal.h"), os.path.join(ROOT, "include", "kvdec.h")]
LIB = os.path.join(HERE, "libkvdec.so")
# counter-calibration probe for bench.py (not part of the decode library)
PROBE_SOURCES = [os.path.join(CSRC, "read_probe.hip")]
PROBE_LIB = os.path.join(HERE, "libkvdec_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    if not os.path.exists(PROBE_LIB):
        return True
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS + PROBE_SOURCES)


def _hipcc(out, sources, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden",
           "-Wall", "-Wno-unused-command-line-argument", *DEVICE_FLAGS,
           "-I", os.path.join(ROOT, "include"), "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-6000:]}")
    os.replace(tmp, out)


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and not _stale():
        return LIB
    _hipcc(LIB, SOURCES, verbose)
    _hipcc(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
