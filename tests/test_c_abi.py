"""The boundary from C: tests/c/abi_check.c, compiled as C99 with gcc against
include/kvdec.h and linked to libkvdec.so, runs the argument checks that
return before any device work (no GPU needed); tests/c/abi_step.c runs a
real decode step from C on the GPU and checks it against the oracle."""
import os
import shutil
import subprocess

import pytest

from kv_cached_decode_kvdec_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_c99_program_links_and_runs(tmp_path):
    lib_dir = os.path.dirname(B.LIB_PATH)
    if not os.path.exists(B.LIB_PATH):
        pytest.fail(f"{B.LIB_PATH} is missing: build it first")
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
           "-L", lib_dir, "-lkvdec", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    built = subprocess.run(cmd, capture_output=True, text=True)
    assert built.returncode == 0, built.stderr
    ran = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert ran.returncode == 0, ran.stdout + ran.stderr
    assert ran.stdout.strip() == "0 failed"


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_c99_program_runs_a_decode_step(tmp_path):
    """Device buffers from the HIP runtime, kvdec_cache_create for a self and a
    static cache, kvdec_seed, kvdec_append_attend_cross for a token (outputs
    against the oracle, appended rows bit for bit), then a refused overflow."""
    import oracle
    lib_dir = os.path.dirname(B.LIB_PATH)
    oracle_dir = os.path.dirname(oracle.load()._name)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = tmp_path / "abi_step"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(rocm, "include"),
           os.path.join(ROOT, "tests", "c", "abi_step.c"),
           "-L", lib_dir, "-lkvdec", "-L", oracle_dir, "-lkvdec_oracle",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{lib_dir}:{oracle_dir}:{os.path.join(rocm, 'lib')}", "-o", str(exe)]
    built = subprocess.run(cmd, capture_output=True, text=True)
    assert built.returncode == 0, built.stderr
    ran = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert ran.returncode == 0, ran.stdout + ran.stderr
    assert ran.stdout.strip() == "0 failed"
