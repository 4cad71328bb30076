"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU oracle and of the host
side of the C ABI, each driven by a small C program over small shapes (CPU only: the host
code of libepoch is instrumented, its device code is built as usual and never launched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_diffusion_sparse_amd", "csrc")
SOURCES = ["epoch_abi", "router", "plan", "experts", "decode"]
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{out[-4000:]}"
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off", "-o", exe,
         os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_check.c"), "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", OMP_NUM_THREADS="2")
    out = run([exe], env=env, timeout=300)
    assert "oracle sanitizer check ok" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out


def test_host_abi_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
             "-I", os.path.join(ROOT, "include")]
    procs = []
    objs = []
    for s in SOURCES:
        obj = str(tmp_path / f"{s}.o")
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc, *flags, "-c", os.path.join(CSRC, f"{s}.hip"), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out[-4000:]
    drv = str(tmp_path / "abi_check.o")
    run([hipcc, "-O1", "-g", *HOST_SAN, "-x", "c", "-c", os.path.join(SAN, "abi_check.c"), "-o", drv])
    exe = str(tmp_path / "abi_check")
    run([hipcc, "--offload-arch=gfx950", *HOST_SAN, "-o", exe, *objs, drv])
    # the HIP runtime's own allocations at load are not this library's: no leak check
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    out = run([exe], env=env, timeout=300)
    assert "abi sanitizer check ok" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out
