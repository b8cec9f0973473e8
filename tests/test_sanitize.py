"""CPU tier: the oracle and the library's host-side argument checks built with
AddressSanitizer and UndefinedBehaviorSanitizer and run through drivers under
tests/sanitize/ (no GPU needed; every ABI call there fails a check before
anything is enqueued). A memory error, leak (oracle) or undefined operation
aborts the driver with a report."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "quantized_decode_q4_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{cmd[0]} failed ({res.returncode}):\n{res.stdout}\n{res.stderr[-4000:]}"
    return res


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_asan")
    run(["gcc", "-std=c11", "-O1", "-g", "-D_GNU_SOURCE", "-fno-fast-math", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "q4k_oracle.c"),
         "-o", exe, "-lm"])
    res = run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"}, timeout=300)
    assert "oracle driver: ok" in res.stdout
    assert "runtime error" not in res.stderr


def test_abi_host_code_under_asan_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm toolchain not available")
    objs = []
    procs = []
    for name in sorted(os.path.splitext(os.path.basename(f))[0]
                       for f in glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / f"{name}.o")
        objs.append(obj)
        # sanitizers on the host pass only (the kernels are compiled as usual)
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, f"{name}.hip"), "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-4000:]
    drv = str(tmp_path / "abi_driver.o")
    run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         f"-I{INCLUDE}", "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_asan")
    run([CLANGXX, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime's own allocations are not this library's: no leak check
    res = run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"}, timeout=120)
    assert "abi driver: ok" in res.stdout
    assert "runtime error" not in res.stderr
