"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's host side (csrc/api.hip) is rebuilt with the sanitizers on the host
pass only (-Xarch_host before each -fsanitize=; device code is untouched),
linked with the normally built scheduler and GEMM objects and a C driver
(tests/abi_driver.c) that takes every entry point down its validation paths.
Nothing is launched, so no GPU is needed."""
import os
import shutil
import subprocess

import pytest

from moe_grouped_gemm_sizes_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
OBJ = os.path.join(os.path.dirname(B.CSRC), "_build")


@pytest.mark.timeout(300)
def test_api_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = B.hipcc()
    objs = [os.path.join(OBJ, "sched.o"), os.path.join(OBJ, "gemm.o")]
    if not all(os.path.exists(o) for o in objs):
        B.build(verbose=False)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_san.o")
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([hipcc, *B.HIPFLAGS, *san, "-c", os.path.join(B.CSRC, "api.hip"), "-o", api_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    drv_o = str(tmp_path / "abi_driver.o")
    cc = shutil.which("gcc") or "cc"
    r = subprocess.run([cc, "-std=c99", "-O1", "-g", "-Wall", "-c", os.path.join(HERE, "abi_driver.c"), "-o", drv_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", *san, drv_o, api_o, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-3000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
