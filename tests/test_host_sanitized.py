"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/host_fuzz.cpp and csrc/qkv_prep_api.cpp are
built with g++ -fsanitize=address,undefined (host code only: the two kernel
launchers are stubbed and the six HIP runtime calls the host API makes are a
fake two-device runtime, so no GPU and no HIP library are involved).  400 000
extreme and random configs and arguments go through qkv_prep_validate,
qkv_prep_launch_shape, qkv_prep_supported and qkv_prep_strerror, and 100 000
handles run qkv_prep_run and qkv_prep_gather on random arguments, and
200 000 cases go through the MXFP8 entry points (qkv_prep_mxfp8_scale_bytes,
qkv_prep_mxfp8_norm_quant, from mxfp8_api.cpp).  Any
undefined operation (signed overflow in the size arithmetic, a bad shift) or
out-of-bounds access aborts the run; the codes, the launch arguments, the grid
and the restored current device are checked against the header's contract."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_host_api_fuzz_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_fuzz"
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
         "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
         "-I" + os.path.join(ROOT, "fp8_kv_cache_amd", "csrc"),
         os.path.join(HERE, "host_fuzz.cpp"), os.path.join(ROOT, "fp8_kv_cache_amd", "csrc", "qkv_prep_api.cpp"),
         os.path.join(ROOT, "fp8_kv_cache_amd", "csrc", "mxfp8_api.cpp"),
         "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    own = [l for l in build.stderr.splitlines() if "warning" in l and ROCM not in l]
    assert not own, "\n".join(own)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, (res.stdout + res.stderr)[-3000:]
    assert "contract failures 0" in res.stdout
    # the handle half really launched (the fake runtime lets create succeed)
    assert int(res.stdout.split("runs launched ")[1].split()[0].rstrip(",")) > 10000
    assert int(res.stdout.split("mxfp8 launched ")[1].split()[0].rstrip(",")) > 10000
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
