"""The library used from C with no Python in the loop: tests/c_consumer.c
(C11; the public header and the HIP runtime's C API only) is compiled with gcc
and linked against libqkv_prep.so and the oracle's source.  On the CPU the
test checks that it builds without warnings; on the GPU it runs and must report
q, the cache and the gathered rows bit-exact against the oracle, eagerly and
over three replays of a HIP graph captured from C, and the MXFP8 operator's
codes, scale bytes and residual output bit-exact too."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
PKG = os.path.join(ROOT, "fp8_kv_cache_amd")
LIB = os.path.join(PKG, "libqkv_prep.so")


def build(tmp_path):
    exe = tmp_path / "c_consumer"
    res = subprocess.run(
        ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
         "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
         os.path.join(HERE, "c_consumer.c"), os.path.join(ROOT, "oracle", "qkv_oracle.c"),
         "-L" + PKG, "-lqkv_prep", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath," + PKG, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm", "-o", str(exe)],
        capture_output=True, text=True)
    return exe, res


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists(LIB), reason="needs gcc and the built library")
def test_c_consumer_builds_without_warnings(tmp_path):
    _, res = build(tmp_path)
    assert res.returncode == 0, res.stderr[-3000:]
    own = [l for l in res.stderr.splitlines() if "c_consumer.c" in l]
    assert not own, "\n".join(own)


@pytest.mark.gpu
def test_c_consumer_is_bit_exact_on_the_gpu(tmp_path):
    assert os.path.exists(LIB), "libqkv_prep.so is not built"
    exe, res = build(tmp_path)
    assert res.returncode == 0, res.stderr[-3000:]
    print("running the C consumer", flush=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout.strip(), flush=True)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-2000:]
    assert "bit-exact" in run.stdout
