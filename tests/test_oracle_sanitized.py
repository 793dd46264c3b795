"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): oracle/qkv_oracle.c is built with -fsanitize=address,undefined in a
temporary directory and the whole pin battery runs against it in a child
process, with the sanitizer runtimes preloaded.  Any out-of-bounds access, use
after free or undefined operation (signed overflow, bad shift, misaligned
load) ends the child with an error."""
import os
import subprocess
import sys

import pytest

import oracle
import test_oracle_mutants as M

HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=%s" % name], capture_output=True, text=True).stdout.strip()
    return os.path.realpath(path) if os.path.isabs(path) and os.path.exists(path) else None


NEEDS_RUNTIMES = pytest.mark.skipif(_runtime("libasan.so") is None or _runtime("libubsan.so") is None,
                                    reason="gcc sanitizer runtimes not installed")


def _build(tmp_path, text):
    src = tmp_path / "orc.c"
    src.write_text(text)
    lib = tmp_path / "liborc_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fPIC", "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", str(src), "-o", str(lib), "-lm"], check=True)
    return lib


def _run_battery(lib):
    code = (
        "import ctypes, sys\n"
        "import oracle, test_oracle_mutants as M\n"
        "oracle._lib = oracle.configure(ctypes.CDLL(sys.argv[1]))\n"
        "n = 0\n"
        "for name, fn in M.battery():\n"
        "    if name.split('[')[0] in M.SLOW:\n"
        "        continue\n"
        "    fn()\n"
        "    n += 1\n"
        "print('CLEAN', n)\n")
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([HERE, os.path.dirname(HERE), env.get("PYTHONPATH", "")])
    env["LD_PRELOAD"] = " ".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    env["OMP_NUM_THREADS"] = "4"
    return subprocess.run([sys.executable, "-c", code, str(lib)], capture_output=True, text=True,
                          env=env, timeout=900)


@NEEDS_RUNTIMES
def test_pin_battery_is_clean_under_asan_and_ubsan(tmp_path):
    res = _run_battery(_build(tmp_path, open(M.SRC).read()))
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "CLEAN" in res.stdout, tail
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail


@NEEDS_RUNTIMES
def test_sanitizer_catches_a_planted_out_of_bounds_write(tmp_path):
    # The control: the oracle copy writes a slot at capacity, one slot past the
    # end of the cache buffer; the sanitized run must report it.
    old = "if (slot < 0 || block_size <= 0 || slot >= num_blocks * (int64_t)block_size)"
    text = open(M.SRC).read()
    assert text.count(old) == 1
    res = _run_battery(_build(tmp_path, text.replace(old, old.replace(">=", ">"))))
    assert res.returncode != 0 and "AddressSanitizer" in res.stderr, (res.stdout + res.stderr)[-2000:]
