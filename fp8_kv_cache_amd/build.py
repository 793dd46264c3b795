"""Build the two libraries for gfx950 with hipcc: libqkv_prep.so (the
operators' HIP kernels + C ABI) and libqkv_prep_probe.so (bandwidth ceilings
and number-format probes, used by the tests and the benchmark only).

Run as ``python -m fp8_kv_cache_amd.build``.  The libraries are built in-tree,
next to this file, so that they travel with the source tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqkv_prep.so")
PROBE_LIB = os.path.join(PKG, "libqkv_prep_probe.so")
SOURCES = [os.path.join(CSRC, f) for f in ("qkv_prep_kernels.hip", "qkv_prep_api.cpp", "qkv_prep_gather.hip",
                                           "mxfp8_norm_quant.hip", "mxfp8_api.cpp")]
PROBE_SOURCES = [os.path.join(CSRC, "qkv_prep_probe.hip")]

# -ffp-contract=off: no multiply is fused into an add unless the source asks
# for an fma, so every fp32 step rounds as the numerics contract states.
# -packed-fp32-ops off: keep the compiler from emitting packed fp32 math.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqkv_prep.so)")


def _link(out: str, sources, verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + \
        list(sources) + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % os.path.basename(out))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Build both libraries; returns the path of libqkv_prep.so."""
    _link(PROBE_LIB, PROBE_SOURCES, verbose)
    return _link(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
