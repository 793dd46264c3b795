"""Python binding of the probe library, libqkv_prep_probe.so
(include/qkv_prep_probe.h): bandwidth ceilings (a streaming copy, an in-place
streaming update), policy-selectable streams, and the operators' number-format
code run on arrays.  Used by the tests and the benchmark; the operators never
load it.  Argument marshalling only, with the C names."""
from __future__ import annotations

import ctypes
import os

from fp8_kv_cache_amd.qkv_prep import OK, QkvPrepError

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqkv_prep_probe.so")

EXPORTED = ("qkv_prep_probe_copy", "qkv_prep_probe_update", "qkv_prep_probe_stream",
            "qkv_prep_probe_mxfp8_pattern", "qkv_prep_probe_convert", "qkv_prep_probe_ue8m0")

# qkv_prep_probe_stream kinds and cache-policy bits.
READ, WRITE, COPY, UPDATE = 0, 1, 2, 3
SC0, NT, SC1 = 1, 2, 16
# qkv_prep_probe_mxfp8_pattern streams.
MX_RESIDUAL, MX_CODES, MX_SCALES, MX_BARRIER = 1, 2, 4, 8


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqkv_prep_probe.so is not built (%s); run `python -m fp8_kv_cache_amd.build`"
                          % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.qkv_prep_probe_copy.argtypes = [vp, vp, i64, vp]
    L.qkv_prep_probe_update.argtypes = [vp, i64, vp]
    i32 = ctypes.c_int32
    L.qkv_prep_probe_stream.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, i64, ctypes.c_uint32, vp]
    L.qkv_prep_probe_mxfp8_pattern.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, vp]
    L.qkv_prep_probe_convert.argtypes = [vp, i64, vp, vp, ctypes.c_int32, vp]
    L.qkv_prep_probe_ue8m0.argtypes = [vp, i64, vp, vp, vp, vp]
    for name in EXPORTED:
        getattr(L, name).restype = ctypes.c_int
    return L


_lib = _load()


def library():
    return _lib


def _check(rc, what):
    if rc != OK:
        raise QkvPrepError(rc, what)


def qkv_prep_probe_copy(dst_ptr: int, src_ptr: int, nbytes: int, stream=None) -> None:
    """The streaming-copy probe (a bandwidth ceiling)."""
    _check(_lib.qkv_prep_probe_copy(dst_ptr, src_ptr, nbytes, stream), "qkv_prep_probe_copy")


def qkv_prep_probe_update(buf_ptr: int, nbytes: int, stream=None) -> None:
    """The in-place streaming-update probe (a bandwidth ceiling)."""
    _check(_lib.qkv_prep_probe_update(buf_ptr, nbytes, stream), "qkv_prep_probe_update")


def qkv_prep_probe_stream(kind: int, load_policy: int, store_policy: int, sleep: int, lanes_per_block: int,
                          depth: int, xcd_order: int, dst_ptr, src_ptr, nbytes: int, key: int = 0,
                          stream=None) -> None:
    """A policy-selectable read, write, copy or in-place update stream."""
    _check(_lib.qkv_prep_probe_stream(kind, load_policy, store_policy, sleep, lanes_per_block, depth, xcd_order,
                                      dst_ptr, src_ptr, nbytes, key, stream), "qkv_prep_probe_stream")


def qkv_prep_probe_mxfp8_pattern(x_ptr, residual_ptr, gamma_ptr, residual_out_ptr, codes_ptr, scales_ptr, m: int,
                                 hidden: int, streams: int, stream=None) -> None:
    """The MXFP8 operator's access pattern with no arithmetic."""
    _check(_lib.qkv_prep_probe_mxfp8_pattern(x_ptr, residual_ptr, gamma_ptr, residual_out_ptr, codes_ptr,
                                             scales_ptr, m, hidden, streams, stream), "qkv_prep_probe_mxfp8_pattern")


def qkv_prep_probe_convert(in_ptr: int, n: int, e4m3_ptr, bf16_ptr, convert: int, stream=None) -> None:
    """The operator's E4M3 and bf16 conversions on an array (device pointers)."""
    _check(_lib.qkv_prep_probe_convert(in_ptr, n, e4m3_ptr, bf16_ptr, convert, stream), "qkv_prep_probe_convert")


def qkv_prep_probe_ue8m0(in_ptr, n: int, op_byte_ptr, mx_byte_ptr, mx_inverse_ptr, stream=None) -> None:
    """The operators' two UE8M0 rules on an array (device pointers)."""
    _check(_lib.qkv_prep_probe_ue8m0(in_ptr, n, op_byte_ptr, mx_byte_ptr, mx_inverse_ptr, stream),
           "qkv_prep_probe_ue8m0")
