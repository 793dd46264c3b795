"""CPU oracle for the fused q/kv RMSNorm + RoPE + FP8 quantize + paged-cache insert.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``fp8_kv_cache_amd``) never imports it, and this package imports nothing from
the product path.

The arithmetic lives in ``qkv_oracle.c`` (plain scalar C, fp32 with every
rounding pinned; see that file's header for the pages followed and the
readings taken).  This module only builds that file with gcc and marshals
numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qkv_oracle.c")
_LIB = os.path.join(_HERE, "libqkv_oracle.so")

HEAD_DIM = 512
NOPE_DIM = 448
ROPE_DIM = 64
SLOT_DATA = 576
SLOT_SCALE = 8
SLOT_BYTES = 584

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fused multiply-add contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def configure(L):
    """Declare the C signatures on a loaded oracle library."""
    if True:
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = f32
        L.orc_f32_to_bf16.argtypes = [f32]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f64.restype = ctypes.c_double
        L.orc_f32_to_e4m3.argtypes = [f32]
        L.orc_f32_to_e4m3.restype = ctypes.c_uint8
        L.orc_ue8m0_exponent.argtypes = [f32]
        L.orc_ue8m0_exponent.restype = ctypes.c_int
        L.orc_sum_squares.argtypes = [vp]
        L.orc_sum_squares.restype = f32
        L.orc_inv_rms.argtypes = [f32, f32]
        L.orc_inv_rms.restype = f32
        L.orc_slot_offsets.argtypes = [i64, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.orc_slot_offsets.restype = ctypes.c_int
        L.orc_qkv_prep.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, i64,
                                   i32, f32, ctypes.c_int]
        L.orc_qkv_prep.restype = ctypes.c_int
        L.orc_qkv_prep_bf16_store.argtypes = L.orc_qkv_prep.argtypes
        L.orc_qkv_prep_bf16_store.restype = ctypes.c_int
        L.orc_gather_dequant.argtypes = [vp, i64, i32, vp, i64, vp]
        L.orc_sum_squares_n.argtypes = [vp, i64]
        L.orc_sum_squares_n.restype = f32
        L.orc_ue8m0_ceil_byte.argtypes = [f32]
        L.orc_ue8m0_ceil_byte.restype = ctypes.c_uint32
        L.orc_ue8m0_inverse.argtypes = [ctypes.c_uint32]
        L.orc_ue8m0_inverse.restype = f32
        L.orc_mxfp8_scale_offset.argtypes = [i64, i64, i64]
        L.orc_mxfp8_scale_offset.restype = i64
        L.orc_mxfp8_norm_quant.argtypes = [i64, i64, vp, vp, vp, vp, f32, vp, vp]
        L.orc_mxfp8_norm_quant.restype = ctypes.c_int
        L.orc_f32_to_bf16_array.argtypes = [vp, vp, i64]
        L.orc_f32_to_e4m3_array.argtypes = [vp, vp, i64]
        L.orc_ue8m0_exponent_array.argtypes = [vp, vp, i64]
        L.orc_ue8m0_ceil_byte_array.argtypes = [vp, vp, i64]
        L.orc_rows.argtypes = [i64, vp, vp, f32, vp, vp, vp, vp]
        L.orc_quant_rows.argtypes = [i64, vp, vp, vp]
    return L


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return a


# ---------------------------------------------------------------- formats

def f32_to_bf16(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_array(_p(x), _p(out), x.size)
    return out


def bf16_to_f32(b) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_e4m3(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_f32_to_e4m3_array(_p(x), _p(out), x.size)
    return out


def e4m3_to_f64(c) -> np.ndarray:
    L = lib()
    c = np.asarray(c, dtype=np.uint8)
    table = np.array([L.orc_e4m3_to_f64(i) for i in range(256)], dtype=np.float64)
    return table[c]


def ue8m0_exponent(amax) -> np.ndarray:
    a = _c(np.asarray(amax, dtype=np.float32), np.float32)
    out = np.empty(a.shape, np.int32)
    lib().orc_ue8m0_exponent_array(_p(a), _p(out), a.size)
    return out


# ---------------------------------------------------------------- rows

def rows(x_bf16, w_bf16, eps, cs):
    """Per-row intermediates: (y before rotation, z after, sum_sq, inv_rms).

    x_bf16: uint16 [n, 512]; w_bf16: uint16 [512] or None; cs: fp32 [n, 64]."""
    x = _c(np.asarray(x_bf16, dtype=np.uint16).reshape(-1, HEAD_DIM), np.uint16)
    n = x.shape[0]
    cs = _c(np.asarray(cs, dtype=np.float32).reshape(n, 64), np.float32)
    w = None if w_bf16 is None else _c(np.asarray(w_bf16, dtype=np.uint16), np.uint16)
    y = np.empty((n, HEAD_DIM), np.float32)
    z = np.empty((n, HEAD_DIM), np.float32)
    st = np.empty((n, 2), np.float32)
    lib().orc_rows(n, _p(x), _p(w), float(eps), _p(cs), _p(y), _p(z), _p(st))
    return y, z, st[:, 0].copy(), st[:, 1].copy()


def quant_rows(y):
    """y: fp32 [n, 448] -> (codes uint8 [n, 448], scale bytes uint8 [n, 7])."""
    y = _c(np.asarray(y, dtype=np.float32).reshape(-1, NOPE_DIM), np.float32)
    n = y.shape[0]
    codes = np.empty((n, NOPE_DIM), np.uint8)
    scales = np.empty((n, 7), np.uint8)
    lib().orc_quant_rows(n, _p(y), _p(codes), _p(scales))
    return codes, scales


def slot_offsets(slot, num_blocks, block_size):
    """(data_offset, scale_offset) of a slot in the cache, or None when skipped."""
    d, s = ctypes.c_int64(), ctypes.c_int64()
    ok = lib().orc_slot_offsets(int(slot), int(num_blocks), int(block_size),
                                ctypes.byref(d), ctypes.byref(s))
    return (d.value, s.value) if ok else None


# ---------------------------------------------------------------- operator

def qkv_prep(q, kv, q_w, kv_w, positions, cos_sin, slot_mapping, cache,
             num_blocks, block_size, eps, nthreads=1, kv_store="fp8", out=None):
    """Run the whole operator on host arrays.

    q: uint16 [T, H, 512] (bf16 bits) -- not modified; the new q is returned.
    cache: uint8 [num_blocks, block_size*584] for kv_store="fp8", or
    [num_blocks, block_size*1024] for kv_store="bf16" -- updated in place.
    out: optional contiguous uint16 array shaped like q to receive the new q
    (so that a timing loop allocates nothing).
    Returns the new q (uint16 [T, H, 512])."""
    q = _c(np.asarray(q, dtype=np.uint16), np.uint16)
    T, H = q.shape[0], q.shape[1]
    kv = _c(np.asarray(kv, dtype=np.uint16), np.uint16)
    q_w = None if q_w is None else _c(np.asarray(q_w, dtype=np.uint16), np.uint16)
    kv_w = _c(np.asarray(kv_w, dtype=np.uint16), np.uint16)
    positions = _c(np.asarray(positions, dtype=np.int64), np.int64)
    cos_sin = _c(np.asarray(cos_sin, dtype=np.float32), np.float32)
    slot_mapping = _c(np.asarray(slot_mapping, dtype=np.int64), np.int64)
    if not (cache.flags["C_CONTIGUOUS"] and cache.dtype == np.uint8):
        raise TypeError("cache must be a contiguous uint8 array")
    slot_bytes = {"fp8": SLOT_BYTES, "bf16": 1024}[kv_store]
    if cache.size != num_blocks * block_size * slot_bytes:
        raise ValueError("cache size does not match num_blocks*block_size*%d" % slot_bytes)
    assert kv.shape == (T, HEAD_DIM) and positions.shape == (T,) and slot_mapping.shape == (T,)
    if out is None:
        out = np.empty_like(q)
    elif not (out.flags["C_CONTIGUOUS"] and out.dtype == np.uint16 and out.shape == q.shape):
        raise TypeError("out must be a contiguous uint16 array shaped like q")
    fn = lib().orc_qkv_prep if kv_store == "fp8" else lib().orc_qkv_prep_bf16_store
    rc = fn(T, H, _p(q), _p(out), _p(kv), _p(q_w), _p(kv_w),
                            _p(positions), _p(cos_sin), cos_sin.shape[0],
                            _p(slot_mapping), _p(cache), int(num_blocks), int(block_size),
                            float(eps), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (position out of range?)")
    return out


def gather_dequant(cache, num_blocks, block_size, slots):
    """Read slots back out of an FP8 + UE8M0 cache: fp32 [n, 512] (zeros for
    skipped slots)."""
    if not (cache.flags["C_CONTIGUOUS"] and cache.dtype == np.uint8):
        raise TypeError("cache must be a contiguous uint8 array")
    slots = _c(np.asarray(slots, dtype=np.int64).reshape(-1), np.int64)
    out = np.empty((slots.size, HEAD_DIM), np.float32)
    lib().orc_gather_dequant(_p(cache), int(num_blocks), int(block_size), _p(slots), slots.size,
                             _p(out))
    return out


# ---------------------------------------------------------------- MXFP8 variant

def mxfp8_scale_bytes(m, hidden):
    cols = hidden // 32
    return (m + 127) // 128 * 128 * ((cols + 3) // 4 * 4)


def mxfp8_norm_quant(x, gamma, eps, residual=None):
    """Residual add + Gemma RMSNorm + MXFP8 quantization (see qkv_oracle.c, M1-M7).

    x, residual: uint16 [m, hidden] bf16 bits; gamma: uint16 [hidden].
    Returns (codes uint8 [m, hidden], swizzled scales uint8 [...], prenorm
    uint16 [m, hidden] or None)."""
    x = _c(np.asarray(x, dtype=np.uint16), np.uint16)
    m, hidden = x.shape
    gamma = _c(np.asarray(gamma, dtype=np.uint16), np.uint16)
    res = None if residual is None else _c(np.asarray(residual, dtype=np.uint16), np.uint16)
    res_out = None if residual is None else np.empty_like(x)
    codes = np.empty((m, hidden), np.uint8)
    scales = np.full(mxfp8_scale_bytes(m, hidden), 0xEE, np.uint8)
    rc = lib().orc_mxfp8_norm_quant(m, hidden, _p(x), _p(res), _p(res_out), _p(gamma),
                                    float(eps), _p(codes), _p(scales))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (hidden must be a multiple of 128)")
    return codes, scales, res_out


def mxfp8_scale_offset(row, col, padded_cols):
    return lib().orc_mxfp8_scale_offset(int(row), int(col), int(padded_cols))


def ue8m0_ceil_byte(v):
    return int(lib().orc_ue8m0_ceil_byte(float(v)))


def ue8m0_ceil_bytes(v) -> np.ndarray:
    """The MXFP8 scale byte of every value of a float32 array (uint8)."""
    v = _c(np.asarray(v, dtype=np.float32), np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_ue8m0_ceil_byte_array(_p(v), _p(out), v.size)
    return out


def ue8m0_inverse(byte):
    return float(lib().orc_ue8m0_inverse(int(byte)))
