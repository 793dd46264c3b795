"""Python binding of the qkv_prep C ABI (include/qkv_prep.h).

Argument marshalling only: every step of the operator runs in the HIP kernels
of libqkv_prep.so.  The functions keep the C names; ``QkvPrep`` is a small
convenience wrapper that takes torch tensors (torch supplies device memory and
the stream, nothing else).  There is no fallback: if the library is missing
the import of this module raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqkv_prep.so")

OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED = 2
ERR_MISALIGNED = 3
ERR_NO_DEVICE = 4
ERR_LAUNCH = 5
ERR_DEVICE = 6

HEAD_DIM = 512
NOPE_DIM = 448
ROPE_DIM = 64
SLOT_DATA_BYTES = 576
SLOT_SCALE_BYTES = 8
SLOT_BYTES = 584

CONVERT_INTEGER = 1
CONVERT_INSTRUCTIONS = 2

KV_FP8 = 0
KV_BF16 = 1
BF16_SLOT_BYTES = 1024
OUT_F32 = 0
OUT_BF16 = 1

# Every symbol the header declares (checked by the ABI tests).
EXPORTED = ("qkv_prep_create", "qkv_prep_run", "qkv_prep_destroy", "qkv_prep_supported",
            "qkv_prep_launch_shape", "qkv_prep_validate", "qkv_prep_strerror",
            "qkv_prep_gather", "qkv_prep_mxfp8_norm_quant", "qkv_prep_mxfp8_scale_bytes")


class QkvPrepConfig(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rows_per_wave", ctypes.c_int32),
                ("waves_per_block", ctypes.c_int32), ("convert", ctypes.c_int32),
                ("kv_store", ctypes.c_int32), ("kv_per_wave", ctypes.c_int32)]


class QkvPrepArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("q_norm_w", ctypes.c_void_p),
                ("kv_norm_w", ctypes.c_void_p), ("positions", ctypes.c_void_p),
                ("cos_sin", ctypes.c_void_p), ("max_position", ctypes.c_int64),
                ("slot_mapping", ctypes.c_void_p), ("kv_cache", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("num_tokens", ctypes.c_int64)]


class QkvPrepGatherArgs(ctypes.Structure):
    _fields_ = [("kv_cache", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
                ("slots", ctypes.c_void_p), ("n", ctypes.c_int64), ("out", ctypes.c_void_p),
                ("out_dtype", ctypes.c_int32)]


class QkvPrepMxfp8Args(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("residual_out", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("quant_out", ctypes.c_void_p), ("scale_out", ctypes.c_void_p),
                ("m", ctypes.c_int64), ("hidden", ctypes.c_int32), ("eps", ctypes.c_float)]


class QkvPrepLaunch(ctypes.Structure):
    _fields_ = [("rows_per_wave", ctypes.c_int32), ("waves_per_block", ctypes.c_int32),
                ("convert", ctypes.c_int32), ("kv_per_wave", ctypes.c_int32), ("kv_blocks", ctypes.c_int64),
                ("q_blocks", ctypes.c_int64), ("grid", ctypes.c_int64), ("kv_period", ctypes.c_int64)]


class QkvPrepError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__("%s: %s (code %d)" % (what or "qkv_prep", qkv_prep_strerror(code), code))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqkv_prep.so is not built (%s); run `python -m fp8_kv_cache_amd.build`"
                          % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.qkv_prep_create.argtypes = [P(QkvPrepConfig), ctypes.c_int, P(ctypes.c_void_p)]
    L.qkv_prep_create.restype = ctypes.c_int
    L.qkv_prep_run.argtypes = [ctypes.c_void_p, P(QkvPrepArgs), ctypes.c_void_p]
    L.qkv_prep_run.restype = ctypes.c_int
    L.qkv_prep_destroy.argtypes = [ctypes.c_void_p]
    L.qkv_prep_destroy.restype = ctypes.c_int
    L.qkv_prep_supported.argtypes = [ctypes.c_int32] * 3
    L.qkv_prep_supported.restype = ctypes.c_int
    L.qkv_prep_launch_shape.argtypes = [P(QkvPrepConfig), ctypes.c_int32, ctypes.c_int64,
                                        P(QkvPrepLaunch)]
    L.qkv_prep_launch_shape.restype = ctypes.c_int
    L.qkv_prep_validate.argtypes = [P(QkvPrepConfig), P(QkvPrepArgs)]
    L.qkv_prep_validate.restype = ctypes.c_int
    L.qkv_prep_strerror.argtypes = [ctypes.c_int]
    L.qkv_prep_strerror.restype = ctypes.c_char_p
    L.qkv_prep_gather.argtypes = [ctypes.c_void_p, P(QkvPrepGatherArgs), ctypes.c_void_p]
    L.qkv_prep_gather.restype = ctypes.c_int
    L.qkv_prep_mxfp8_norm_quant.argtypes = [P(QkvPrepMxfp8Args), ctypes.c_int, ctypes.c_void_p]
    L.qkv_prep_mxfp8_norm_quant.restype = ctypes.c_int
    L.qkv_prep_mxfp8_scale_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32]
    L.qkv_prep_mxfp8_scale_bytes.restype = ctypes.c_int64
    return L


_lib = _load()


def library():
    return _lib


def make_config(num_heads, *, block_size=64, eps=1e-6, rows_per_wave=0, waves_per_block=0,
                convert=0, kv_store=KV_FP8, kv_per_wave=0) -> QkvPrepConfig:
    return QkvPrepConfig(num_heads, HEAD_DIM, ROPE_DIM, block_size, eps, rows_per_wave,
                         waves_per_block, convert, kv_store, kv_per_wave)


# ------------------------------------------------------------ C-named calls

def qkv_prep_strerror(code: int) -> str:
    return _lib.qkv_prep_strerror(code).decode()


def qkv_prep_supported(num_heads: int, head_dim: int = HEAD_DIM, rope_dim: int = ROPE_DIM) -> bool:
    return bool(_lib.qkv_prep_supported(num_heads, head_dim, rope_dim))


def qkv_prep_create(cfg: QkvPrepConfig, device: int = 0) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    rc = _lib.qkv_prep_create(ctypes.byref(cfg), device, ctypes.byref(h))
    if rc != OK:
        raise QkvPrepError(rc, "qkv_prep_create")
    return h


def qkv_prep_run(handle, args: QkvPrepArgs, stream=None) -> None:
    rc = _lib.qkv_prep_run(handle, ctypes.byref(args), stream)
    if rc != OK:
        raise QkvPrepError(rc, "qkv_prep_run")


def qkv_prep_destroy(handle) -> None:
    _lib.qkv_prep_destroy(handle)


def qkv_prep_launch_shape(cfg: QkvPrepConfig, num_cus: int, num_tokens: int) -> QkvPrepLaunch:
    out = QkvPrepLaunch()
    rc = _lib.qkv_prep_launch_shape(ctypes.byref(cfg), num_cus, num_tokens, ctypes.byref(out))
    if rc != OK:
        raise QkvPrepError(rc, "qkv_prep_launch_shape")
    return out


def qkv_prep_validate(cfg: QkvPrepConfig, args: QkvPrepArgs) -> int:
    return _lib.qkv_prep_validate(ctypes.byref(cfg), ctypes.byref(args))


def qkv_prep_gather(handle, args: QkvPrepGatherArgs, stream=None) -> None:
    rc = _lib.qkv_prep_gather(handle, ctypes.byref(args), stream)
    if rc != OK:
        raise QkvPrepError(rc, "qkv_prep_gather")


def qkv_prep_mxfp8_scale_bytes(m: int, hidden: int) -> int:
    return _lib.qkv_prep_mxfp8_scale_bytes(m, hidden)


def qkv_prep_mxfp8_norm_quant(args: QkvPrepMxfp8Args, device: int = 0, stream=None) -> None:
    rc = _lib.qkv_prep_mxfp8_norm_quant(ctypes.byref(args), device, stream)
    if rc != OK:
        raise QkvPrepError(rc, "qkv_prep_mxfp8_norm_quant")


def mxfp8_norm_quant(x, gamma, eps, *, residual=None, residual_out=None, quant_out=None,
                     scale_out=None, stream=None):
    """Torch wrapper of qkv_prep_mxfp8_norm_quant: x [m, hidden] bf16.  Returns
    (codes uint8 [m, hidden], swizzled scales uint8 [...])."""
    launch = prepare_mxfp8_norm_quant(x, gamma, eps, residual=residual, residual_out=residual_out,
                                      quant_out=quant_out, scale_out=scale_out, stream=stream)
    launch()
    return launch.outputs


# ------------------------------------------------------------ torch wrapper

def _ptr(t):
    return None if t is None else t.data_ptr()


def _expect(name, t, dtype, shape, device):
    """One tensor's dtype, contiguity, device and (if given) shape."""
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def check_op_tensors(num_heads, block_size, slot_bytes, device, q, kv, q_norm_w, kv_norm_w, positions,
                     cos_sin, slot_mapping, kv_cache):
    """What the C side cannot see, since it takes bare pointers: every
    tensor's dtype, contiguity, device and shape (q [T, H, 512], kv [T, 512],
    weights [512], positions and slot_mapping [T], cos_sin [P, 64] with P >= 1,
    a uint8 cache of whole blocks).  A wrong shape would otherwise become an
    out-of-bounds access on the device.  Raises TypeError or ValueError."""
    import torch
    device = torch.device(device)
    if q.dim() != 3 or q.shape[1] != num_heads or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [T, %d, 512], got %s" % (num_heads, tuple(q.shape)))
    T = q.shape[0]
    _expect("q", q, torch.bfloat16, None, device)
    _expect("kv", kv, torch.bfloat16, (T, HEAD_DIM), device)
    if q_norm_w is not None:
        _expect("q_norm_w", q_norm_w, torch.bfloat16, (HEAD_DIM,), device)
    _expect("kv_norm_w", kv_norm_w, torch.bfloat16, (HEAD_DIM,), device)
    _expect("positions", positions, torch.int64, (T,), device)
    _expect("slot_mapping", slot_mapping, torch.int64, (T,), device)
    _expect("cos_sin", cos_sin, torch.float32, None, device)
    if cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM or cos_sin.shape[0] < 1:
        raise ValueError("cos_sin must be [P, 64] with P >= 1, got %s" % (tuple(cos_sin.shape),))
    if kv_cache is not None:
        _expect("kv_cache", kv_cache, torch.uint8, None, device)
        if kv_cache.numel() % (block_size * slot_bytes):
            raise ValueError("kv_cache must hold whole blocks of %d x %d bytes" % (block_size, slot_bytes))


def check_gather_tensors(block_size, device, kv_cache, slots, out):
    """The cache reader's tensors: a uint8 cache, int64 slots [n], an fp32 or
    bf16 out [n, 512], all contiguous on `device`."""
    import torch
    device = torch.device(device)
    _expect("kv_cache", kv_cache, torch.uint8, None, device)
    if kv_cache.numel() % (block_size * SLOT_BYTES):
        raise ValueError("kv_cache must hold whole blocks of %d x %d bytes" % (block_size, SLOT_BYTES))
    if slots.dim() != 1:
        raise ValueError("slots must be 1-D")
    _expect("slots", slots, torch.int64, None, device)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16, got %s" % out.dtype)
    _expect("out", out, out.dtype, (slots.numel(), HEAD_DIM), device)


def check_mxfp8_tensors(x, gamma, residual, residual_out, quant_out, scale_out):
    """The MXFP8 operator's tensors: bf16 x [m, hidden], gamma [hidden],
    residual / residual_out [m, hidden] or None, uint8 codes [m, hidden] and a
    uint8 scale buffer of at least qkv_prep_mxfp8_scale_bytes(m, hidden)
    bytes, all contiguous on x's device."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [m, hidden]")
    m, hidden = x.shape
    _expect("x", x, torch.bfloat16, None, x.device)
    _expect("gamma", gamma, torch.bfloat16, (hidden,), x.device)
    for name, t in (("residual", residual), ("residual_out", residual_out)):
        if t is not None:
            _expect(name, t, torch.bfloat16, (m, hidden), x.device)
    _expect("quant_out", quant_out, torch.uint8, (m, hidden), x.device)
    _expect("scale_out", scale_out, torch.uint8, None, x.device)
    need = qkv_prep_mxfp8_scale_bytes(m, hidden)
    if need > 0 and scale_out.numel() < need:
        raise ValueError("scale_out needs %d bytes, has %d" % (need, scale_out.numel()))


def make_args(q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache,
              num_blocks=None) -> QkvPrepArgs:
    """Pointers and sizes from torch tensors (no copies; the tensors are
    checked by check_op_tensors first)."""
    T = q.shape[0]
    if num_blocks is None:
        num_blocks = kv_cache.shape[0] if kv_cache is not None else 0
    return QkvPrepArgs(_ptr(q), _ptr(kv), _ptr(q_norm_w), _ptr(kv_norm_w), _ptr(positions),
                       _ptr(cos_sin), cos_sin.shape[0], _ptr(slot_mapping), _ptr(kv_cache),
                       num_blocks, T)


def _stream_of(stream, device):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream(device).cuda_stream


class Launch:
    """One launch whose tensors were checked and whose argument struct was
    built once, for callers that repeat the same call (a serving loop over
    fixed buffers, a benchmark).  Calling it only calls the C entry point and
    checks the return code, so its host cost is one ctypes call.

    It keeps references to the tensors and to the owning object, so the
    pointers it holds stay valid while it lives; the tensors must not be
    resized or re-strided in place meanwhile.  The stream is fixed when the
    launch is prepared, so a launch meant for a HIP graph is prepared inside
    the capture (where the current stream is the capturing one)."""

    __slots__ = ("_fn", "_cargs", "_what", "_keep")

    def __init__(self, fn, cargs, what, keep):
        self._fn = fn
        self._cargs = cargs
        self._what = what
        self._keep = keep

    def __call__(self) -> None:
        rc = self._fn(*self._cargs)
        if rc != OK:
            raise QkvPrepError(rc, self._what)

    def on_stream(self, stream) -> "Launch":
        """The same launch on another stream (the stream is the C call's last
        argument), e.g. on the capturing stream inside a HIP graph capture."""
        return type(self)(self._fn, self._cargs[:-1] + (stream,), self._what, self._keep)


class _MxLaunch(Launch):
    __slots__ = ()

    @property
    def outputs(self):
        return self._keep[4], self._keep[5]


def prepare_mxfp8_norm_quant(x, gamma, eps, *, residual=None, residual_out=None, quant_out=None,
                             scale_out=None, stream=None) -> Launch:
    """mxfp8_norm_quant with every check done now: returns a Launch that
    enqueues the operator on ``stream`` (default: the current torch stream
    at this call).  Outputs are allocated here when not given; the Launch's
    ``outputs`` are (quant_out, scale_out)."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be [m, hidden]")
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device, got %s" % x.device)
    m, hidden = x.shape
    if quant_out is None:
        quant_out = torch.empty((m, hidden), dtype=torch.uint8, device=x.device)
    if scale_out is None:
        scale_out = torch.empty(max(qkv_prep_mxfp8_scale_bytes(m, hidden), 0), dtype=torch.uint8,
                                device=x.device)
    check_mxfp8_tensors(x, gamma, residual, residual_out, quant_out, scale_out)
    args = QkvPrepMxfp8Args(x.data_ptr(), _ptr(residual), _ptr(residual_out), gamma.data_ptr(),
                            quant_out.data_ptr(), scale_out.data_ptr(), m, hidden, eps)
    device = x.device.index if x.device.index is not None else torch.cuda.current_device()
    keep = (x, gamma, residual, residual_out, quant_out, scale_out, args)
    return _MxLaunch(_lib.qkv_prep_mxfp8_norm_quant,
                     (ctypes.byref(args), device, _stream_of(stream, x.device)),
                     "qkv_prep_mxfp8_norm_quant", keep)


class QkvPrep:
    """A qkv_prep handle bound to one device.

    ``op(q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache)``
    enqueues the operator on the current torch stream (or ``stream``).
    ``op.prepare(...)`` and ``op.prepare_gather(...)`` check the same tensors
    once and return a Launch that repeats the call at the cost of one ctypes
    call."""

    def __init__(self, num_heads, *, device=0, block_size=64, eps=1e-6, rows_per_wave=0,
                 waves_per_block=0, convert=0, kv_store=KV_FP8, kv_per_wave=0):
        self.cfg = make_config(num_heads, block_size=block_size, eps=eps,
                               rows_per_wave=rows_per_wave, waves_per_block=waves_per_block,
                               convert=convert, kv_store=kv_store, kv_per_wave=kv_per_wave)
        self.slot_bytes = SLOT_BYTES if kv_store == KV_FP8 else BF16_SLOT_BYTES
        self.device = device
        self.handle = qkv_prep_create(self.cfg, device)

    def __call__(self, q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache,
                 stream=None):
        args = self._op_args(q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache)
        qkv_prep_run(self.handle, args, _stream_of(stream, q.device))
        return q

    def _op_args(self, q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache):
        import torch
        check_op_tensors(self.cfg.num_heads, self.cfg.block_size, self.slot_bytes,
                         torch.device("cuda", self.device), q, kv, q_norm_w, kv_norm_w, positions,
                         cos_sin, slot_mapping, kv_cache)
        per_block = self.cfg.block_size * self.slot_bytes
        return make_args(q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache,
                         None if kv_cache is None else kv_cache.numel() // per_block)

    def prepare(self, q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache,
                stream=None) -> Launch:
        """The operator call of ``__call__``, checked and marshalled now.  The
        returned Launch enqueues it on ``stream`` (default: the current torch
        stream at this call) each time it is called."""
        args = self._op_args(q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache)
        rc = qkv_prep_validate(self.cfg, args)
        if rc != OK:
            raise QkvPrepError(rc, "qkv_prep_validate")
        keep = (self, q, kv, q_norm_w, kv_norm_w, positions, cos_sin, slot_mapping, kv_cache, args)
        return Launch(_lib.qkv_prep_run, (self.handle, ctypes.byref(args), _stream_of(stream, q.device)),
                      "qkv_prep_run", keep)

    def prepare_gather(self, kv_cache, slots, out, stream=None) -> Launch:
        """``gather`` checked and marshalled now; the Launch enqueues it on
        ``stream`` (default: the current torch stream at this call)."""
        import torch
        check_gather_tensors(self.cfg.block_size, torch.device("cuda", self.device), kv_cache, slots, out)
        args = self._gather_args(kv_cache, slots, out)
        keep = (self, kv_cache, slots, out, args)
        return Launch(_lib.qkv_prep_gather, (self.handle, ctypes.byref(args), _stream_of(stream, out.device)),
                      "qkv_prep_gather", keep)

    def _gather_args(self, kv_cache, slots, out):
        import torch
        return QkvPrepGatherArgs(kv_cache.data_ptr(), kv_cache.numel() // (self.cfg.block_size * SLOT_BYTES),
                                 slots.data_ptr(), slots.numel(), out.data_ptr(),
                                 OUT_F32 if out.dtype == torch.float32 else OUT_BF16)

    def gather(self, kv_cache, slots, out, stream=None):
        """Read `slots` back out of an FP8 cache into `out` ([n, 512] fp32 or bf16)."""
        import torch
        check_gather_tensors(self.cfg.block_size, torch.device("cuda", self.device), kv_cache, slots, out)
        args = self._gather_args(kv_cache, slots, out)
        if stream is None:
            stream = torch.cuda.current_stream(out.device).cuda_stream
        qkv_prep_gather(self.handle, args, stream)
        return out

    def launch_shape(self, num_tokens, num_cus=256) -> QkvPrepLaunch:
        return qkv_prep_launch_shape(self.cfg, num_cus, num_tokens)

    def close(self):
        """Destroy the handle.  A Launch prepared from this object shares the
        handle's ctypes cell, which is cleared here, so calling it afterwards
        raises (invalid argument) instead of using a freed handle."""
        h, self.handle = self.handle, None
        if h:
            qkv_prep_destroy(h)
            h.value = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
