"""ctypes binding of liblbf.so (C ABI in include/lbf.h).

Argument marshalling only: every step of encode, decode and the fused
products runs in the library's HIP kernels.  PyTorch provides device memory
and the current stream.  The library must be built (``__graft_entry__.build()``
or ``python -m decode_byte_split_amd.build_lib``); importing this module
without it raises, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblbf.so")

LBF_OK = 0
LBF_E_INVAL = -1
LBF_E_SHAPE = -2
LBF_E_ALIGN = -3
LBF_E_DESC = -4
LBF_E_CAPACITY = -5
LBF_E_HIP = -6
LBF_E_UNSUPPORTED = -7
LBF_F32 = 0
LBF_BF16 = 1
TILE = 1024
MAX_GROUPS = 64
NOALLOC_SCRATCH_BYTES = 1 << 20  # LBF_NOALLOC_SCRATCH_BYTES: lbf_encode_noalloc's workspace


class Desc(ctypes.Structure):
    """Mirror of ``lbf_desc`` (96 bytes, the first bytes of every blob)."""

    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("version", ctypes.c_uint16),
        ("tile_log2", ctypes.c_uint16),
        ("rows", ctypes.c_uint64),
        ("cols", ctypes.c_uint64),
        ("n_esc", ctypes.c_uint64),
        ("off_raw", ctypes.c_uint64),
        ("off_nib", ctypes.c_uint64),
        ("off_idx", ctypes.c_uint64),
        ("off_esc", ctypes.c_uint64),
        ("blob_bytes", ctypes.c_uint64),
        ("lut", ctypes.c_uint8 * 16),
        ("n_codes", ctypes.c_uint8),
        ("reserved", ctypes.c_uint8 * 3),
        ("desc_crc", ctypes.c_uint32),
    ]

    def to_bytes(self) -> bytes:
        return ctypes.string_at(ctypes.addressof(self), ctypes.sizeof(self))

    @classmethod
    def from_bytes(cls, b) -> "Desc":
        b = bytes(b)[:ctypes.sizeof(cls)]
        return cls.from_buffer_copy(b)


assert ctypes.sizeof(Desc) == 96


class HDesc(ctypes.Structure):
    """Mirror of ``lbf_hdesc`` (128 bytes, the first bytes of every K15H blob)."""

    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("version", ctypes.c_uint16),
        ("tile_log2", ctypes.c_uint16),
        ("rows", ctypes.c_uint64),
        ("cols", ctypes.c_uint64),
        ("n_esc", ctypes.c_uint64),
        ("off_raw", ctypes.c_uint64),
        ("off_bits", ctypes.c_uint64),
        ("off_woff", ctypes.c_uint64),
        ("off_idx", ctypes.c_uint64),
        ("off_esc", ctypes.c_uint64),
        ("blob_bytes", ctypes.c_uint64),
        ("stream_words", ctypes.c_uint64),
        ("lut", ctypes.c_uint8 * 16),
        ("n_codes", ctypes.c_uint8),
        ("max_len", ctypes.c_uint8),
        ("reserved", ctypes.c_uint8 * 2),
        ("len", ctypes.c_uint8 * 16),
        ("desc_crc", ctypes.c_uint32),
    ]

    def to_bytes(self) -> bytes:
        return ctypes.string_at(ctypes.addressof(self), ctypes.sizeof(self))

    @classmethod
    def from_bytes(cls, b) -> "HDesc":
        b = bytes(b)[:ctypes.sizeof(cls)]
        return cls.from_buffer_copy(b)


assert ctypes.sizeof(HDesc) == 128


class LbfError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (what, strerror(status), status))


_lib = None


def lib():
    """Load liblbf.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("liblbf.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, u64, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int
        dp = ctypes.POINTER(Desc)
        vpp = ctypes.POINTER(ctypes.c_void_p)
        L.lbf_strerror.restype = ctypes.c_char_p
        L.lbf_strerror.argtypes = [i32]
        L.lbf_encode_work_bytes.restype = u64
        L.lbf_encode_work_bytes.argtypes = [u64, u64]
        L.lbf_desc_check.restype = i32
        L.lbf_desc_check.argtypes = [dp]
        L.lbf_encode.restype = i32
        L.lbf_encode.argtypes = [vp, u64, u64, vp, u64, vp, u64, dp, vp]
        L.lbf_encode_noalloc.restype = i32
        L.lbf_encode_noalloc.argtypes = [vp, u64, u64, vp, u64, dp, vp]
        L.lbf_decode.restype = i32
        L.lbf_decode.argtypes = [dp, vp, vp, vp]
        L.lbf_verify.restype = i32
        L.lbf_verify.argtypes = [dp, vp, vp, vp]
        L.lbf_crc32.restype = i32
        L.lbf_crc32.argtypes = [vp, u64, vp, vp]
        L.lbf_gemv_swiglu.restype = i32
        L.lbf_gemv_swiglu.argtypes = [dp, vp, dp, vp, vp, i32, vp, i32, vp]
        hp = ctypes.POINTER(HDesc)
        L.lbf_hdesc_check.restype = i32
        L.lbf_hdesc_check.argtypes = [hp]
        L.lbf_hencode_work_bytes.restype = u64
        L.lbf_hencode_work_bytes.argtypes = [dp]
        L.lbf_hencode.restype = i32
        L.lbf_hencode.argtypes = [dp, vp, vp, u64, vp, u64, hp, vp]
        L.lbf_hdecode.restype = i32
        L.lbf_hdecode.argtypes = [hp, vp, vp, vp]
        for name in ("lbf_gemv", "lbf_gemm"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [dp, vpp, i32, vpp, i32, vpp, i32, vp]
        _lib = L
    return _lib


EXPORTS = ("lbf_strerror", "lbf_encode_work_bytes", "lbf_desc_check", "lbf_encode", "lbf_encode_noalloc",
           "lbf_decode", "lbf_verify",
           "lbf_crc32", "lbf_gemv", "lbf_gemm", "lbf_gemv_swiglu", "lbf_hdesc_check", "lbf_hencode_work_bytes", "lbf_hencode",
           "lbf_hdecode")


def strerror(status: int) -> str:
    return lib().lbf_strerror(status).decode()


def desc_check(d: Desc) -> int:
    return int(lib().lbf_desc_check(ctypes.byref(d)))


def _torch():
    import torch

    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _order_after_current(stream) -> None:
    """Work this module enqueues on an explicit ``stream`` reads tensors that
    were made (copies, fresh allocations) on the current stream: make
    ``stream`` wait for everything enqueued there so far."""
    if stream is not None:
        torch = _torch()
        cur = torch.cuda.current_stream(stream.device)
        if cur != stream:
            stream.wait_stream(cur)


def _keep_for(stream, *tensors) -> None:
    """Tensors used by work on an explicit ``stream`` stay allocated until
    that work is done, whatever happens to them on the current stream."""
    if stream is not None:
        for t in tensors:
            t.record_stream(stream)


def _ptr(t) -> int:
    return int(t.data_ptr())


@dataclass
class Blob:
    """A coded weight tensor: host descriptor + device blob (torch uint8)."""

    desc: Desc
    data: "object"  # torch.Tensor, uint8, on the GPU

    @property
    def rows(self) -> int:
        return int(self.desc.rows)

    @property
    def cols(self) -> int:
        return int(self.desc.cols)

    @property
    def n_esc(self) -> int:
        return int(self.desc.n_esc)

    @property
    def nbytes(self) -> int:
        return int(self.desc.blob_bytes)


def _check(rc: int, what: str):
    if rc != LBF_OK:
        raise LbfError(rc, what)


def _check_blob(blob, desc=None):
    """The device buffer must hold at least the descriptor's blob_bytes (the
    kernels read that far) and sit on the GPU."""
    d = blob.desc if desc is None else desc
    t = blob.data
    if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() < int(d.blob_bytes):
        raise ValueError("blob data must be a contiguous GPU buffer of at least %d bytes" % int(d.blob_bytes))


def _check_word(t, what: str):
    if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() < 4:
        raise ValueError("%s must be a contiguous GPU tensor of at least 4 bytes" % what)


def _check_tensor(t, numel: int, dtype, what: str):
    """The library writes or reads exactly `numel` elements of `dtype` at
    t.data_ptr(): refuse anything that would let it run past the tensor."""
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous() or t.numel() != numel:
        raise ValueError("%s must be a contiguous %s tensor of %d elements on the GPU" % (what, dtype, numel))


def encode(w, stream=None) -> Blob:
    """Code a 2-D BF16 tensor (torch.bfloat16 or int16/uint16 bit patterns on the GPU)."""
    torch = _torch()
    if w.dim() != 2 or not w.is_cuda or w.element_size() != 2:
        raise ValueError("encode takes a 2-D 16-bit tensor on the GPU")
    w = w.contiguous()
    rows, cols = w.shape
    L = lib()
    s = _stream(stream)
    wb = int(L.lbf_encode_work_bytes(rows, cols))
    work = torch.empty(max(wb, 256), dtype=torch.uint8, device=w.device)
    _order_after_current(stream)  # the contiguous copy and the workspace come from the current stream
    d = Desc()
    _check(L.lbf_encode(_ptr(w), rows, cols, _ptr(work), work.numel(), None, 0, ctypes.byref(d), s), "lbf_encode phase 1")
    blob = torch.empty(int(d.blob_bytes), dtype=torch.uint8, device=w.device)
    _order_after_current(stream)
    _check(L.lbf_encode(_ptr(w), rows, cols, _ptr(work), work.numel(), _ptr(blob), blob.numel(), ctypes.byref(d), s),
           "lbf_encode phase 2")
    _keep_for(stream, w, work, blob)
    return Blob(d, blob)


def from_host_blob(blob_bytes: np.ndarray, device="cuda") -> Blob:
    """Wrap a blob produced elsewhere (e.g. a saved file) as a device Blob."""
    torch = _torch()
    b = np.ascontiguousarray(blob_bytes, dtype=np.uint8)
    d = Desc.from_bytes(b[:96].tobytes())
    _check(desc_check(d), "blob header")
    t = torch.from_numpy(b.copy()).to(device)
    return Blob(d, t)


def decode(blob: Blob, out=None, stream=None):
    """Rebuild the exact BF16 tensor (torch.bfloat16 [rows, cols])."""
    torch = _torch()
    if out is None:
        out = torch.empty((blob.rows, blob.cols), dtype=torch.bfloat16, device=blob.data.device)
    _check_blob(blob)
    _check_tensor(out, blob.rows * blob.cols, torch.bfloat16, "out")
    _order_after_current(stream)
    _check(lib().lbf_decode(ctypes.byref(blob.desc), _ptr(blob.data), _ptr(out), _stream(stream)), "lbf_decode")
    _keep_for(stream, out)
    return out


def swiglu(gate: Blob, up: Blob, x, h_dtype: int = LBF_F32, out=None, stream=None):
    """h = silu(gate x) * (up x) in one launch (x: bf16 [batch, cols], batch 1..8)."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != gate.cols or not x.is_cuda:
        raise ValueError("x must be bfloat16 [batch, cols of the weights] on the GPU")
    x = x.contiguous()
    batch = int(x.shape[0])
    hdt = torch.float32 if h_dtype == LBF_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((batch, gate.rows), dtype=hdt, device=x.device)
    _check_blob(gate)
    _check_blob(up)
    _check_tensor(out, batch * gate.rows, hdt, "out")
    _order_after_current(stream)  # x may be a fresh contiguous copy
    _check(lib().lbf_gemv_swiglu(ctypes.byref(gate.desc), _ptr(gate.data), ctypes.byref(up.desc), _ptr(up.data),
                                 _ptr(x), batch, _ptr(out), h_dtype, _stream(stream)), "lbf_gemv_swiglu")
    _keep_for(stream, x, out)
    return out


@dataclass
class HBlob:
    """An entropy-coded (K15H) weight tensor: host descriptor + device blob."""

    desc: HDesc
    data: "object"  # torch.Tensor, uint8, on the GPU

    @property
    def rows(self) -> int:
        return int(self.desc.rows)

    @property
    def cols(self) -> int:
        return int(self.desc.cols)

    @property
    def n_esc(self) -> int:
        return int(self.desc.n_esc)

    @property
    def nbytes(self) -> int:
        return int(self.desc.blob_bytes)


def hdesc_check(d: HDesc) -> int:
    return int(lib().lbf_hdesc_check(ctypes.byref(d)))


def hencode(blob: Blob, stream=None) -> HBlob:
    """Re-code a format-v1 blob as an entropy-coded K15H blob on the GPU."""
    torch = _torch()
    L = lib()
    s = _stream(stream)
    _check_blob(blob)
    wb = int(L.lbf_hencode_work_bytes(ctypes.byref(blob.desc)))
    if wb == 0:
        raise LbfError(LBF_E_DESC, "lbf_hencode_work_bytes")
    work = torch.empty(wb, dtype=torch.uint8, device=blob.data.device)
    _order_after_current(stream)
    h = HDesc()
    _check(L.lbf_hencode(ctypes.byref(blob.desc), _ptr(blob.data), _ptr(work), wb, None, 0, ctypes.byref(h), s),
           "lbf_hencode phase 1")
    out = torch.empty(int(h.blob_bytes), dtype=torch.uint8, device=blob.data.device)
    _order_after_current(stream)
    _check(L.lbf_hencode(ctypes.byref(blob.desc), _ptr(blob.data), _ptr(work), wb, _ptr(out), out.numel(),
                         ctypes.byref(h), s), "lbf_hencode phase 2")
    _keep_for(stream, work, out)
    return HBlob(h, out)


def from_host_hblob(blob_bytes: np.ndarray, device="cuda") -> HBlob:
    """Wrap a K15H blob produced elsewhere as a device HBlob."""
    torch = _torch()
    b = np.ascontiguousarray(blob_bytes, dtype=np.uint8)
    d = HDesc.from_bytes(b[:128].tobytes())
    _check(hdesc_check(d), "K15H blob header")
    return HBlob(d, torch.from_numpy(b.copy()).to(device))


def hdecode(blob: HBlob, out=None, stream=None):
    """Rebuild the exact BF16 tensor from a K15H blob."""
    torch = _torch()
    if out is None:
        out = torch.empty((blob.rows, blob.cols), dtype=torch.bfloat16, device=blob.data.device)
    _check_blob(blob)
    _check_tensor(out, blob.rows * blob.cols, torch.bfloat16, "out")
    _order_after_current(stream)
    _check(lib().lbf_hdecode(ctypes.byref(blob.desc), _ptr(blob.data), _ptr(out), _stream(stream)), "lbf_hdecode")
    _keep_for(stream, out)
    return out


VERIFY_HEADER, VERIFY_INDEX, VERIFY_COUNT, VERIFY_CODE, VERIFY_ESCAPE, VERIFY_PADDING = 1, 2, 4, 8, 16, 32


def verify_into(blob: Blob, flags, desc: Desc | None = None, stream=None) -> None:
    """Enqueue the structural check of a device blob against ``desc`` (default:
    its own descriptor); the failed-check mask lands in ``flags`` (a one-element
    int32 or uint32 device tensor) when the stream reaches it.  Does not wait."""
    d = blob.desc if desc is None else desc
    _check_blob(blob, d)
    _check_word(flags, "flags")
    _check(lib().lbf_verify(ctypes.byref(d), _ptr(blob.data), _ptr(flags), _stream(stream)), "lbf_verify")


def verify(blob: Blob, desc: Desc | None = None, stream=None) -> int:
    """Structural check of a device blob against ``desc`` (default: its own
    descriptor) on the GPU; returns the failed-check mask (0: all pass).
    Waits for the stream."""
    torch = _torch()
    flags = torch.empty(1, dtype=torch.int32, device=blob.data.device)
    _order_after_current(stream)
    verify_into(blob, flags, desc, stream)
    if stream is not None:
        stream.synchronize()
    return int(flags.item()) & 0xFFFFFFFF


def crc32_into(t, out, stream=None) -> None:
    """Enqueue zlib's CRC-32 of a contiguous device tensor's bytes into ``out``
    (a one-element int32 or uint32 device tensor).  Does not wait."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("crc32 takes a contiguous tensor on the GPU")
    _check_word(out, "out")
    _check(lib().lbf_crc32(_ptr(t), t.numel() * t.element_size(), _ptr(out), _stream(stream)), "lbf_crc32")


def crc32(t, stream=None) -> int:
    """CRC-32 (zlib's) of a contiguous device tensor's bytes, on the GPU.
    Waits for the stream."""
    torch = _torch()
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("crc32 takes a contiguous tensor on the GPU")
    out = torch.empty(1, dtype=torch.int32, device=t.device)
    _order_after_current(stream)
    crc32_into(t, out, stream)
    if stream is not None:
        stream.synchronize()
    return int(out.item()) & 0xFFFFFFFF


class Prepared:
    """One fused product with its arguments marshalled once: each call is a
    single lbf_gemv / lbf_gemm call on the stream captured at preparation.
    Holds references to every tensor it points at."""

    def __init__(self, fn, what, blobs: Sequence[Blob], xs, y_dtype, outs, stream):
        torch = _torch()
        n = len(blobs)
        if len(xs) != n:
            raise ValueError("one x per blob")
        for b in blobs:
            _check_blob(b)
        batch = int(xs[0].shape[0])
        xs = [x.contiguous() for x in xs]
        for x, b in zip(xs, blobs):
            if (x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[0] != batch or x.shape[1] != b.cols
                    or not x.is_cuda):
                raise ValueError("x must be bfloat16 [batch, cols] on the GPU with the same batch for every group")
        tdt = torch.float32 if y_dtype == LBF_F32 else torch.bfloat16
        if outs is None:
            outs = [torch.empty((batch, b.rows), dtype=tdt, device=b.data.device) for b in blobs]
        if len(outs) != n:
            raise ValueError("one output per blob")
        for y, b in zip(outs, blobs):
            _check_tensor(y, batch * b.rows, tdt, "each output")
        # x copies and fresh outputs were made on the current stream: the
        # launch stream waits for them once, and keeps them while it uses them
        _order_after_current(stream)
        _keep_for(stream, *xs, *outs)
        self._keep = (list(blobs), xs, outs)
        self.outs = outs
        self._fn, self._what = fn, what
        self._args = ((Desc * n)(*[b.desc for b in blobs]), (ctypes.c_void_p * n)(*[_ptr(b.data) for b in blobs]), n,
                      (ctypes.c_void_p * n)(*[_ptr(x) for x in xs]), batch,
                      (ctypes.c_void_p * n)(*[_ptr(y) for y in outs]), y_dtype, _stream(stream))

    def __call__(self):
        _check(self._fn(*self._args), self._what)
        return self.outs


def _product(fn, what, blobs: Sequence[Blob], xs, y_dtype, outs, stream):
    return Prepared(fn, what, blobs, xs, y_dtype, outs, stream)()


def prepare(blobs, xs, y_dtype: int = LBF_F32, outs=None, stream=None) -> Prepared:
    """Marshal a grouped product once (gemv for batch 1..8, gemm above); the
    returned object launches it when called."""
    if isinstance(blobs, Blob):
        blobs, xs = [blobs], [xs]
        outs = None if outs is None else [outs]
    b = int(xs[0].shape[0])
    L = lib()
    fn, what = (L.lbf_gemv, "lbf_gemv") if b <= 8 else (L.lbf_gemm, "lbf_gemm")
    return Prepared(fn, what, blobs, xs, y_dtype, outs, stream)


def gemv(blobs, xs, y_dtype: int = LBF_F32, outs=None, stream=None):
    """Fused decode-GEMV, batch 1..8: y_g = x_g @ W_g^T for each group (one launch)."""
    single = isinstance(blobs, Blob)
    if single:
        blobs, xs = [blobs], [xs]
        outs = None if outs is None else [outs]
    ys = _product(lib().lbf_gemv, "lbf_gemv", blobs, xs, y_dtype, outs, stream)
    return ys[0] if single else ys


def gemm(blobs, xs, y_dtype: int = LBF_BF16, outs=None, stream=None):
    """Fused decode-GEMM on MFMA, batch >= 9."""
    single = isinstance(blobs, Blob)
    if single:
        blobs, xs = [blobs], [xs]
        outs = None if outs is None else [outs]
    ys = _product(lib().lbf_gemm, "lbf_gemm", blobs, xs, y_dtype, outs, stream)
    return ys[0] if single else ys


def matmul(blobs, xs, y_dtype: int = LBF_F32, outs=None, stream=None):
    """Dispatch by batch: gemv for 1..8, gemm above."""
    b = (xs if not isinstance(blobs, Blob) else [xs])[0].shape[0]
    return (gemv if b <= 8 else gemm)(blobs, xs, y_dtype, outs, stream)
