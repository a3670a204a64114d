"""ctypes shim over the CPU oracle (``lbf_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The GPU library and
its Python binding never import this module.  Nothing here does arithmetic of
the method; it only moves numpy arrays in and out of the C functions, whose
header comment cites the pages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lbf_oracle.c")
_LIB = os.path.join(_HERE, "liblbfo.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_f64p = ctypes.POINTER(ctypes.c_double)
_u64 = ctypes.c_uint64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/liblbfo.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        L.lbfo_crc32.restype = ctypes.c_uint32
        L.lbfo_crc32.argtypes = [_u8p, _u64]
        L.lbfo_histogram.restype = None
        L.lbfo_histogram.argtypes = [_u16p, _u64, _u64p]
        L.lbfo_code_table.restype = None
        L.lbfo_code_table.argtypes = [_u64p, _u8p, _u8p]
        L.lbfo_plan.restype = ctypes.c_int
        L.lbfo_plan.argtypes = [_u16p, _u64, _u64, _u8p, _u8p, _u64p, _u64p]
        L.lbfo_encode.restype = ctypes.c_int
        L.lbfo_encode.argtypes = [_u16p, _u64, _u64, _u8p, _u64]
        L.lbfo_read_header.restype = ctypes.c_int
        L.lbfo_read_header.argtypes = [_u8p, _u64, _u64p, _u64p, _u64p, _u8p, _u8p]
        L.lbfo_decode.restype = ctypes.c_int
        L.lbfo_decode.argtypes = [_u8p, _u64, _u16p, _u64]
        L.lbfo_matvec.restype = None
        L.lbfo_matvec.argtypes = [_u16p, _u64, _u64, _u16p, _u64, _f64p, _f64p]
        L.lbfo_matvec_rows.restype = None
        L.lbfo_matvec_rows.argtypes = [_u16p, _u64, _u64, _u64, _u64, _u16p, _u64, _f64p, _f64p]
        L.lbfo_entropy16.restype = ctypes.c_double
        L.lbfo_entropy16.argtypes = [_u16p, _u64]
        L.lbfo_entropy_exponent.restype = ctypes.c_double
        L.lbfo_entropy_exponent.argtypes = [_u16p, _u64]
        L.lbfo_verify.restype = ctypes.c_uint
        L.lbfo_verify.argtypes = [_u8p, _u64, _u8p]
        L.lbfo_silu.restype = ctypes.c_double
        L.lbfo_silu.argtypes = [ctypes.c_double]
        L.lbfo_swiglu.restype = None
        L.lbfo_swiglu.argtypes = [_u16p, _u16p, _u64, _u64, _u16p, _u64, _f64p, _f64p, _f64p, _f64p, _f64p]
        L.lbfo_huffman_lengths.restype = None
        L.lbfo_huffman_lengths.argtypes = [_u64p, _u8p]
        L.lbfo_canonical_codes.restype = None
        L.lbfo_canonical_codes.argtypes = [_u8p, _u16p]
        L.lbfo_hplan.restype = ctypes.c_int
        L.lbfo_hplan.argtypes = [_u16p, _u64, _u64, _u64p, _u8p, _u64p, _u64p]
        L.lbfo_hencode.restype = ctypes.c_int
        L.lbfo_hencode.argtypes = [_u16p, _u64, _u64, _u8p, _u64]
        L.lbfo_hread_header.restype = ctypes.c_int
        L.lbfo_hread_header.argtypes = [_u8p, _u64, _u64p, _u64p, _u64p, _u64p, _u8p, _u8p, _u8p]
        L.lbfo_hdecode.restype = ctypes.c_int
        L.lbfo_hdecode.argtypes = [_u8p, _u64, _u16p, _u64]
        _lib = L
    return _lib


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _bf16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns as uint16, got %s" % a.dtype)
    return a


def crc32(data: bytes | np.ndarray) -> int:
    b = np.frombuffer(bytes(data), dtype=np.uint8) if not isinstance(data, np.ndarray) else data
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return int(lib().lbfo_crc32(_p(b, _u8p), b.size))


def histogram(w: np.ndarray) -> np.ndarray:
    w = _bf16(w).reshape(-1)
    h = np.zeros(256, dtype=np.uint64)
    lib().lbfo_histogram(_p(w, _u16p), w.size, _p(h, _u64p))
    return h


def code_table(hist: np.ndarray) -> tuple[np.ndarray, int]:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    assert h.size == 256
    lut = np.zeros(16, dtype=np.uint8)
    nc = ctypes.c_uint8(0)
    lib().lbfo_code_table(_p(h, _u64p), _p(lut, _u8p), ctypes.byref(nc))
    return lut, int(nc.value)


@dataclass
class Plan:
    lut: np.ndarray
    n_codes: int
    n_esc: int
    blob_bytes: int


def plan(w: np.ndarray) -> Plan:
    w = _bf16(w)
    rows, cols = w.shape
    lut = np.zeros(16, dtype=np.uint8)
    nc = ctypes.c_uint8(0)
    ne = ctypes.c_uint64(0)
    bb = ctypes.c_uint64(0)
    rc = lib().lbfo_plan(_p(w, _u16p), rows, cols, _p(lut, _u8p), ctypes.byref(nc), ctypes.byref(ne),
                         ctypes.byref(bb))
    if rc != 0:
        raise ValueError("oracle plan failed (%d)" % rc)
    return Plan(lut, int(nc.value), int(ne.value), int(bb.value))


def encode(w: np.ndarray) -> np.ndarray:
    """Encode a 2-D uint16 (bf16 bits) array into a format-v1 blob (uint8)."""
    w = _bf16(w)
    if w.ndim != 2:
        raise ValueError("encode takes a 2-D [rows, cols] array")
    rows, cols = w.shape
    pl = plan(w)
    blob = np.zeros(pl.blob_bytes, dtype=np.uint8)
    rc = lib().lbfo_encode(_p(w, _u16p), rows, cols, _p(blob, _u8p), blob.size)
    if rc != 0:
        raise ValueError("oracle encode failed (%d)" % rc)
    return blob


@dataclass
class Header:
    rows: int
    cols: int
    n_esc: int
    lut: np.ndarray
    n_codes: int


def read_header(blob: np.ndarray) -> Header:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    r, c, e = ctypes.c_uint64(0), ctypes.c_uint64(0), ctypes.c_uint64(0)
    lut = np.zeros(16, dtype=np.uint8)
    nc = ctypes.c_uint8(0)
    rc = lib().lbfo_read_header(_p(blob, _u8p), blob.size, ctypes.byref(r), ctypes.byref(c), ctypes.byref(e),
                                _p(lut, _u8p), ctypes.byref(nc))
    if rc != 0:
        raise ValueError("oracle: bad header (%d)" % rc)
    return Header(int(r.value), int(c.value), int(e.value), lut, int(nc.value))


def decode(blob: np.ndarray) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    h = read_header(blob)
    out = np.zeros((h.rows, h.cols), dtype=np.uint16)
    rc = lib().lbfo_decode(_p(blob, _u8p), blob.size, _p(out, _u16p), out.size)
    if rc != 0:
        raise ValueError("oracle decode failed (%d)" % rc)
    return out


VERIFY_HEADER, VERIFY_INDEX, VERIFY_COUNT, VERIFY_CODE, VERIFY_ESCAPE, VERIFY_PADDING = 1, 2, 4, 8, 16, 32


def verify(blob: np.ndarray, desc96: np.ndarray | bytes | None = None) -> int:
    """Bit mask of failed structural checks of ``blob`` against the 96
    descriptor bytes ``desc96`` (default: the blob's own first 96 bytes)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    d = blob[:96].copy() if desc96 is None else np.frombuffer(bytes(desc96), dtype=np.uint8).copy()
    return int(lib().lbfo_verify(_p(blob, _u8p), blob.size, _p(d, _u8p)))


def matvec(W: np.ndarray, x: np.ndarray, rows: tuple[int, int] | None = None):
    """y[b, r] = sum_k W[r, k] x[b, k] in float64, and A[b, r] = sum |W||x|.

    ``W`` is [rows, cols] bf16 bits; ``x`` is [batch, cols] bf16 bits.  With
    ``rows=(r0, r1)`` only that row range is computed; outputs are
    [batch, r1 - r0].
    """
    W = _bf16(W)
    x = _bf16(x)
    if x.ndim == 1:
        x = x[None, :]
    R, K = W.shape
    B = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x has %d columns, W has %d" % (x.shape[1], K))
    if rows is None:
        y = np.zeros((B, R), dtype=np.float64)
        a = np.zeros((B, R), dtype=np.float64)
        lib().lbfo_matvec(_p(W, _u16p), R, K, _p(x, _u16p), B, _p(y, _f64p), _p(a, _f64p))
    else:
        r0, r1 = rows
        r1 = min(r1, R)
        y = np.zeros((B, r1 - r0), dtype=np.float64)
        a = np.zeros((B, r1 - r0), dtype=np.float64)
        lib().lbfo_matvec_rows(_p(W, _u16p), R, K, r0, r1, _p(x, _u16p), B, _p(y, _f64p), _p(a, _f64p))
    return y, a


def entropy16(w: np.ndarray) -> float:
    w = _bf16(w).reshape(-1)
    return float(lib().lbfo_entropy16(_p(w, _u16p), w.size))


def entropy_exponent(w: np.ndarray) -> float:
    w = _bf16(w).reshape(-1)
    return float(lib().lbfo_entropy_exponent(_p(w, _u16p), w.size))


# ---- the entropy-coded variant (K15H) --------------------------------------


def huffman_lengths(count) -> np.ndarray:
    """Huffman code lengths (uint8[16]) of 16 symbols from their counts."""
    c = np.ascontiguousarray(count, dtype=np.uint64)
    assert c.size == 16
    out = np.zeros(16, dtype=np.uint8)
    lib().lbfo_huffman_lengths(_p(c, _u64p), _p(out, _u8p))
    return out


def canonical_codes(lengths) -> np.ndarray:
    """Canonical code values (uint16[16]) for 16 code lengths (0 = unused)."""
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    assert ln.size == 16
    out = np.zeros(16, dtype=np.uint16)
    lib().lbfo_canonical_codes(_p(ln, _u8p), _p(out, _u16p))
    return out


@dataclass
class HPlan:
    code_count: np.ndarray
    lengths: np.ndarray
    stream_words: int
    blob_bytes: int


def hplan(w: np.ndarray) -> HPlan:
    w = _bf16(w)
    rows, cols = w.shape
    cc = np.zeros(16, dtype=np.uint64)
    ln = np.zeros(16, dtype=np.uint8)
    sw, bb = ctypes.c_uint64(0), ctypes.c_uint64(0)
    rc = lib().lbfo_hplan(_p(w, _u16p), rows, cols, _p(cc, _u64p), _p(ln, _u8p), ctypes.byref(sw), ctypes.byref(bb))
    if rc != 0:
        raise ValueError("oracle hplan failed (%d)" % rc)
    return HPlan(cc, ln, int(sw.value), int(bb.value))


def hencode(w: np.ndarray) -> np.ndarray:
    """Encode a 2-D uint16 (bf16 bits) array into a K15H blob (uint8)."""
    w = _bf16(w)
    if w.ndim != 2:
        raise ValueError("hencode takes a 2-D [rows, cols] array")
    rows, cols = w.shape
    pl = hplan(w)
    blob = np.zeros(pl.blob_bytes, dtype=np.uint8)
    rc = lib().lbfo_hencode(_p(w, _u16p), rows, cols, _p(blob, _u8p), blob.size)
    if rc != 0:
        raise ValueError("oracle hencode failed (%d)" % rc)
    return blob


@dataclass
class HHeader:
    rows: int
    cols: int
    n_esc: int
    stream_words: int
    lut: np.ndarray
    n_codes: int
    lengths: np.ndarray


def hread_header(blob: np.ndarray) -> HHeader:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    r, c, e, sw = (ctypes.c_uint64(0) for _ in range(4))
    lut = np.zeros(16, dtype=np.uint8)
    ln = np.zeros(16, dtype=np.uint8)
    nc = ctypes.c_uint8(0)
    rc = lib().lbfo_hread_header(_p(blob, _u8p), blob.size, ctypes.byref(r), ctypes.byref(c), ctypes.byref(e),
                                 ctypes.byref(sw), _p(lut, _u8p), ctypes.byref(nc), _p(ln, _u8p))
    if rc != 0:
        raise ValueError("oracle: bad K15H header (%d)" % rc)
    return HHeader(int(r.value), int(c.value), int(e.value), int(sw.value), lut, int(nc.value), ln)


def hdecode(blob: np.ndarray) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    h = hread_header(blob)
    out = np.zeros((h.rows, h.cols), dtype=np.uint16)
    rc = lib().lbfo_hdecode(_p(blob, _u8p), blob.size, _p(out, _u16p), out.size)
    if rc != 0:
        raise ValueError("oracle hdecode failed (%d)" % rc)
    return out


# ---- the gated MLP product ---------------------------------------------------


def silu(z: float) -> float:
    return float(lib().lbfo_silu(float(z)))


def swiglu(G: np.ndarray, U: np.ndarray, x: np.ndarray):
    """h[b, r] = silu(G x)[b, r] * (U x)[b, r] in float64; also g, u, and the
    magnitude sums ag = sum |G||x|, au = sum |U||x| (all [batch, rows])."""
    G, U, x = _bf16(G), _bf16(U), _bf16(x)
    if x.ndim == 1:
        x = x[None, :]
    R, K = G.shape
    if U.shape != G.shape or x.shape[1] != K:
        raise ValueError("gate and up must have one shape, x one column per input")
    B = x.shape[0]
    out = [np.zeros((B, R), dtype=np.float64) for _ in range(5)]
    lib().lbfo_swiglu(_p(G, _u16p), _p(U, _u16p), R, K, _p(x, _u16p), B, *[_p(o, _f64p) for o in out])
    return tuple(out)  # h, g, u, ag, au
