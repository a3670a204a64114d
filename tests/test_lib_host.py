"""Host-side checks of liblbf.so that need no GPU: it loads, exports every
symbol include/lbf.h declares, and its descriptor validation (which runs before
any launch) agrees with the oracle's header and rejects corrupt descriptors."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lbf():
    from decode_byte_split_amd import lbf

    return lbf


def test_header_declarations_are_exported():
    lbf = _lbf()
    L = lbf.lib()
    with open(os.path.join(ROOT, "include", "lbf.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(lbf_\w+)\s*\(", text, flags=re.M))
    assert declared, "no declarations found"
    assert declared == set(lbf.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_strerror():
    lbf = _lbf()
    assert lbf.strerror(0) == "ok"
    assert "descriptor" in lbf.strerror(lbf.LBF_E_DESC)


def test_work_bytes():
    lbf = _lbf()
    n = lbf.lib().lbf_encode_work_bytes(14336, 4096)
    assert n >= 1024 + 4 * (14336 * 4096 // 1024)
    assert lbf.lib().lbf_encode_work_bytes(1 << 20, 1 << 20) == 0  # n >= 2^32


def _oracle_desc(W):
    lbf = _lbf()
    blob = O.encode(W)
    return lbf.Desc.from_bytes(blob[:96].tobytes()), blob


@pytest.mark.parametrize("shape", [(1024, 1024), (3, 5), (0, 8), (256, 256)])
def test_oracle_headers_pass_library_check(shape):
    lbf = _lbf()
    if shape == (256, 256):
        W = synth.all_patterns(256, 256)
    else:
        W = synth.gaussian(np.random.default_rng(1), shape[0], shape[1], 0.02, 0.001, 100.0)
    d, blob = _oracle_desc(W)
    assert lbf.desc_check(d) == 0
    assert d.blob_bytes == blob.size


def test_corrupt_descriptors_rejected():
    lbf = _lbf()
    W, _ = synth.single_tensor()
    d, _ = _oracle_desc(W)
    raw = bytearray(d.to_bytes())
    for off in range(0, 96):
        bad = bytearray(raw)
        bad[off] ^= 0x10
        bd = lbf.Desc.from_bytes(bytes(bad))
        assert lbf.desc_check(bd) == lbf.LBF_E_DESC, off


def test_self_consistent_but_invalid_descriptors_rejected():
    # fields re-signed with a valid CRC but violating the format's invariants
    lbf = _lbf()
    W, _ = synth.single_tensor()
    d, _ = _oracle_desc(W)

    def resign(x):
        x.desc_crc = O.crc32(np.frombuffer(x.to_bytes()[:92], dtype=np.uint8))
        return x

    assert lbf.desc_check(resign(lbf.Desc.from_bytes(d.to_bytes()))) == 0
    bad = lbf.Desc.from_bytes(d.to_bytes())
    bad.lut[0], bad.lut[1] = bad.lut[1], bad.lut[0]  # table not ascending
    assert lbf.desc_check(resign(bad)) == lbf.LBF_E_DESC
    bad = lbf.Desc.from_bytes(d.to_bytes())
    bad.off_esc += 256
    assert lbf.desc_check(resign(bad)) == lbf.LBF_E_DESC
    bad = lbf.Desc.from_bytes(d.to_bytes())
    bad.n_esc = bad.rows * bad.cols + 1
    assert lbf.desc_check(resign(bad)) == lbf.LBF_E_DESC
    bad = lbf.Desc.from_bytes(d.to_bytes())
    bad.n_codes = 16
    assert lbf.desc_check(resign(bad)) == lbf.LBF_E_DESC


def test_calls_validate_before_touching_the_gpu():
    # A corrupt descriptor is refused before any HIP call, so this runs on a
    # machine without a GPU; the pointers are never dereferenced.
    lbf = _lbf()
    L = lbf.lib()
    W, _ = synth.single_tensor()
    d, _ = _oracle_desc(W)
    bad = lbf.Desc.from_bytes(d.to_bytes())
    bad.rows += 1
    assert L.lbf_decode(ctypes.byref(bad), 256, 256, None) == lbf.LBF_E_DESC
    descs = (lbf.Desc * 1)(bad)
    p = (ctypes.c_void_p * 1)(256)
    assert L.lbf_gemv(descs, p, 1, p, 1, p, 0, None) == lbf.LBF_E_DESC
    good = (lbf.Desc * 1)(d)
    assert L.lbf_gemv(good, p, 1, p, 9, p, 0, None) == lbf.LBF_E_INVAL  # batch 9 is not a GEMV
    assert L.lbf_gemv(good, p, 1, p, 1, p, 7, None) == lbf.LBF_E_INVAL  # unknown output type
    assert L.lbf_gemm(good, p, 1, p, 8, p, 0, None) == lbf.LBF_E_INVAL
    assert L.lbf_gemm(good, p, 1, p, 257, p, 0, None) == lbf.LBF_E_INVAL
    wide = _oracle_desc(np.zeros((1, 16385 * 1024), dtype=np.uint16))[0]  # 16,385 tiles per row
    assert L.lbf_gemm((lbf.Desc * 1)(wide), p, 1, p, 16, p, 0, None) == lbf.LBF_E_UNSUPPORTED
    misaligned = (ctypes.c_void_p * 1)(256 + 8)
    assert L.lbf_gemv(good, misaligned, 1, p, 1, p, 0, None) == lbf.LBF_E_ALIGN
    small = _oracle_desc(np.zeros((3, 5), dtype=np.uint16))[0]
    assert L.lbf_gemv((lbf.Desc * 1)(small), p, 1, p, 1, p, 0, None) == lbf.LBF_E_SHAPE  # cols % 1024
    assert L.lbf_encode(256, 1 << 20, 1 << 20, 256, 1 << 30, None, 0, ctypes.byref(lbf.Desc()), None) == lbf.LBF_E_SHAPE
    assert L.lbf_verify(ctypes.byref(bad), 256, 256, None) == lbf.LBF_E_DESC
    assert L.lbf_verify(ctypes.byref(d), 256 + 16, 256, None) == lbf.LBF_E_ALIGN
    assert L.lbf_verify(ctypes.byref(d), 256, 258, None) == lbf.LBF_E_ALIGN
    assert L.lbf_verify(ctypes.byref(d), None, 256, None) == lbf.LBF_E_INVAL
    assert L.lbf_crc32(256 + 4, 100, 256, None) == lbf.LBF_E_ALIGN
    assert L.lbf_crc32(None, 100, 256, None) == lbf.LBF_E_INVAL
    assert L.lbf_crc32(256, 100, None, None) == lbf.LBF_E_INVAL


# ---- K15H descriptors -----------------------------------------------------------

def _oracle_hdesc(W):
    lbf = _lbf()
    blob = O.hencode(W)
    return lbf.HDesc.from_bytes(blob[:128].tobytes()), blob


@pytest.mark.parametrize("case", ["gauss", "ragged", "empty", "patterns", "one_symbol", "outliers"])
def test_oracle_hheaders_pass_library_check(case):
    lbf = _lbf()
    rng = np.random.default_rng(2)
    W = {"gauss": lambda: synth.gaussian(rng, 64, 1024, 0.02, 0.001, 100.0),
         "ragged": lambda: synth.gaussian(rng, 3, 5, 0.02, 0.0, 1.0),
         "empty": lambda: np.zeros((0, 8), dtype=np.uint16),
         "patterns": lambda: synth.all_patterns(64, 1024),
         "one_symbol": lambda: np.full((2, 1500), 0x3F80, dtype=np.uint16),
         "outliers": lambda: synth.gaussian(rng, 16, 1024, 0.02, 0.2, 100.0)}[case]()
    h, blob = _oracle_hdesc(W)
    assert lbf.hdesc_check(h) == 0
    assert h.blob_bytes == blob.size
    # the library's own code lengths for the oracle's counts are the oracle's
    d, _ = _oracle_desc(W)
    assert lbf.lib().lbf_hencode_work_bytes(ctypes.byref(d)) >= 256 + 4 * (2 * ((W.size + 1023) // 1024) + 1)


def test_corrupt_hdescriptors_rejected():
    lbf = _lbf()
    h, _ = _oracle_hdesc(synth.gaussian(np.random.default_rng(3), 8, 1024, 0.02, 0.001, 100.0))
    raw = bytearray(h.to_bytes())
    for off in range(0, 128):
        bad = bytearray(raw)
        bad[off] ^= 0x10
        assert lbf.hdesc_check(lbf.HDesc.from_bytes(bytes(bad))) == lbf.LBF_E_DESC, off


def test_self_consistent_but_invalid_hdescriptors_rejected():
    lbf = _lbf()
    h, _ = _oracle_hdesc(synth.gaussian(np.random.default_rng(4), 8, 1024, 0.02, 0.001, 100.0))

    def resign(x):
        x.desc_crc = O.crc32(np.frombuffer(x.to_bytes()[:124], dtype=np.uint8))
        return x

    def variant(edit):
        x = lbf.HDesc.from_bytes(h.to_bytes())
        edit(x)
        return lbf.hdesc_check(resign(x))

    assert variant(lambda x: None) == 0
    used = [c for c in range(16) if h.len[c]]
    assert variant(lambda x: x.len.__setitem__(used[0], x.len[used[0]] + 1)) == lbf.LBF_E_DESC  # Kraft sum < 1
    assert variant(lambda x: x.len.__setitem__(used[-1], 16)) == lbf.LBF_E_DESC  # longer than 15
    assert variant(lambda x: setattr(x, "max_len", x.max_len + 1)) == lbf.LBF_E_DESC
    assert variant(lambda x: x.len.__setitem__(14, 0) if h.n_codes == 15 else x.len.__setitem__(13, 3)) == lbf.LBF_E_DESC
    assert variant(lambda x: setattr(x, "stream_words", x.stream_words + 64)) == lbf.LBF_E_DESC  # layout moves
    assert variant(lambda x: setattr(x, "off_bits", x.off_bits + 256)) == lbf.LBF_E_DESC
    assert variant(lambda x: setattr(x, "stream_words", 480 * 8 + 1)) == lbf.LBF_E_DESC  # more than 480 words/tile


def test_hcalls_validate_before_touching_the_gpu():
    lbf = _lbf()
    L = lbf.lib()
    W = synth.gaussian(np.random.default_rng(5), 4, 1024, 0.02, 0.001, 100.0)
    h, _ = _oracle_hdesc(W)
    d, _ = _oracle_desc(W)
    bad = lbf.HDesc.from_bytes(h.to_bytes())
    bad.rows += 1
    assert L.lbf_hdecode(ctypes.byref(bad), 256, 256, None) == lbf.LBF_E_DESC
    assert L.lbf_hdecode(ctypes.byref(h), 256 + 16, 256, None) == lbf.LBF_E_ALIGN
    assert L.lbf_hdecode(ctypes.byref(h), None, 256, None) == lbf.LBF_E_INVAL
    wb = L.lbf_hencode_work_bytes(ctypes.byref(d))
    assert L.lbf_hencode(ctypes.byref(d), 256, 256, wb - 1, None, 0, ctypes.byref(lbf.HDesc()), None) == lbf.LBF_E_CAPACITY
    assert L.lbf_hencode(ctypes.byref(d), 256 + 8, 256, wb, None, 0, ctypes.byref(lbf.HDesc()), None) == lbf.LBF_E_ALIGN
    assert L.lbf_hencode(ctypes.byref(d), None, 256, wb, None, 0, ctypes.byref(lbf.HDesc()), None) == lbf.LBF_E_INVAL
    vbad = lbf.Desc.from_bytes(d.to_bytes())
    vbad.cols += 1
    assert L.lbf_hencode(ctypes.byref(vbad), 256, 256, wb, None, 0, ctypes.byref(lbf.HDesc()), None) == lbf.LBF_E_DESC
    # phase 2 with a K15H descriptor of another tensor
    other, _ = _oracle_hdesc(synth.gaussian(np.random.default_rng(6), 4, 1024, 0.02, 0.001, 100.0))
    if bytes(other.len) != bytes(h.len) or bytes(other.lut) != bytes(h.lut):
        assert L.lbf_hencode(ctypes.byref(d), 256, 256, wb, 256, 1 << 30, ctypes.byref(bad), None) == lbf.LBF_E_DESC
    assert L.lbf_hencode(ctypes.byref(d), 256, 256, wb, 256, h.blob_bytes - 1, ctypes.byref(h), None) == lbf.LBF_E_CAPACITY


def test_swiglu_validates_before_touching_the_gpu():
    lbf = _lbf()
    L = lbf.lib()
    d, _ = _oracle_desc(np.zeros((8, 2048), dtype=np.uint16))
    other, _ = _oracle_desc(np.zeros((8, 3072), dtype=np.uint16))
    wide, _ = _oracle_desc(np.zeros((1, 65536), dtype=np.uint16))
    bad = lbf.Desc.from_bytes(d.to_bytes())
    bad.cols += 1
    r = ctypes.byref
    assert L.lbf_gemv_swiglu(r(bad), 256, r(d), 256, 256, 1, 256, 0, None) == lbf.LBF_E_DESC
    assert L.lbf_gemv_swiglu(r(d), 256, r(other), 256, 256, 1, 256, 0, None) == lbf.LBF_E_SHAPE
    assert L.lbf_gemv_swiglu(r(d), 256, r(d), 256, 256, 9, 256, 0, None) == lbf.LBF_E_INVAL
    assert L.lbf_gemv_swiglu(r(d), 256, r(d), 256, 256, 0, 256, 0, None) == lbf.LBF_E_INVAL
    assert L.lbf_gemv_swiglu(r(d), 256, r(d), 256, 256, 1, 256, 5, None) == lbf.LBF_E_INVAL
    assert L.lbf_gemv_swiglu(None, 256, r(d), 256, 256, 1, 256, 0, None) == lbf.LBF_E_INVAL
    assert L.lbf_gemv_swiglu(r(d), 256 + 64, r(d), 256, 256, 1, 256, 0, None) == lbf.LBF_E_ALIGN
    assert L.lbf_gemv_swiglu(r(d), 256, r(d), 256, 256 + 8, 1, 256, 0, None) == lbf.LBF_E_ALIGN
    assert L.lbf_gemv_swiglu(r(wide), 256, r(wide), 256, 256, 2, 256, 0, None) == lbf.LBF_E_UNSUPPORTED
    small, _ = _oracle_desc(np.zeros((3, 5), dtype=np.uint16))
    assert L.lbf_gemv_swiglu(r(small), 256, r(small), 256, 256, 1, 256, 0, None) == lbf.LBF_E_SHAPE


def test_binding_constants_match_the_header():
    lbf = _lbf()
    with open(os.path.join(ROOT, "include", "lbf.h")) as f:
        text = f.read()
    assert re.search(r"#define LBF_MAX_GROUPS (\d+)", text).group(1) == str(lbf.MAX_GROUPS)
    m = re.search(r"#define LBF_NOALLOC_SCRATCH_BYTES \(1u << (\d+)\)", text)
    assert 1 << int(m.group(1)) == lbf.NOALLOC_SCRATCH_BYTES


def test_noalloc_encode_refuses_before_touching_the_gpu():
    """Sizes past the library's array and bad arguments are refused on the
    host (no GPU in this process)."""
    lbf = _lbf()
    L = lbf.lib()
    d = lbf.Desc()
    big = (lbf.NOALLOC_SCRATCH_BYTES - 1024) // 4 + 1
    assert L.lbf_encode_noalloc(None, big, 1024, None, 0, ctypes.byref(d), None) == lbf.LBF_E_CAPACITY
    assert L.lbf_encode_noalloc(None, 1 << 20, 1 << 20, None, 0, ctypes.byref(d), None) == lbf.LBF_E_SHAPE
    assert L.lbf_encode_noalloc(None, 4, 1024, None, 0, None, None) == lbf.LBF_E_INVAL
