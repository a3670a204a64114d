"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Every check here is independent of the oracle's own code: hand-worked golden
fixtures (tests/golden/, each citing its source), closed forms, the exhaustive
round trip over all 65,536 BF16 patterns, library routines (zlib's CRC-32,
numpy float64 matmul, math.fsum), and theorems (Kraft/Gibbs entropy bound).
"""
import json
import math
import os
import zlib

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def u32(blob, off):
    return int(np.frombuffer(blob[off:off + 4].tobytes(), dtype="<u4")[0])


def u64(blob, off):
    return int(np.frombuffer(blob[off:off + 8].tobytes(), dtype="<u8")[0])


# ---- CRC-32 -------------------------------------------------------------------

def test_crc32_check_value():
    # the standard CRC-32 check value of the ASCII string "123456789"
    assert O.crc32(b"123456789") == 0xCBF43926
    rnd = np.random.default_rng(5).integers(0, 256, 1000).astype(np.uint8)
    assert O.crc32(rnd) == zlib.crc32(rnd.tobytes())


# ---- hand-worked encodings ------------------------------------------------------

def test_tiny_fields_golden():
    g = golden("tiny_six.json")
    W = np.array(g["bits"], dtype=np.uint16).reshape(g["rows"], g["cols"])
    blob = O.encode(W)
    assert blob.size == g["blob_bytes"]
    assert u32(blob, 0) == 0x3146424C and blob[4] == 1 and blob[6] == 10
    assert u64(blob, 8) == g["rows"] and u64(blob, 16) == g["cols"]
    assert u64(blob, 24) == g["n_esc"]
    for key, off in (("off_raw", 32), ("off_nib", 40), ("off_idx", 48), ("off_esc", 56), ("blob_bytes", 64)):
        assert u64(blob, off) == g[key], key
    assert list(blob[72:88]) == g["lut"]
    assert blob[88] == g["n_codes"]
    assert u32(blob, 92) == zlib.crc32(blob[:92].tobytes())
    assert not blob[96:256].any()
    n = g["rows"] * g["cols"]
    assert list(blob[g["off_raw"]:g["off_raw"] + n]) == g["raw"]
    assert not blob[g["off_raw"] + n:g["off_nib"]].any()
    assert list(blob[g["off_nib"]:g["off_nib"] + len(g["nib"])]) == g["nib"]
    idx = np.frombuffer(blob[g["off_idx"]:g["off_idx"] + 8].tobytes(), dtype="<u4")
    assert list(idx) == g["idx"]
    assert np.array_equal(O.decode(blob), W)


def _escape_ties_tensor(g):
    n = g["rows"] * g["cols"]
    exps = np.full(n, 110, dtype=np.uint32)
    sign = np.zeros(n, dtype=np.uint32)
    for j, e in enumerate(list(range(101, 110)) + list(range(111, 116))):
        exps[100 + 10 * j:100 + 10 * j + 10] = e
    exps[1020:1030] = 116
    exps[5] = 100
    exps[2047] = 200
    sign[2047] = 1
    mant = np.arange(n, dtype=np.uint32) % 128
    return ((sign << 15) | (exps << 7) | mant).astype(np.uint16).reshape(g["rows"], g["cols"])


def test_escape_ties_golden():
    g = golden("escape_ties.json")
    W = _escape_ties_tensor(g)
    blob = O.encode(W)
    assert blob.size == g["blob_bytes"]
    for key, off in (("off_raw", 32), ("off_nib", 40), ("off_idx", 48), ("off_esc", 56)):
        assert u64(blob, off) == g[key], key
    assert list(blob[72:88]) == g["lut"]
    assert blob[88] == g["n_codes"]
    assert u64(blob, 24) == g["n_esc"]
    oe = g["off_esc"]
    assert list(blob[oe:oe + g["n_esc"]]) == g["esc"]
    idx = np.frombuffer(blob[g["off_idx"]:g["off_idx"] + 12].tobytes(), dtype="<u4")
    assert list(idx) == g["idx"]
    for pos, val in g["nib_at"].items():
        assert blob[g["off_nib"] + int(pos)] == val, pos
    for pos, val in g["raw_at"].items():
        assert blob[g["off_raw"] + int(pos)] == val, pos
    assert np.array_equal(O.decode(blob), W)


# ---- structural verification (corruption must be detected, fail closed) ----------
# Expected flags are worked out from the goldens' hand-derived layouts:
# 1 header, 2 index, 4 code-15 count, 8 unused code, 16 escape is a coded
# exponent, 32 nonzero padding.

def _corrupt(blob, pos, value=None, xor=None):
    b = blob.copy()
    if value is not None:
        b[pos] = value
    else:
        b[pos] ^= xor
    return b


def test_verify_tiny_six_corruptions():
    g = golden("tiny_six.json")
    W = np.array(g["bits"], dtype=np.uint16).reshape(g["rows"], g["cols"])
    blob = O.encode(W)
    d = blob[:96].copy()
    on, orw, oi = g["off_nib"], g["off_raw"], g["off_idx"]
    assert O.verify(blob, d) == 0
    assert O.verify(_corrupt(blob, on, 0x23), d) == O.VERIFY_CODE       # weight 0: code 3 >= n_codes
    assert O.verify(_corrupt(blob, on, 0x2F), d) == O.VERIFY_COUNT      # weight 0: code 15, no escape indexed
    assert O.verify(_corrupt(blob, on + 2, xor=0x10), d) == O.VERIFY_PADDING  # padding weight 6 gets code 1
    assert O.verify(_corrupt(blob, orw + 6, 1), d) == O.VERIFY_PADDING  # n = 6 even: byte 6 must stay 0
    assert O.verify(_corrupt(blob, orw + 7, 0x80), d) == O.VERIFY_PADDING
    assert O.verify(_corrupt(blob, oi + 4, 1), d) == O.VERIFY_INDEX | O.VERIFY_COUNT  # idx[1] = 1 != n_esc
    assert O.verify(_corrupt(blob, oi + 8, 7), d) == O.VERIFY_PADDING   # gap after the index
    assert O.verify(_corrupt(blob, 100, 1), d) == O.VERIFY_HEADER
    assert O.verify(_corrupt(blob, 8, xor=1), d) == O.VERIFY_HEADER     # rows differ from the trusted descriptor
    flipped = _corrupt(blob, orw, xor=0x02)                             # a mantissa bit of a real weight:
    assert O.verify(flipped, d) == 0                                    # no structural trace ...
    assert O.crc32(flipped) != O.crc32(blob)                            # ... the blob hash catches it


def test_verify_escape_ties_corruptions():
    g = golden("escape_ties.json")
    blob = O.encode(_escape_ties_tensor(g))
    d = blob[:96].copy()
    oe, oi, on = g["off_esc"], g["off_idx"], g["off_nib"]
    assert O.verify(blob, d) == 0
    assert O.verify(_corrupt(blob, oe, 101), d) == O.VERIFY_ESCAPE      # 101 has code 0
    assert O.verify(_corrupt(blob, oe, 99), d) == 0                     # another uncoded exponent: hash only
    assert O.verify(_corrupt(blob, oe + g["n_esc"], 5), d) == O.VERIFY_PADDING
    assert O.verify(_corrupt(blob, oi + 4, 6), d) == O.VERIFY_COUNT     # idx = 0, 6, 12: tiles hold 5 and 7
    assert O.verify(_corrupt(blob, oi + 4, 13), d) == O.VERIFY_INDEX | O.VERIFY_COUNT  # idx decreases
    assert O.verify(_corrupt(blob, on, 0x9F), d) == O.VERIFY_COUNT      # weight 0 becomes a sixth escape in tile 0


@pytest.mark.parametrize("shape", [(0, 7), (1, 1), (3, 5), (5, 4097), (256, 256)])
def test_verify_accepts_encoder_output(shape):
    rows, cols = shape
    W = synth.all_patterns(rows, cols) if shape == (256, 256) else \
        synth.gaussian(np.random.default_rng([9, rows, cols]), rows, cols, 0.02, 0.01, 100.0)
    assert O.verify(O.encode(W)) == 0


# ---- the round trip is the identity (lossless means bit-exact) -----------------

def test_roundtrip_all_65536_patterns():
    W = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    blob = O.encode(W)
    out = O.decode(blob)
    assert out.dtype == np.uint16
    assert np.array_equal(out, W)  # NaN payloads, +-0, +-Inf, denormals included


def test_all_patterns_closed_forms():
    # Each exponent occurs with 2 signs x 128 mantissas = 256 times; all tie, so
    # the 15 smallest exponents 0..14 get codes and 241 * 256 = 61,696 escape.
    W = synth.all_patterns(256, 256)
    h = O.histogram(W)
    assert np.all(h == 256)
    p = O.plan(W)
    assert p.n_codes == 15
    assert list(p.lut[:15]) == list(range(15)) and p.lut[15] == 0
    assert p.n_esc == 61696
    # tiled 96 times over a 1536 x 4096 expert: 241 * 24,576 = 5,922,816 escapes
    assert O.plan(synth.all_patterns(1536, 4096)).n_esc == 5922816


@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 7), (3, 5), (1, 1023), (1, 1025), (7, 333), (2, 1024),
                                       (5, 4097)])
def test_roundtrip_ragged(rows, cols):
    rng = np.random.default_rng([99, rows, cols])
    W = synth.gaussian(rng, rows, cols, 0.02, 0.01, 100.0)
    assert np.array_equal(O.decode(O.encode(W)), W)
    # a tensor with more than 15 distinct exponents everywhere
    V = rng.integers(0, 65536, size=(rows, cols), dtype=np.uint32).astype(np.uint16)
    assert np.array_equal(O.decode(O.encode(V)), V)


def test_roundtrip_empty():
    W = np.zeros((0, 64), dtype=np.uint16)
    blob = O.encode(W)
    assert blob.size == 512 and u64(blob, 24) == 0
    assert O.decode(blob).shape == (0, 64)


@pytest.mark.parametrize("distinct", [1, 14, 15, 16, 17])
def test_distinct_exponent_counts(distinct):
    # exponent e_j = 100 + j occurs (j + 1) * 10 times: 15 or fewer distinct ->
    # no escapes; otherwise the (distinct - 15) least frequent escape.
    exps = np.concatenate([np.full((j + 1) * 10, 100 + j) for j in range(distinct)]).astype(np.uint32)
    rng = np.random.default_rng(distinct)
    rng.shuffle(exps)
    W = ((exps << 7) | (np.arange(exps.size) % 128)).astype(np.uint16)[None, :]
    p = O.plan(W)
    assert p.n_codes == min(15, distinct)
    expect_esc = sum((j + 1) * 10 for j in range(max(0, distinct - 15)))
    assert p.n_esc == expect_esc
    assert list(p.lut[:p.n_codes]) == list(range(100 + max(0, distinct - 15), 100 + distinct))
    assert np.array_equal(O.decode(O.encode(W)), W)


def test_all_equal_counts_tie_break():
    # 20 exponents, 7 each: all tie -> the 15 smallest get codes
    exps = np.repeat(np.arange(50, 70, dtype=np.uint32), 7)
    W = (exps << 7).astype(np.uint16)[None, :]
    p = O.plan(W)
    assert list(p.lut[:15]) == list(range(50, 65)) and p.n_esc == 35


def _check_top15(W, p):
    """S is a valid top-15 set for the histogram (numpy's own bincount)."""
    e = (W.reshape(-1).astype(np.uint32) >> 7) & 0xFF
    hist = np.bincount(e, minlength=256)
    present = np.flatnonzero(hist)
    S = [int(v) for v in p.lut[:p.n_codes]]
    assert p.n_codes == min(15, present.size)
    assert S == sorted(S) and len(set(S)) == len(S)
    assert all(hist[s] > 0 for s in S)
    if present.size > 15:
        worst = min(hist[s] for s in S)
        for v in present:
            if v in S:
                continue
            assert hist[v] <= worst
            if hist[v] == worst:  # a tied exponent left out is larger than every tied one kept
                assert all(v > s for s in S if hist[s] == worst)
    assert p.n_esc == int(sum(hist[v] for v in present if v not in S))


@pytest.mark.parametrize("cfg", ["single", "expert1", "expert3", "expert4", "laplace"])
def test_top15_property_and_escape_count(cfg):
    if cfg == "single":
        W, _ = synth.single_tensor()
    elif cfg == "laplace":
        W = synth.laplace(np.random.default_rng([4, 62]), 256, 1024, 0.02)
    else:
        e = int(cfg[-1])
        W = synth.gaussian(np.random.default_rng([4, e]), 256, 1024, 0.02, synth.EXPERT_OUTLIER_RATES[e], 100.0)
    p = O.plan(W)
    _check_top15(W, p)
    assert np.array_equal(O.decode(O.encode(W)), W)


# ---- size and the entropy bound -----------------------------------------------

def test_blob_bytes_and_reduction_gaussian():
    W, _ = synth.single_tensor()
    blob = O.encode(W)
    n = W.size
    p = O.plan(W)
    # every byte is charged: header, both planes, the index and the escapes
    payload = n + (n + 1) // 2 + 4 * ((n + 1023) // 1024 + 1) + p.n_esc + 256
    assert payload <= blob.size < payload + 4 * 256
    reduction = 1.0 - blob.size / (2.0 * n)
    assert reduction >= 0.24  # >= 24 % on Gaussian-shaped weights


@pytest.mark.parametrize("cfg", ["single", "patterns", "laplace", "wide"])
def test_entropy_lower_bound(cfg):
    # The code gives 12 bits to a weight whose exponent has a code and 20 bits
    # to an escaped one.  Kraft sum over all 65,536 values: at most
    # 15*256*2^-12 + 241*256*2^-20 < 1, so by Gibbs' inequality the mean code
    # length cannot fall below the order-0 entropy H0 of the 16-bit values.
    if cfg == "single":
        W, _ = synth.single_tensor()
    elif cfg == "patterns":
        W = synth.all_patterns(256, 256)
    elif cfg == "laplace":
        W = synth.laplace(np.random.default_rng(3), 512, 1024, 0.02)
    else:
        W = synth.gaussian(np.random.default_rng(4), 512, 1024, 0.02, 0.2, 100.0)
    kraft = 15 * 256 * 2.0 ** -12 + 241 * 256 * 2.0 ** -20
    assert kraft <= 1.0
    n = W.size
    blob = O.encode(W)
    h0 = O.entropy16(W)
    # numpy's own count gives the same entropy
    cnt = np.bincount(W.reshape(-1), minlength=65536)
    pr = cnt[cnt > 0] / n
    assert abs(h0 - float(-(pr * np.log2(pr)).sum())) < 1e-9
    assert 8.0 * blob.size >= n * h0
    p = O.plan(W)
    assert 12 * n + 8 * p.n_esc >= n * h0


def test_entropy_closed_forms():
    assert O.entropy16(np.full(1000, 0x3F80, dtype=np.uint16)) == 0.0
    assert abs(O.entropy16(np.array([1, 2] * 50, dtype=np.uint16)) - 1.0) < 1e-12
    assert abs(O.entropy16(synth.all_patterns(256, 256)) - 16.0) < 1e-12
    assert abs(O.entropy_exponent(synth.all_patterns(256, 256)) - 8.0) < 1e-12


def test_synthetic_exponent_entropy_is_realistic():
    # The meowlab page measured 2.59-2.64 bits of exponent entropy on real
    # Qwen3-8B tensors; the Gaussian stand-in should sit near that.
    W = synth.layer_tensor(1)  # k_proj, 1024 x 4096
    h = O.entropy_exponent(W)
    assert 2.4 < h < 2.8


# ---- corrupted headers are refused --------------------------------------------

def test_corrupt_header_refused():
    W, _ = synth.single_tensor()
    blob = O.encode(W[:4])
    for off in (0, 4, 8, 24, 40, 72, 88, 92):
        bad = blob.copy()
        bad[off] ^= 0x01
        with pytest.raises(ValueError):
            O.decode(bad)


def test_corrupt_index_refused():
    g = golden("escape_ties.json")
    blob = O.encode(_escape_ties_tensor(g))
    bad = blob.copy()
    bad[g["off_idx"] + 4] += 1  # idx[1] 5 -> 6: tile 0 holds 5 escapes, not 6
    with pytest.raises(ValueError):
        O.decode(bad)


# ---- y = W x in float64 ---------------------------------------------------------

def test_matvec_golden():
    g = golden("matvec_small.json")
    W = synth.bf16_bits(np.array(g["W"], dtype=np.float32))
    x = synth.bf16_bits(np.array(g["x"], dtype=np.float32))
    y, a = O.matvec(W, x)
    assert np.array_equal(y, np.array(g["y"]))
    assert np.array_equal(a, np.array(g["A"]))


def test_matvec_one_hot_extracts_column():
    W, _ = synth.single_tensor()
    W = W[:64]
    for k in (0, 5, 1023):
        x = np.zeros((1, 1024), dtype=np.uint16)
        x[0, k] = 0x3F80  # 1.0
        y, _ = O.matvec(W, x)
        assert np.array_equal(y[0], synth.bf16_to_f32(W[:, k]).astype(np.float64))


def test_matvec_vs_numpy_and_fsum():
    rng = np.random.default_rng(11)
    W = synth.gaussian(rng, 37, 300, 0.02, 0.01, 50.0)  # not square: a transposed read fails
    x = synth.activations(rng, 3, 300)
    y, a = O.matvec(W, x)
    Wf = synth.bf16_to_f32(W).astype(np.float64)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref = xf @ Wf.T
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(xf) @ np.abs(Wf).T))
    assert np.allclose(a, np.abs(xf) @ np.abs(Wf).T, rtol=1e-14, atol=0)
    for b in range(3):
        for r in (0, 17, 36):
            exact = math.fsum(Wf[r] * xf[b])  # products are exact in float64
            assert abs(y[b, r] - exact) <= 300 * 2.0 ** -52 * a[b, r]


def test_matvec_row_range_matches_full():
    rng = np.random.default_rng(12)
    W = synth.gaussian(rng, 50, 64, 0.02, 0.0, 1.0)
    x = synth.activations(rng, 2, 64)
    y, a = O.matvec(W, x)
    ys, as_ = O.matvec(W, x, rows=(10, 30))
    assert np.array_equal(ys, y[:, 10:30]) and np.array_equal(as_, a[:, 10:30])


def test_matvec_nonfinite_propagates():
    W = synth.all_patterns(16, 4096)
    x = synth.activations(np.random.default_rng(1), 1, 4096)
    y, _ = O.matvec(W, x)
    # rows 7 and 15 hold the patterns 0x7000-0x7FFF and 0xF000-0xFFFF, which
    # include NaNs; every other row is finite
    assert np.isnan(y[0, 7]) and np.isnan(y[0, 15])
    assert np.isfinite(np.delete(y[0], [7, 15])).all()


# ---- the gated MLP product (SwiGLU) ------------------------------------------

def test_silu_against_scipy_and_identities():
    from scipy.special import expit

    z = np.concatenate([np.linspace(-30, 30, 121), [0.0, 1e-8, -1e-8, 700.0, -700.0]])
    got = np.array([O.silu(v) for v in z])
    assert np.allclose(got, z * expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(0.0) == 0.0
    # sigma(z) + sigma(-z) = 1, so silu(z) - silu(-z) = z
    assert np.allclose([O.silu(v) - O.silu(-v) for v in z[:121]], z[:121], rtol=1e-13, atol=1e-13)


def test_swiglu_one_hot_and_components():
    rng = np.random.default_rng(91)
    G = synth.gaussian(rng, 9, 1024, 0.05, 0.0, 1.0)
    U = synth.gaussian(rng, 9, 1024, 0.05, 0.0, 1.0)
    k = 77
    x = np.zeros((1, 1024), dtype=np.uint16)
    x[0, k] = 0x3F80  # one-hot 1.0: g and u are column k exactly
    h, g, u, ag, au = O.swiglu(G, U, x)
    gk = synth.bf16_to_f32(G[:, k]).astype(np.float64)
    uk = synth.bf16_to_f32(U[:, k]).astype(np.float64)
    from scipy.special import expit

    assert np.array_equal(g[0], gk) and np.array_equal(u[0], uk)
    assert np.allclose(h[0], gk * expit(gk) * uk, rtol=1e-14, atol=0)
    assert np.array_equal(ag[0], np.abs(gk)) and np.array_equal(au[0], np.abs(uk))
    # the components agree with the plain product
    xr = synth.activations(rng, 2, 1024)
    h2, g2, u2, _, _ = O.swiglu(G, U, xr)
    assert np.array_equal(g2, O.matvec(G, xr)[0]) and np.array_equal(u2, O.matvec(U, xr)[0])
