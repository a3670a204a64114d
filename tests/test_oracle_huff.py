"""Pins for the oracle's entropy-coded variant (K15H): Huffman code lengths,
canonical codes, the stream layout and the decoder, each checked against
something other than the oracle itself — hand-derived fixtures
(tests/golden/huff_*.json), a textbook Huffman example, the canonical-code
example of RFC 1951 section 3.2.2, brute-force optimality over every length
assignment on small alphabets, Shannon's bounds, exhaustive round trips and
the order-0 entropy theorem."""
import itertools
import json
import math
import os

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


def counts16(pairs):
    c = [0] * 16
    for s, n in pairs.items():
        c[s] = n
    return c


# ---- code lengths ---------------------------------------------------------------

def test_textbook_example():
    # the six-character example of Cormen et al., "Introduction to Algorithms",
    # section 16.3: frequencies a45 b13 c12 d16 e9 f5 give lengths 1,3,3,3,4,4
    # and an encoded length of 224 (thousand) bits
    freq = [45, 13, 12, 16, 9, 5]
    ln = O.huffman_lengths(freq + [0] * 10)
    assert list(ln[:6]) == [1, 3, 3, 3, 4, 4] and not ln[6:].any()
    assert sum(f * int(l) for f, l in zip(freq, ln)) == 224


def test_tie_goes_to_the_leaf():
    # counts 1,1,2,2: merging s0+s1 makes a node of weight 2; the leaves s2 and
    # s3 (weight 2) win the next ties, so every length is 2 (the node-first rule
    # would give 3,3,2,1)
    assert list(O.huffman_lengths(counts16({0: 1, 1: 1, 2: 2, 3: 2}))[:4]) == [2, 2, 2, 2]


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_equal_counts_give_equal_lengths(k):
    ln = O.huffman_lengths([7] * (1 << k) + [0] * (16 - (1 << k)))
    assert list(ln[:1 << k]) == [k] * (1 << k) and not ln[1 << k:].any()


def test_one_and_no_symbols():
    assert list(O.huffman_lengths(counts16({9: 1000}))) == [0] * 9 + [1] + [0] * 6
    assert not O.huffman_lengths([0] * 16).any()


def _optimal_cost(counts):
    """Minimum sum(count * length) over every length vector with Kraft sum <= 1
    (brute force; lengths 1..m-1 suffice for m symbols)."""
    m = len(counts)
    best = None
    for ls in itertools.product(range(1, m), repeat=m):
        if sum(2.0 ** -l for l in ls) <= 1.0:
            cost = sum(c * l for c, l in zip(counts, ls))
            best = cost if best is None else min(best, cost)
    return best


@pytest.mark.parametrize("seed", range(12))
def test_lengths_are_optimal_brute_force(seed):
    rng = np.random.default_rng([61, seed])
    m = int(rng.integers(2, 7))
    syms = sorted(rng.choice(16, m, replace=False).tolist())
    cnt = rng.integers(1, 30, m).tolist()
    ln = O.huffman_lengths(counts16(dict(zip(syms, cnt))))
    used = [int(ln[s]) for s in syms]
    assert all(l >= 1 for l in used) and sum(int(l) for l in ln) == sum(used)
    assert sum(2.0 ** -l for l in used) == 1.0  # a full binary tree
    assert sum(c * l for c, l in zip(cnt, used)) == _optimal_cost(cnt)


@pytest.mark.parametrize("seed", range(8))
def test_shannon_bounds(seed):
    # H <= average length < H + 1 for every distribution with >= 2 symbols
    rng = np.random.default_rng([62, seed])
    cnt = rng.integers(0, 10 ** int(rng.integers(1, 7)), 16)
    cnt[rng.integers(0, 16, 2)] += 1
    if (cnt > 0).sum() < 2:
        cnt[:2] += 1
    ln = O.huffman_lengths(cnt)
    p = cnt[cnt > 0] / cnt.sum()
    h = float(-(p * np.log2(p)).sum())
    avg = float((cnt * ln).sum() / cnt.sum())
    assert h - 1e-12 <= avg < h + 1 and int(ln.max()) <= 15


def test_maximum_depth_fifteen():
    # Fibonacci counts force the deepest tree: 16 symbols, lengths 1..15 and 15
    fib = [1, 1]
    while len(fib) < 16:
        fib.append(fib[-1] + fib[-2])
    ln = O.huffman_lengths(fib)
    assert sorted(int(l) for l in ln) == [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 15]


# ---- canonical codes -------------------------------------------------------------

def test_canonical_codes_rfc1951_example():
    # RFC 1951 section 3.2.2: lengths (3,3,3,3,3,2,4,4) for A..H give the codes
    # 010 011 100 101 110 00 1110 1111
    codes = O.canonical_codes([3, 3, 3, 3, 3, 2, 4, 4] + [0] * 8)
    assert list(codes[:8]) == [0b010, 0b011, 0b100, 0b101, 0b110, 0b00, 0b1110, 0b1111]


@pytest.mark.parametrize("seed", range(6))
def test_canonical_codes_are_prefix_free(seed):
    rng = np.random.default_rng([63, seed])
    ln = O.huffman_lengths(rng.integers(1, 1000, 16))
    codes = O.canonical_codes(ln)
    words = [format(int(c), "0%db" % int(l)) for c, l in zip(codes, ln)]
    for a, b in itertools.permutations(words, 2):
        assert not b.startswith(a)


# ---- the blob ----------------------------------------------------------------------

@pytest.mark.parametrize("name", ["huff_tiny_six.json", "huff_sixteen.json"])
def test_golden_blob(name):
    g = golden(name)
    w = np.array(g["bits"], dtype=np.uint16).reshape(g["rows"], g["cols"])
    b = O.hencode(w)
    assert b.size == g["blob_bytes"]
    assert u32(b, 0) == 0x4846424C and u64(b, 8) == g["rows"] and u64(b, 16) == g["cols"]
    assert u64(b, 24) == g["n_esc"] and u64(b, 80) == len(g["stream_words"])
    offs = [u64(b, o) for o in (32, 40, 48, 56, 64, 72)]
    assert offs == [g["off_raw"], g["off_bits"], g["off_woff"], g["off_idx"], g["off_esc"], g["blob_bytes"]]
    assert list(b[108:124]) == g["lengths"] and b[105] == g["max_len"]
    assert list(O.canonical_codes(g["lengths"])) == g["codes"]
    assert [u32(b, g["off_bits"] + 4 * i) for i in range(len(g["stream_words"]))] == g["stream_words"]
    assert [u32(b, g["off_woff"] + 4 * i) for i in range(len(g["woff"]))] == g["woff"]
    if g["n_esc"]:
        assert [u32(b, g["off_idx"] + 4 * i) for i in range(2)] == g["idx"]
        assert list(b[g["off_esc"]:g["off_esc"] + g["n_esc"]]) == g["escapes"]
    # raw plane identical to format v1's for the same tensor
    v1 = O.encode(w)
    assert (b[256:256 + 1024] == v1[256:256 + 1024]).all()
    assert (O.hdecode(b) == w).all()


def test_roundtrip_all_patterns():
    w = np.arange(65536, dtype=np.uint16).reshape(64, 1024)
    b = O.hencode(w)
    assert (O.hdecode(b) == w).all()
    h = O.hread_header(b)
    assert h.n_esc == 65536 - 15 * 256  # closed form: 15 coded exponents of 256 patterns each


@pytest.mark.parametrize("shape", [(0, 5), (1, 1), (3, 7), (1, 1023), (1, 1025), (5, 333), (2, 2048)])
def test_roundtrip_ragged(shape):
    rng = np.random.default_rng([64, shape[0], shape[1]])
    w = synth.gaussian(rng, shape[0], shape[1], 0.02, 0.001, 100.0)
    assert (O.hdecode(O.hencode(w)) == w).all()


def test_one_symbol_tensor():
    # every weight has exponent 127: one used symbol of length 1, so each tile
    # stream is 1024 zero bits (32 words); n = 3000 -> 3 tiles (32 + 32 + 30 words)
    w = np.full((3, 1000), 0x3F80, dtype=np.uint16)
    w[:, ::2] |= 0x8000
    b = O.hencode(w)
    h = O.hread_header(b)
    assert list(h.lengths) == [1] + [0] * 15 and h.stream_words == 32 + 32 + 30
    assert not b[u64(b, 40):u64(b, 40) + 4 * h.stream_words].any()
    assert (O.hdecode(b) == w).all()


def test_stream_size_matches_code_lengths():
    rng = np.random.default_rng(65)
    w = synth.gaussian(rng, 7, 1500, 0.02, 0.001, 100.0)
    pl = O.hplan(w)
    codes = O.encode(w)  # v1 blob: the K15 code of every weight
    n = w.size
    nib = codes[u64(codes, 40):]
    i = np.arange(n)
    c = (nib[(i // 8) * 4 + (i % 4)] >> ((i % 8) // 4 * 4)) & 15
    assert (np.bincount(c, minlength=16) == pl.code_count).all()
    per_tile = [int(pl.lengths[c[t * 1024:(t + 1) * 1024]].astype(np.int64).sum()) for t in range((n + 1023) // 1024)]
    assert pl.stream_words == sum((b + 31) // 32 for b in per_tile)


def test_size_is_above_order0_entropy():
    # each weight's K15H bits (8 raw + its code length + 8 per escape) form a
    # prefix code over the 65,536 BF16 values (Kraft sum <= 1), so the payload
    # is at least n * H0 (Shannon); the gap is what the Huffman rounding costs
    rng = np.random.default_rng(66)
    for W in (synth.gaussian(rng, 512, 4096, 1 / 64, 0.0003, 50.0), synth.laplace(rng, 256, 4096, 0.02),
              synth.all_patterns(64, 1024)):
        pl = O.hplan(W)
        h = O.hread_header(O.hencode(W))
        payload = 8 * W.size + int((pl.code_count * pl.lengths).sum()) + 8 * h.n_esc
        assert payload >= W.size * O.entropy16(W) - 1e-6 * W.size


def test_decoder_refuses_corruption():
    g = golden("huff_sixteen.json")
    w = np.array(g["bits"], dtype=np.uint16).reshape(1, 16)
    b = O.hencode(w)
    for byte in range(124):
        for bit in (0, 5):
            bad = b.copy()
            bad[byte] ^= 1 << bit
            with pytest.raises(ValueError):
                O.hdecode(bad)
    bad = b.copy()
    bad[g["off_bits"] + 7] ^= 0x80  # flip a code bit: symbol 15 of the last weight becomes 7, an escape goes unused
    with pytest.raises(ValueError):
        O.hdecode(bad)
