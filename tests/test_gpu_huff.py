"""GPU parity of the entropy-coded variant (K15H) with the oracle: the GPU
re-coding of a v1 blob is the oracle's K15H blob byte for byte, and the GPU
decoder rebuilds every bit of the source tensor, on the hand-derived goldens,
ragged and degenerate shapes, escape-heavy tensors, and a full-size gate_proj
of the 8B-shaped layer."""
import json
import os

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth
from gpu_util import dev, host, make_env, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def env():
    return make_env()


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    return np.array(g["bits"], dtype=np.uint16).reshape(g["rows"], g["cols"])


def cases():
    rng = np.random.default_rng(71)
    return {
        "golden_tiny_six": lambda: _golden("huff_tiny_six.json"),
        "golden_sixteen": lambda: _golden("huff_sixteen.json"),
        "single_1024x1024": lambda: synth.single_tensor()[0],
        "ragged_1x37": lambda: synth.gaussian(np.random.default_rng(72), 1, 37, 0.02, 0.0, 1.0),
        "ragged_5x4097": lambda: synth.gaussian(np.random.default_rng(73), 5, 4097, 0.02, 0.002, 100.0),
        "ragged_7x333": lambda: synth.gaussian(np.random.default_rng(74), 7, 333, 0.02, 0.01, 100.0),
        "patterns_256x512": lambda: synth.all_patterns(256, 512),
        "one_symbol_3x1000": lambda: np.full((3, 1000), 0x3F80, dtype=np.uint16) | (np.arange(3000).reshape(3, 1000) % 2 << 15).astype(np.uint16),
        "two_symbols_2x2048": lambda: np.where(np.random.default_rng(75).random((2, 2048)) < 0.9, 0x3F80, 0x4000).astype(np.uint16),
        "rate20pct_64x2048": lambda: synth.gaussian(np.random.default_rng(76), 64, 2048, 0.02, 0.2, 100.0),
        "laplace_33x1024": lambda: synth.laplace(np.random.default_rng(77), 33, 1024, 0.02),
        "layer_sigma_512x4096": lambda: synth.gaussian(np.random.default_rng(78), 512, 4096, 1 / 64, 0.0003, 50.0),
    }


CASES = cases()


def _gpu_hblob(torch, lbf, W):
    return lbf.hencode(lbf.encode(dev(torch, W)))


@pytest.mark.parametrize("name", sorted(CASES))
def test_hencode_matches_oracle_and_decodes_exactly(env, name):
    torch, lbf = env
    W = CASES[name]()
    ref = O.hencode(W)
    hb = _gpu_hblob(torch, lbf, W)
    got = hb.data.cpu().numpy()
    assert got.size == ref.size
    if not np.array_equal(got, ref):
        bad = np.nonzero(got != ref)[0]
        raise AssertionError("%s: %d bytes differ, first at %d" % (name, bad.size, bad[0]))
    assert np.array_equal(host(lbf.hdecode(hb)), W)
    # and the GPU decoder on the oracle's own blob
    assert np.array_equal(host(lbf.hdecode(lbf.from_host_hblob(ref))), W)


def test_empty_tensor(env):
    torch, lbf = env
    W = np.zeros((0, 16), dtype=np.uint16)
    ref = O.hencode(W)
    hb = lbf.hencode(lbf.from_host_blob(O.encode(W)))
    assert np.array_equal(hb.data.cpu().numpy(), ref)
    assert lbf.hdecode(hb).numel() == 0


def test_full_size_gate_proj(env):
    torch, lbf = env
    W = synth.layer_tensor(synth.GATE)
    say("K15H gate_proj %dx%d: GPU re-code and decode vs oracle" % W.shape)
    hb = _gpu_hblob(torch, lbf, W)
    ref = O.hencode(W)
    assert np.array_equal(hb.data.cpu().numpy(), ref)
    assert np.array_equal(host(lbf.hdecode(hb)), W)
    bits = 8.0 * hb.nbytes / W.size
    h0 = O.entropy16(W)
    say("K15H gate_proj: %.4f bits/weight (order-0 bound %.4f), %.3f %% smaller than BF16" %
        (bits, h0, 100 * (1 - bits / 16)))
    assert h0 <= bits < h0 + 1.0


def test_corrupt_stream_decodes_in_bounds(env):
    # a damaged stream or word index must decode to some values without
    # reading or writing outside the blob and the output (the decoder clamps
    # every tile's words to the stream and every escape range to the index)
    torch, lbf = env
    W = synth.gaussian(np.random.default_rng(79), 16, 4096, 0.02, 0.001, 100.0)
    ref = O.hencode(W)
    u64 = lambda o: int(np.frombuffer(ref[o:o + 8].tobytes(), dtype="<u8")[0])
    off_bits, off_woff, words = u64(40), u64(48), u64(80)
    rng = np.random.default_rng(80)
    bad = ref.copy()
    pos = off_bits + rng.integers(0, 4 * words, 200)
    bad[pos] ^= rng.integers(1, 256, 200).astype(np.uint8)
    woff = bad[off_woff:off_woff + 4 * 65].view(np.uint32)
    woff[5] = 0xFFFFFFFF  # a word offset past the stream
    woff[9] = woff[8] - 3 if woff[8] >= 3 else 0  # a tile with negative length
    guard = torch.full((W.size + 4096,), 0x5A5A, dtype=torch.int16, device="cuda")
    out = guard[:W.size].view(torch.bfloat16).view(W.shape)
    lbf.hdecode(lbf.from_host_hblob(bad), out=out)
    torch.cuda.synchronize()
    assert not np.array_equal(host(out), W)
    assert (guard[W.size:].cpu().numpy() == 0x5A5A).all()
