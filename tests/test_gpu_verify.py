"""GPU integrity checks against the oracle: lbf_verify's failed-check mask
equals the oracle's on clean and corrupted blobs, and lbf_crc32 equals zlib's
CRC-32 (the oracle's CRC is pinned to zlib in the oracle tests)."""
import zlib

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import synth
from gpu_util import dev, make_env, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    return make_env()


def blobs():
    rng = np.random.default_rng(21)
    return {
        "single_1024x1024": O.encode(synth.single_tensor()[0]),
        "patterns_256x256": O.encode(synth.all_patterns(256, 256)),
        "ragged_5x4097": O.encode(synth.gaussian(rng, 5, 4097, 0.02, 0.002, 100.0)),
        "ragged_7x333": O.encode(synth.gaussian(rng, 7, 333, 0.02, 0.01, 100.0)),
        "rate20pct_64x2048": O.encode(synth.gaussian(rng, 64, 2048, 0.02, 0.2, 100.0)),
        "laplace_33x1024": O.encode(synth.laplace(rng, 33, 1024, 0.02)),
    }


BLOBS = blobs()


def regions(blob):
    """(name, start, end) byte ranges of each part of a blob."""
    u64 = lambda o: int(np.frombuffer(blob[o:o + 8].tobytes(), dtype="<u8")[0])
    off_raw, off_nib, off_idx, off_esc, size = u64(32), u64(40), u64(48), u64(56), u64(64)
    n_esc = u64(24)
    return [("header", 0, 256), ("raw", off_raw, off_nib), ("nib", off_nib, off_idx), ("idx", off_idx, off_esc),
            ("esc", off_esc, off_esc + n_esc), ("tail", off_esc + n_esc, size)]


@pytest.mark.parametrize("name", sorted(BLOBS))
def test_verify_matches_oracle_on_corruptions(env, name):
    torch, lbf = env
    blob = BLOBS[name]
    good = lbf.from_host_blob(blob)
    assert lbf.verify(good) == 0 == O.verify(blob)
    rng = np.random.default_rng([22, len(name)])
    seen = set()
    for region, a, b in regions(blob):
        if b <= a:
            continue
        for _ in range(12):
            c = blob.copy()
            pos = int(rng.integers(a, b))
            c[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
            want = O.verify(c, blob[:96])
            got = lbf.verify(lbf.Blob(good.desc, torch.from_numpy(c).cuda()))
            assert got == want, (region, pos, got, want)
            seen.add(want)
    say("%s: flag masks seen %s" % (name, sorted(seen)))


def test_verify_full_size_tensor(env):
    """gate_proj of the 8B-shaped layer (88 MB coded): clean, then one flipped
    code nibble far into the plane."""
    torch, lbf = env
    W = synth.layer_tensor(synth.GATE)
    blob = lbf.encode(dev(torch, W))
    assert lbf.verify(blob) == 0
    host = blob.data.cpu().numpy()
    assert lbf.crc32(blob.data) == zlib.crc32(host.tobytes())
    # a code far into the nibble plane becomes 15 (an escape nobody indexed)
    off_nib, off_idx = int(blob.desc.off_nib), int(blob.desc.off_idx)
    pos = off_nib + (off_idx - off_nib) * 2 // 3
    while host[pos] & 0x0F == 0x0F:
        pos += 1
    bad = host.copy()
    bad[pos] |= 0x0F
    got = lbf.verify(lbf.Blob(blob.desc, torch.from_numpy(bad).cuda()))
    assert got == O.verify(bad, host[:96]) == O.VERIFY_COUNT


@pytest.mark.parametrize("n", [0, 1, 3, 15, 16, 17, 1023, 1024, 1025, 4099, 65536 + 7, 1 << 20, (5 << 20) + 11])
def test_crc32_matches_zlib(env, n):
    torch, lbf = env
    data = np.random.default_rng([23, n]).integers(0, 256, n, dtype=np.uint8)
    buf = torch.from_numpy(np.concatenate([data, np.zeros(1, np.uint8)])).cuda()[:n] if n else \
        torch.empty(0, dtype=torch.uint8, device="cuda")
    assert lbf.crc32(buf) == zlib.crc32(data.tobytes())


def test_crc32_of_blob_equals_oracle(env):
    torch, lbf = env
    for name, blob in BLOBS.items():
        t = torch.from_numpy(blob).cuda()
        assert lbf.crc32(t) == O.crc32(blob), name


def test_artifact_layer_loads_verified_and_decodes_exactly(env, tmp_path):
    """The 8B-shaped layer, coded on the GPU, through an artifact file: loaded
    with host and GPU checks, every tensor decodes to its source bits; a
    corrupted copy of the file is refused."""
    torch, lbf = env
    from decode_byte_split_amd import artifact as A

    names = [m[0] for m in synth.LAYER]
    blobs = {name: lbf.encode(dev(torch, synth.layer_tensor(m))) for m, name in enumerate(names)}
    path = str(tmp_path / "layer.lbfa")
    A.save(path, blobs)
    rep = A.size_report(path)
    say("layer artifact: %d bytes, %.4f bits/weight, %.3f %% smaller than BF16"
        % (rep["file_bytes"], rep["bits_per_weight"], 100 * rep["reduction_vs_bf16"]))
    assert rep["reduction_vs_bf16"] > 0.24
    ok = A.check_against(path, lambda name: synth.layer_tensor(names.index(name)))
    assert all(ok.values()) and len(ok) == len(names)
    e = A.read_manifest(path)[0]
    raw = bytearray(open(path, "rb").read())
    raw[e.offset + 5000] ^= 0x01
    bad = str(tmp_path / "bad.lbfa")
    open(bad, "wb").write(bytes(raw))
    with pytest.raises(A.ArtifactError):
        A.load(bad, [e.name])
