"""The serialized artifact (decode_byte_split_amd.artifact): round trip of
oracle-coded blobs through the file, fully charged size, and refusal of a
corrupted or truncated file (host-side checks; no GPU needed)."""
import os

import numpy as np
import pytest

from oracle import oracle as O
from decode_byte_split_amd import artifact as A
from decode_byte_split_amd import synth


@pytest.fixture(scope="module")
def coded():
    rng = np.random.default_rng(31)
    Ws = {"q": synth.gaussian(rng, 64, 1024, 0.02, 0.001, 100.0),
          "k": synth.gaussian(rng, 16, 2048, 0.03, 0.0, 1.0),
          "patterns": synth.all_patterns(8, 1024),
          "ragged": synth.gaussian(rng, 3, 333, 0.02, 0.01, 50.0)}
    return Ws, {name: O.encode(W) for name, W in Ws.items()}


def test_roundtrip_and_size(tmp_path, coded):
    Ws, blobs = coded
    path = str(tmp_path / "m.lbfa")
    entries = A.save(path, blobs)
    assert [e.name for e in entries] == list(blobs)
    assert all(e.offset % A.ALIGN == 0 for e in entries)
    back = A.load_host(path)
    for name, b in blobs.items():
        assert np.array_equal(back[name], b)
        assert np.array_equal(O.decode(back[name]), Ws[name])
    rep = A.size_report(path)
    n = sum(W.size for W in Ws.values())
    assert rep["weights"] == n and rep["file_bytes"] == os.path.getsize(path)
    assert rep["blob_bytes"] == sum(b.size for b in blobs.values())
    assert rep["reduction_vs_bf16"] == pytest.approx(1 - rep["file_bytes"] / (2 * n))
    assert rep["file_bytes"] % A.ALIGN == 0


def test_corruptions_are_refused(tmp_path, coded):
    _, blobs = coded
    path = str(tmp_path / "m.lbfa")
    entries = A.save(path, blobs)
    raw = bytearray(open(path, "rb").read())
    e = entries[1]

    def write(data, name):
        p = str(tmp_path / name)
        open(p, "wb").write(bytes(data))
        return p

    bad = bytearray(raw)
    bad[e.offset + e.bytes // 2] ^= 0x40  # a byte inside a blob
    with pytest.raises(A.ArtifactError, match="hash"):
        A.load_host(write(bad, "b1"))
    bad = bytearray(raw)
    bad[30] ^= 1  # the manifest
    with pytest.raises(A.ArtifactError, match="manifest"):
        A.read_manifest(write(bad, "b2"))
    with pytest.raises(A.ArtifactError):
        A.load_host(write(raw[:e.offset + 100], "b3"))  # truncated
    bad = bytearray(raw)
    bad[0:4] = b"XXXX"
    with pytest.raises(A.ArtifactError, match="not an lbf artifact"):
        A.read_manifest(write(bad, "b4"))
    # a manifest entry whose shape disagrees with the blob header is refused,
    # even with a valid manifest CRC and blob hashes
    import json
    import zlib
    pre = A._PREFIX.unpack(bytes(raw[:A._PREFIX.size]))
    doc = json.loads(bytes(raw[A._PREFIX.size:A._PREFIX.size + pre[2]]))
    doc["tensors"][1]["rows"] += 1
    m = json.dumps(doc, sort_keys=True).encode()
    assert len(m) == pre[2]  # 16 -> 17 rows: same length, blobs stay where they are
    bad = bytearray(raw)
    bad[:A._PREFIX.size] = A._PREFIX.pack(A.MAGIC, A.VERSION, len(m), zlib.crc32(m), 0)
    bad[A._PREFIX.size:A._PREFIX.size + len(m)] = m
    with pytest.raises(A.ArtifactError, match="header disagrees"):
        A.load_host(write(bad, "b5"))


def test_save_refuses_non_blobs(tmp_path):
    with pytest.raises(A.ArtifactError):
        A.save(str(tmp_path / "x.lbfa"), {"a": np.zeros(300, dtype=np.uint8)})
