"""A serialized artifact of coded tensors: one file, self-describing, hashed.

A production claim for lossless weight coding needs the shipped container to
hold every tensor, charged with all metadata, to be validated by hash, and to
decode back to the source bytes tensor by tensor ("Lossless LLM Weight
Compression vs 8-bit GGUF", sections "Is the GLM-5.2 result production-ready?"
and "Questions to ask a vendor or research team").  This module writes and
reads such a file; loading fails closed on any mismatch.

File layout (little-endian):
  [0, 24)    b"LBFA", u32 version (1), u64 manifest length, u32 CRC-32 of the
             manifest, u32 zero
  [24, ...)  manifest: UTF-8 JSON {"format": "lbf-artifact", "version": 1,
             "tensors": [{"name", "rows", "cols", "offset", "bytes", "n_esc",
             "crc32", "sha256"}, ...]}
  blobs      each blob (format v1, header included) at a 4096-aligned offset;
             the gaps are zero
"""
from __future__ import annotations

import hashlib
import json
import os
import struct
import zlib
from dataclasses import dataclass
from typing import Callable, Iterable, Mapping

import numpy as np

MAGIC = b"LBFA"
VERSION = 1
ALIGN = 4096
_PREFIX = struct.Struct("<4sIQII")


class ArtifactError(RuntimeError):
    """The file, a manifest entry or a tensor failed a check."""


@dataclass
class Entry:
    name: str
    rows: int
    cols: int
    offset: int
    bytes: int
    n_esc: int
    crc32: int
    sha256: str


def _host_bytes(blob) -> np.ndarray:
    """uint8 host copy of a blob (a device lbf.Blob or a host uint8 array)."""
    data = getattr(blob, "data", blob)
    if hasattr(data, "cpu"):
        data = data.cpu().numpy()
    return np.ascontiguousarray(data, dtype=np.uint8)


def _u64(b: np.ndarray, o: int) -> int:
    return int(np.frombuffer(b[o:o + 8].tobytes(), dtype="<u8")[0])


def save(path: str, tensors: Mapping[str, object] | Iterable[tuple[str, object]]) -> list[Entry]:
    """Write the named blobs (lbf.Blob on the GPU, or host uint8 arrays as the
    encoder writes them) to one artifact file."""
    items = list(tensors.items()) if isinstance(tensors, Mapping) else list(tensors)
    hosts = [(name, _host_bytes(b)) for name, b in items]
    entries = []
    for name, h in hosts:
        if h.size < 256 or h[:4].tobytes() != b"LBF1":
            raise ArtifactError("%s: not a coded blob" % name)
        entries.append(Entry(name, _u64(h, 8), _u64(h, 16), 0, int(h.size), _u64(h, 24),
                             zlib.crc32(h.tobytes()), hashlib.sha256(h.tobytes()).hexdigest()))
    if len({e.name for e in entries}) != len(entries):
        raise ArtifactError("tensor names must be unique")

    def manifest_bytes():
        return json.dumps({"format": "lbf-artifact", "version": VERSION,
                           "tensors": [e.__dict__ for e in entries]}, sort_keys=True).encode()

    # offsets depend on the manifest length, which depends on the offsets'
    # digits: iterate until the layout is stable
    prev = None
    while True:
        m = manifest_bytes()
        off = -(-(_PREFIX.size + len(m)) // ALIGN) * ALIGN
        for e in entries:
            e.offset = off
            off += -(-e.bytes // ALIGN) * ALIGN
        m2 = manifest_bytes()
        if m2 == prev:
            break
        prev = m2
    with open(path, "wb") as f:
        f.write(_PREFIX.pack(MAGIC, VERSION, len(m2), zlib.crc32(m2), 0))
        f.write(m2)
        for e, (_, h) in zip(entries, hosts):
            f.write(b"\0" * (e.offset - f.tell()))
            f.write(h.tobytes())
        end = -(-f.tell() // ALIGN) * ALIGN
        f.write(b"\0" * (end - f.tell()))
    return entries


def read_manifest(path: str) -> list[Entry]:
    with open(path, "rb") as f:
        pre = f.read(_PREFIX.size)
        if len(pre) != _PREFIX.size:
            raise ArtifactError("truncated file")
        magic, version, mlen, mcrc, zero = _PREFIX.unpack(pre)
        if magic != MAGIC or version != VERSION or zero != 0:
            raise ArtifactError("not an lbf artifact (v%d)" % VERSION)
        m = f.read(mlen)
    if len(m) != mlen or zlib.crc32(m) != mcrc:
        raise ArtifactError("manifest corrupt")
    doc = json.loads(m)
    if doc.get("format") != "lbf-artifact" or doc.get("version") != VERSION:
        raise ArtifactError("manifest of another format")
    size = os.path.getsize(path)
    out = []
    for t in doc["tensors"]:
        e = Entry(**t)
        if e.offset % ALIGN or e.offset + e.bytes > size:
            raise ArtifactError("%s: entry outside the file" % e.name)
        out.append(e)
    return out


def _read_checked(path: str, e: Entry) -> np.ndarray:
    b = np.fromfile(path, dtype=np.uint8, count=e.bytes, offset=e.offset)
    if b.size != e.bytes:
        raise ArtifactError("%s: truncated" % e.name)
    if hashlib.sha256(b.tobytes()).hexdigest() != e.sha256 or zlib.crc32(b.tobytes()) != e.crc32:
        raise ArtifactError("%s: hash mismatch" % e.name)
    if _u64(b, 8) != e.rows or _u64(b, 16) != e.cols or _u64(b, 24) != e.n_esc or _u64(b, 64) != e.bytes:
        raise ArtifactError("%s: header disagrees with the manifest" % e.name)
    return b


def load_host(path: str, names: Iterable[str] | None = None) -> dict[str, np.ndarray]:
    """Host copies of the blobs, each checked against its SHA-256 and CRC-32."""
    want = None if names is None else set(names)
    return {e.name: _read_checked(path, e) for e in read_manifest(path) if want is None or e.name in want}


def load(path: str, names: Iterable[str] | None = None, device: str = "cuda", stream=None) -> dict:
    """Device blobs (lbf.Blob), each checked on the host (SHA-256, CRC-32,
    header against manifest, descriptor) and again on the GPU after upload
    (lbf_verify, lbf_crc32).  Raises ArtifactError on the first failure."""
    import torch

    from . import lbf

    out = {}
    want = None if names is None else set(names)
    for e in read_manifest(path):
        if want is not None and e.name not in want:
            continue
        b = _read_checked(path, e)
        d = lbf.Desc.from_bytes(b[:96].tobytes())
        if lbf.desc_check(d) != lbf.LBF_OK:
            raise ArtifactError("%s: descriptor fails validation" % e.name)
        blob = lbf.Blob(d, torch.from_numpy(b).to(device))
        flags = lbf.verify(blob, stream=stream)
        if flags:
            raise ArtifactError("%s: device blob fails verification (checks %#x)" % (e.name, flags))
        if lbf.crc32(blob.data, stream=stream) != e.crc32:
            raise ArtifactError("%s: device copy differs from the file" % e.name)
        out[e.name] = blob
    return out


def size_report(path: str) -> dict:
    """Fully charged size: the whole file (manifest, headers, index, escapes,
    alignment) against the tensors' BF16 bytes."""
    entries = read_manifest(path)
    n = sum(e.rows * e.cols for e in entries)
    size = os.path.getsize(path)
    return {"tensors": len(entries), "weights": n, "bf16_bytes": 2 * n, "file_bytes": size,
            "blob_bytes": sum(e.bytes for e in entries), "escapes": sum(e.n_esc for e in entries),
            "bits_per_weight": 8.0 * size / n if n else 0.0,
            "reduction_vs_bf16": 1.0 - size / (2.0 * n) if n else 0.0}


def check_against(path: str, source: Callable[[str], np.ndarray], names: Iterable[str] | None = None) -> dict:
    """Decode every tensor of the artifact on the GPU, one at a time, and
    compare its bits with ``source(name)`` (uint16 BF16 patterns).  Returns
    {name: True/False}; raises ArtifactError if the file fails a check."""
    import torch

    from . import lbf

    result = {}
    want = None if names is None else list(names)
    for e in read_manifest(path):
        if want is not None and e.name not in want:
            continue
        blob = load(path, [e.name])[e.name]
        got = lbf.decode(blob).view(torch.int16).cpu().numpy().view(np.uint16)
        ref = np.ascontiguousarray(source(e.name), dtype=np.uint16).reshape(e.rows, e.cols)
        result[e.name] = bool(np.array_equal(got, ref))
        del blob
    return result
