"""Independent reader and writer of the expert-record container.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the product package.

The container is the library's own byte layout for the conversion path of
[VQ3R page] §4 (codebooks stored with the container, expert records verified
one by one against the source weights) and §5 (VQ4P records); the page refers
to a format specification it does not reproduce. This module writes and parses
that layout from its written description (the comment at the top of the
library's container header) with `struct` and numpy, sharing no code with the
library, so that a test can check that both sides agree byte for byte. The
checksum is zlib's CRC-32.

[VQ3R page] = the page titled "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".

Parity unpinned against the page: the page fixes no byte layout. The layout
is pinned by the library/oracle agreement and by the round-trip tests.
"""
from __future__ import annotations

import struct
import zlib

import numpy as np

MAGIC = b"VQC1"
VERSION = 1
PAGE = 4096
ENTRY = 64


def _up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def layout(fmt: str, rows: int, cols: int, n: int) -> dict:
    stages, entries = (3, 256) if fmt == "vq3r" else (4, 64)
    d = {"format": 0 if fmt == "vq3r" else 1, "stages": stages, "entries": entries, "rows": rows, "cols": cols,
         "n": n}
    d["cb_off"] = PAGE
    d["cb_bytes"] = stages * entries * 8 * 4
    d["table_off"] = _up(d["cb_off"] + d["cb_bytes"], PAGE)
    d["table_bytes"] = n * ENTRY
    d["rec_off"] = _up(d["table_off"] + d["table_bytes"], PAGE)
    d["sc_bytes"] = rows * 2
    d["idx_off"] = _up(d["sc_bytes"], 256)
    d["idx_bytes"] = rows * (cols // 8) * 3
    d["stride"] = _up(d["idx_off"] + d["idx_bytes"], PAGE)
    d["total"] = d["rec_off"] + n * d["stride"]
    return d


def _header(L: dict, cb_crc: int) -> bytes:
    h = bytearray(PAGE)
    struct.pack_into("<4sIIIII", h, 0, MAGIC, VERSION, L["format"], L["stages"], L["entries"], 0)
    struct.pack_into("<11Q", h, 24, L["rows"], L["cols"], L["n"], L["cb_off"], L["cb_bytes"], L["table_off"],
                     L["table_bytes"], L["rec_off"], L["stride"], L["sc_bytes"], L["idx_off"])
    struct.pack_into("<Q", h, 112, L["idx_bytes"])
    struct.pack_into("<I", h, 120, cb_crc)
    struct.pack_into("<I", h, 124, zlib.crc32(bytes(h[:124])))
    return bytes(h)


def write(path, fmt: str, codebooks: np.ndarray, idx: np.ndarray, scales: np.ndarray, rel_err=None) -> None:
    """codebooks f32 [S, K, 8]; idx u8 [n, rows, cols/8, 3]; scales u16 [n, rows];
    rel_err f64 [n, S] or None (stored as NaN)."""
    n, rows, V, _ = idx.shape
    L = layout(fmt, rows, V * 8, n)
    cb = np.ascontiguousarray(codebooks, dtype=np.float32).tobytes()
    out = bytearray(L["total"])
    out[0:PAGE] = _header(L, zlib.crc32(cb))
    out[L["cb_off"]:L["cb_off"] + len(cb)] = cb
    for r in range(n):
        off = L["rec_off"] + r * L["stride"]
        sb = np.ascontiguousarray(scales[r], dtype=np.uint16).tobytes()
        ib = np.ascontiguousarray(idx[r], dtype=np.uint8).tobytes()
        out[off:off + len(sb)] = sb
        out[off + L["idx_off"]:off + L["idx_off"] + len(ib)] = ib
        errs = [float("nan")] * 4
        if rel_err is not None:
            for s in range(L["stages"]):
                errs[s] = float(rel_err[r][s])
        e = L["table_off"] + r * ENTRY
        struct.pack_into("<QII4d", out, e, off, zlib.crc32(ib, zlib.crc32(sb)), 1, *errs)
    with open(path, "wb") as f:
        f.write(bytes(out))


def read(path) -> dict:
    """Parses and checks every field; raises ValueError on any mismatch.
    Returns {'fmt', 'codebooks', 'idx', 'scales', 'rel_err', 'layout'}."""
    data = open(path, "rb").read()
    if len(data) < PAGE:
        raise ValueError("short file")
    h = data[:PAGE]
    magic, ver, fmtc, stages, entries, zero = struct.unpack_from("<4sIIIII", h, 0)
    if magic != MAGIC or ver != VERSION or fmtc not in (0, 1):
        raise ValueError("not a container")
    if struct.unpack_from("<I", h, 124)[0] != zlib.crc32(h[:124]):
        raise ValueError("header checksum")
    rows, cols, n = struct.unpack_from("<3Q", h, 24)
    fmt = "vq3r" if fmtc == 0 else "vq4p"
    L = layout(fmt, rows, cols, n)
    cb_crc = struct.unpack_from("<I", h, 120)[0]
    if h != _header(L, cb_crc):
        raise ValueError("header fields")
    if len(data) < L["total"]:
        raise ValueError("truncated")
    cbb = data[L["cb_off"]:L["cb_off"] + L["cb_bytes"]]
    if zlib.crc32(cbb) != cb_crc:
        raise ValueError("codebook checksum")
    S, K = L["stages"], L["entries"]
    idx = np.empty((n, rows, cols // 8, 3), dtype=np.uint8)
    scales = np.empty((n, rows), dtype=np.uint16)
    rel = np.empty((n, S), dtype=np.float64)
    for r in range(n):
        off, crc, flags, *errs = struct.unpack_from("<QII4d", data, L["table_off"] + r * ENTRY)
        if off != L["rec_off"] + r * L["stride"] or not (flags & 1):
            raise ValueError("record %d missing" % r)
        sb = data[off:off + L["sc_bytes"]]
        ib = data[off + L["idx_off"]:off + L["idx_off"] + L["idx_bytes"]]
        if zlib.crc32(ib, zlib.crc32(sb)) != crc:
            raise ValueError("record %d checksum" % r)
        scales[r] = np.frombuffer(sb, dtype=np.uint16)
        idx[r] = np.frombuffer(ib, dtype=np.uint8).reshape(rows, cols // 8, 3)
        rel[r] = errs[:S]
    return {"fmt": fmt, "codebooks": np.frombuffer(cbb, dtype=np.float32).reshape(S, K, 8).copy(), "idx": idx,
            "scales": scales, "rel_err": rel, "layout": L}
