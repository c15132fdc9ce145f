"""The expert-record container (include/vq_container.h) on the CPU: the
library's CRC-32 against the published check value and zlib, the library and
the independent oracle reader/writer agreeing byte for byte, and every
corruption the format is meant to catch. No call here touches a GPU."""
import os
import struct
import zlib

import numpy as np
import pytest

import residual_vector_quantization_amd as vq
from oracle import container as oc

EIO, EFORMAT, EINVAL = 6, 7, 1


def test_crc32_check_value_and_zlib():
    # the CRC-32 check value of the ASCII string "123456789" is 0xCBF43926
    # (the standard CRC catalogue entry for CRC-32/ISO-HDLC)
    assert vq.crc32(b"123456789") == 0xCBF43926
    assert zlib.crc32(b"123456789") == 0xCBF43926
    rng = np.random.default_rng(1)
    for n in [0, 1, 3, 7, 8, 9, 15, 16, 17, 255, 4096, 100003]:
        b = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert vq.crc32(b) == zlib.crc32(b), n
    a, b = b"hello ", b"world"
    assert vq.crc32(b, vq.crc32(a)) == zlib.crc32(a + b)  # continuation


def _records(fmt, n, rows, cols, seed):
    rng = np.random.default_rng(seed)
    S, K = vq.stages_entries(fmt)
    cb = rng.standard_normal((S, K, 8)).astype(np.float32)
    if fmt == "vq3r":
        idx = rng.integers(0, 256, (n, rows, cols // 8, 3), dtype=np.uint8)
    else:
        i4 = rng.integers(0, 64, (n * rows * (cols // 8), 4))
        import oracle
        idx = oracle.pack_vq4p(i4).reshape(n, rows, cols // 8, 3)
    sc = rng.integers(0, 0x7BFF, (n, rows), dtype=np.uint16)
    rel = rng.random((n, S))
    return cb, idx, sc, rel


@pytest.mark.parametrize("fmt,n,rows,cols", [("vq3r", 5, 40, 192), ("vq4p", 3, 33, 64), ("vq3r", 1, 2048, 512),
                                             ("vq3r", 0, 8, 8)])
def test_library_and_oracle_agree_byte_for_byte(tmp_path, fmt, n, rows, cols):
    cb, idx, sc, rel = _records(fmt, n, rows, cols, seed=rows)
    a, b = tmp_path / "lib.vqc", tmp_path / "oracle.vqc"
    vq.write_container(a, fmt, cb, idx, sc, rel_err=rel)
    oc.write(b, fmt, cb, idx, sc, rel_err=rel)
    assert a.read_bytes() == b.read_bytes()
    L = oc.layout(fmt, rows, cols, n)
    assert os.path.getsize(a) == L["total"] == vq.container_layout(fmt, rows, cols, n)["bytes"]
    for k in ("table_off", "rec_off", "stride", "cb_off"):
        assert L[k] % 4096 == 0
    # library reads what the oracle wrote, the oracle reads what the library wrote
    cb2, idx2, sc2, rel2 = vq.read_container(b)
    assert np.array_equal(cb2, cb) and np.array_equal(idx2, idx) and np.array_equal(sc2, sc)
    assert np.array_equal(rel2, rel)
    got = oc.read(a)
    assert got["fmt"] == fmt and np.array_equal(got["idx"], idx) and np.array_equal(got["scales"], sc)
    assert np.array_equal(got["codebooks"], cb) and np.array_equal(got["rel_err"], rel)
    assert vq.container_info(a) == {"fmt": fmt, "rows": rows, "cols": cols, "n_records": n}


def test_partial_reads_and_missing_errors(tmp_path):
    cb, idx, sc, _ = _records("vq3r", 6, 16, 64, seed=3)
    p = tmp_path / "c.vqc"
    vq.write_container(p, "vq3r", cb, idx, sc)
    _, i2, s2, r2 = vq.read_container(p, first=2, count=3)
    assert np.array_equal(i2, idx[2:5]) and np.array_equal(s2, sc[2:5])
    assert np.isnan(r2).all()  # no errors stored
    with pytest.raises(vq.VQError) as e:
        vq.read_container(p, first=4, count=3)
    assert e.value.status == EINVAL


def test_unwritten_record_is_rejected(tmp_path):
    cb, idx, sc, _ = _records("vq3r", 3, 8, 16, seed=4)
    p = str(tmp_path / "c.vqc")
    L = vq.lib()
    assert L.vqc_create(p.encode(), 0, 8, 16, 3, cb.ctypes.data) == 0
    assert L.vqc_write_records(p.encode(), 0, 2, sc.ctypes.data, idx.ctypes.data, None) == 0
    _, i2, _, _ = vq.read_container(p, 0, 2)
    assert np.array_equal(i2, idx[:2])
    with pytest.raises(vq.VQError) as e:
        vq.read_container(p, 2, 1)
    assert e.value.status == EFORMAT
    with pytest.raises(ValueError):
        oc.read(p)


def _flip(path, off):
    b = bytearray(open(path, "rb").read())
    b[off] ^= 0x10
    open(path, "wb").write(bytes(b))


@pytest.mark.parametrize("where", ["magic", "header_field", "codebook", "scale", "index", "table_crc"])
def test_corruption_is_detected(tmp_path, where):
    cb, idx, sc, _ = _records("vq3r", 2, 24, 128, seed=5)
    p = tmp_path / "c.vqc"
    vq.write_container(p, "vq3r", cb, idx, sc)
    L = oc.layout("vq3r", 24, 128, 2)
    rec1 = L["rec_off"] + L["stride"]
    off = {"magic": 0, "header_field": 25, "codebook": L["cb_off"] + 100, "scale": rec1 + 3,
           "index": rec1 + L["idx_off"] + 200, "table_crc": L["table_off"] + 64 + 8}[where]
    _flip(p, off)
    with pytest.raises(vq.VQError) as e:
        vq.read_container(p)
    assert e.value.status == EFORMAT
    with pytest.raises(ValueError):
        oc.read(p)
    if where in ("scale", "index", "table_crc"):
        # the intact record still reads
        _, i0, _, _ = vq.read_container(p, 0, 1)
        assert np.array_equal(i0, idx[:1])


def test_padding_bytes_are_not_covered_by_the_record_crc(tmp_path):
    # the CRC covers scale bytes then index bytes; zero padding between and
    # after them is outside it (a reader does not depend on it)
    cb, idx, sc, _ = _records("vq3r", 1, 24, 128, seed=6)
    p = tmp_path / "c.vqc"
    vq.write_container(p, "vq3r", cb, idx, sc)
    L = oc.layout("vq3r", 24, 128, 1)
    raw = open(p, "rb").read()
    off, crc = struct.unpack_from("<QI", raw, L["table_off"])
    sb = raw[off:off + 48]
    ib = raw[off + L["idx_off"]:off + L["idx_off"] + L["idx_bytes"]]
    assert crc == zlib.crc32(ib, zlib.crc32(sb))
    assert raw[off + 48:off + L["idx_off"]] == bytes(L["idx_off"] - 48)
    assert raw[off + L["idx_off"] + L["idx_bytes"]:off + L["stride"]] == bytes(
        L["stride"] - L["idx_off"] - L["idx_bytes"])


def test_truncated_missing_and_foreign_files(tmp_path):
    cb, idx, sc, _ = _records("vq4p", 2, 16, 64, seed=7)
    p = tmp_path / "c.vqc"
    vq.write_container(p, "vq4p", cb, idx, sc)
    raw = p.read_bytes()
    p.write_bytes(raw[:-1])
    with pytest.raises(vq.VQError) as e:
        vq.container_info(p)
    assert e.value.status == EFORMAT
    with pytest.raises(vq.VQError) as e:
        vq.container_info(tmp_path / "missing.vqc")
    assert e.value.status == EIO
    (tmp_path / "small").write_bytes(b"VQC1")
    with pytest.raises(vq.VQError) as e:
        vq.container_info(tmp_path / "small")
    assert e.value.status == EFORMAT
    (tmp_path / "foreign").write_bytes(bytes(8192))
    with pytest.raises(vq.VQError) as e:
        vq.container_info(tmp_path / "foreign")
    assert e.value.status == EFORMAT


def test_layout_rejects_invalid_sizes():
    L = vq.lib()
    assert L.vqc_layout(0, 4, 12, 1, None, None, None) == 0       # cols % 8
    assert L.vqc_layout(2, 4, 16, 1, None, None, None) == 0       # format
    assert L.vqc_layout(0, 0, 16, 1, None, None, None) == 0       # rows
    assert L.vqc_layout(0, 4, 16, -1, None, None, None) == 0      # count
    assert L.vqc_layout(0, 1 << 30, 64, 1, None, None, None) == 0  # rows * cols / 8 >= 2^32
    assert L.vqc_layout(0, 2048, 7168, 256, None, None, None) == oc.layout("vq3r", 2048, 7168, 256)["total"]


def test_load_records_argument_errors(tmp_path):
    # host-side checks that return before any HIP call
    cb, idx, sc, _ = _records("vq3r", 2, 16, 64, seed=8)
    p = str(tmp_path / "c.vqc")
    vq.write_container(p, "vq3r", cb, idx, sc)
    L = vq.lib()
    stride = vq.container_layout("vq3r", 16, 64, 2)["record_stride"]
    buf = np.zeros(4 * stride + 4096, dtype=np.uint8)
    al = buf.ctypes.data + (-buf.ctypes.data) % 4096
    fake = np.zeros(4096, dtype=np.uint8)
    d = fake.ctypes.data
    assert L.vqc_load_records(p.encode(), 0, 2, d, d, None, al, stride, None) == 3        # staging < 2 strides
    assert L.vqc_load_records(p.encode(), 0, 2, d, d, None, al + 8, 2 * stride, None) == 3  # misaligned
    assert L.vqc_load_records(p.encode(), 0, 2, None, d, None, al, 2 * stride, None) == EINVAL
    assert L.vqc_load_records(p.encode(), 1, 2, d, d, None, al, 2 * stride, None) == EINVAL
    assert L.vqc_load_records(p.encode(), 0, 0, None, None, None, None, 0, None) == 0     # empty
