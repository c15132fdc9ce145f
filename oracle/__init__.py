"""CPU oracle for VQ3R / VQ4P residual vector quantization.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product package.

The arithmetic of the method lives in vq_oracle.c (plain sequential C, see its
header for the page citations). This module wraps it with ctypes and adds the
parts that are most plainly written with numpy:

  * rtn()          the round-to-nearest baselines of the Gate-3 table
                   ([VQ3R page] §3.1 table: rtn2-g64, rtn3-g64, rtn4-row)
  * mxfp4_qdq()    the MXFP4 source format of the K3 experts ([VQ3R page] §3.2);
                   the format itself is the OCP Microscaling v1.0 definition
  * rel_error()    the Gate-3 metric ||W - W_hat||_F / ||W||_F ([VQ3R page] §3.1)
  * gemv_ref()     y = W_hat x in fp64 for the fused dequant-GEMV
  * pack/unpack    the 3-byte index record of VQ3R (one byte per stage) and of
                   VQ4P (four 6-bit indices in one little-endian 24-bit word,
                   [VQ3R page] §5)

[VQ3R page] = the page titled "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验".

Every function here is pinned by tests/test_oracle_*.py against values fixed
independently of it (values the page prints, closed forms, brute force on tiny
inputs, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        L.vqo_f32_to_f16.argtypes = [ctypes.c_float]
        L.vqo_f32_to_f16.restype = ctypes.c_uint16
        L.vqo_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.vqo_f16_to_f32.restype = ctypes.c_float
        L.vqo_row_scales.argtypes = [P, i64, i64, P]
        L.vqo_dist8.argtypes = [P, P]
        L.vqo_dist8.restype = ctypes.c_float
        L.vqo_argmin.argtypes = [P, P, i32]
        L.vqo_encode.argtypes = [P, i64, i64, i32, i32, P, P, P]
        L.vqo_encode_vectors.argtypes = [P, i64, i32, i32, P, P]
        L.vqo_decode.argtypes = [P, P, P, i64, i64, i32, i32, i32, P]
        L.vqo_fixed_point_bits.argtypes = [ctypes.c_float, i64]
        L.vqo_fit.argtypes = [P, i32, i64, i64, i32, i32, i32, P, P, P, P, P]
        L.vqo_lloyd_on_vectors.argtypes = [P, i64, i32, i32, P, P, P, P]
        L.vqo_splitmix64.argtypes = [P]
        L.vqo_splitmix64.restype = ctypes.c_uint64
        L.vqo_forgy_init.argtypes = [i64, i32, i32, ctypes.c_uint64, P]
        L.vqo_ttp_quantize.argtypes = [P, i64, i64, P, P, P]
        L.vqo_ttp_dequantize.argtypes = [P, P, i64, i64, P]
        L.vqo_max_threads.argtypes = []
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


class OracleError(RuntimeError):
    pass


def _check(st):
    if st != 0:
        raise OracleError("oracle status %d" % st)


# ------------------------------------------------------------------ formats
FORMATS = {"vq3r": (3, 256), "vq4p": (4, 64)}


def f32_to_f16_bits(x: float) -> int:
    return int(lib().vqo_f32_to_f16(float(np.float32(x))))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().vqo_f16_to_f32(int(h)))


# ------------------------------------------------------------------ core
def max_threads() -> int:
    """Host threads the oracle's parallel loops run on (its OpenMP setting)."""
    return int(lib().vqo_max_threads())


def row_scales(w: np.ndarray) -> np.ndarray:
    w = _f32(w)
    rows, cols = w.shape
    s = np.zeros(rows, dtype=np.uint16)
    _check(lib().vqo_row_scales(_p(w), rows, cols, _p(s)))
    return s


def dist8(r, c) -> np.float32:
    r = _f32(r)
    c = _f32(c)
    return np.float32(lib().vqo_dist8(_p(r), _p(c)))


def argmin(r, codebook) -> int:
    r = _f32(r)
    cb = _f32(codebook)
    return int(lib().vqo_argmin(_p(r), _p(cb), cb.shape[0]))


def encode(w: np.ndarray, codebooks: np.ndarray):
    """Greedy residual encode. Returns (idx int32 [rows, cols/8, stages], scales fp16 bits)."""
    w = _f32(w)
    cb = _f32(codebooks)
    stages, K, _ = cb.shape
    rows, cols = w.shape
    idx = np.zeros((rows, cols // 8, stages), dtype=np.int32)
    s = np.zeros(rows, dtype=np.uint16)
    _check(lib().vqo_encode(_p(w), rows, cols, stages, K, _p(cb), _p(s), _p(idx)))
    return idx, s


def encode_vectors(v: np.ndarray, codebooks: np.ndarray) -> np.ndarray:
    """Greedy residual encode of already-normalized vectors [n, 8] -> int32 [n, stages]."""
    v = _f32(v).reshape(-1, 8)
    cb = _f32(codebooks)
    stages, K, _ = cb.shape
    idx = np.zeros((v.shape[0], stages), dtype=np.int32)
    _check(lib().vqo_encode_vectors(_p(v), v.shape[0], stages, K, _p(cb), _p(idx)))
    return idx


def decode(idx: np.ndarray, scales: np.ndarray, codebooks: np.ndarray, stages_used: int | None = None):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    cb = _f32(codebooks)
    stages, K, _ = cb.shape
    rows, V, _ = idx.shape
    out = np.zeros((rows, V * 8), dtype=np.float32)
    _check(lib().vqo_decode(_p(idx), _p(s), _p(cb), rows, V * 8, stages, K,
                            stages if stages_used is None else stages_used, _p(out)))
    return out


def fixed_point_bits(maxabs: float, n: int) -> int:
    return int(lib().vqo_fixed_point_bits(float(np.float32(maxabs)), int(n)))


def fit(mats, stages: int, K: int, iters: int, init: np.ndarray, want_assign=False, want_obj=False,
        want_energy=False):
    """Lloyd fit over the vectors of `mats` (list of equal-shape fp32 matrices).
    Returns codebooks fp32 [stages, K, 8] and a dict of the optional outputs."""
    mats = [_f32(m) for m in mats]
    rows, cols = mats[0].shape
    n = len(mats) * rows * cols // 8
    ptrs = (ctypes.c_void_p * len(mats))(*[m.ctypes.data for m in mats])
    init = np.ascontiguousarray(init, dtype=np.int64).reshape(stages, K)
    cb = np.zeros((stages, K, 8), dtype=np.float32)
    assign = np.zeros((stages, n), dtype=np.int32) if want_assign else None
    obj = np.zeros((stages, iters + 1), dtype=np.float64) if want_obj else None
    energy = np.zeros(stages + 1, dtype=np.float64) if want_energy else None
    _check(lib().vqo_fit(ptrs, len(mats), rows, cols, stages, K, iters, _p(init), _p(cb),
                         _p(assign) if assign is not None else None,
                         _p(obj) if obj is not None else None,
                         _p(energy) if energy is not None else None))
    return cb, {"assign": assign, "obj": obj, "energy": energy}


def splitmix64(state: int, count: int) -> list:
    """The first `count` outputs of SplitMix64 from `state` (vq_oracle.c)."""
    st = ctypes.c_uint64(state)
    return [int(lib().vqo_splitmix64(ctypes.byref(st))) for _ in range(count)]


def forgy_init_seeded(n: int, K: int, stages: int, seed: int) -> np.ndarray:
    """Seeded Forgy init, int64 [stages, K] (the reading of the configs'
    "seeded random vectors"; generator and selection rule in vq_oracle.c)."""
    out = np.zeros((stages, K), dtype=np.int64)
    _check(lib().vqo_forgy_init(int(n), int(K), int(stages), int(seed) & ((1 << 64) - 1), _p(out)))
    return out


def lloyd_on_vectors(R: np.ndarray, K: int, iters: int, init: np.ndarray):
    """One Lloyd stage on an explicit training set. Returns (C, assign, obj, residual)."""
    R = _f32(R).copy()
    n = R.shape[0]
    C = np.zeros((K, 8), dtype=np.float32)
    a = np.zeros(n, dtype=np.int32)
    obj = np.zeros(iters + 1, dtype=np.float64)
    init = np.ascontiguousarray(init, dtype=np.int64)
    _check(lib().vqo_lloyd_on_vectors(_p(R), n, K, iters, _p(init), _p(C), _p(a), _p(obj)))
    return C, a, obj, R


# ------------------------------------------------------------------ records
def pack_vq3r(idx: np.ndarray) -> np.ndarray:
    """int [..., 3] indices -> uint8 [..., 3] record: one byte per stage."""
    idx = np.asarray(idx)
    assert idx.shape[-1] == 3 and idx.min() >= 0 and idx.max() < 256
    return idx.astype(np.uint8)


def unpack_vq3r(rec: np.ndarray) -> np.ndarray:
    return np.asarray(rec, dtype=np.uint8).astype(np.int32)


def pack_vq4p(idx: np.ndarray) -> np.ndarray:
    """int [..., 4] 6-bit indices -> uint8 [..., 3]: little-endian 24-bit word
    i1 | i2 << 6 | i3 << 12 | i4 << 18 ([VQ3R page] §5: 6-bit packed indices,
    byte-for-byte the size of VQ3R)."""
    idx = np.asarray(idx).astype(np.uint32)
    assert idx.shape[-1] == 4 and int(idx.max(initial=0)) < 64
    word = idx[..., 0] | (idx[..., 1] << 6) | (idx[..., 2] << 12) | (idx[..., 3] << 18)
    out = np.stack([word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF], axis=-1)
    return out.astype(np.uint8)


def unpack_vq4p(rec: np.ndarray) -> np.ndarray:
    rec = np.asarray(rec, dtype=np.uint8).astype(np.uint32)
    word = rec[..., 0] | (rec[..., 1] << 8) | (rec[..., 2] << 16)
    return np.stack([(word >> (6 * t)) & 0x3F for t in range(4)], axis=-1).astype(np.int32)


def pack(fmt: str, idx):
    return pack_vq3r(idx) if fmt == "vq3r" else pack_vq4p(idx)


def unpack(fmt: str, rec):
    return unpack_vq3r(rec) if fmt == "vq3r" else unpack_vq4p(rec)


# ------------------------------------------------------------------ Tied Trit-Planes
TTP_GROUP = 256


def ttp_quantize(w: np.ndarray, want_rounds=False):
    """Tied Trit-Planes 9-level quantizer ([TTP page], the page "Новый метод
    квантования Tied Trit-Planes сжимает DeepSeek-V4 до 4.0625 бит на вес"):
    w fp32 [rows, cols] (cols % 256 == 0) -> (codes uint8 [rows, cols/2], two
    4-bit codes q+4 per byte, scales fp16 bits [rows, cols/256]). Readings in
    vq_oracle.c."""
    w = _f32(w)
    rows, cols = w.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // TTP_GROUP), dtype=np.uint16)
    rounds = np.zeros((rows, cols // TTP_GROUP), dtype=np.int32) if want_rounds else None
    _check(lib().vqo_ttp_quantize(_p(w), rows, cols, _p(codes), _p(scales),
                                  _p(rounds) if rounds is not None else None))
    return (codes, scales, rounds) if want_rounds else (codes, scales)


def ttp_levels(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [..., n/2] -> levels q int8 [..., n] in -4..4."""
    c = np.asarray(codes, dtype=np.uint8)
    q = np.stack([c & 0xF, c >> 4], axis=-1).reshape(c.shape[:-1] + (c.shape[-1] * 2,)).astype(np.int8)
    return q - 4


def ttp_dequantize(codes: np.ndarray, scales: np.ndarray):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    rows, half = codes.shape
    out = np.zeros((rows, half * 2), dtype=np.float32)
    _check(lib().vqo_ttp_dequantize(_p(codes), _p(scales), rows, half * 2, _p(out)))
    return out


# ------------------------------------------------------------------ metrics
def rel_error(w: np.ndarray, w_hat: np.ndarray) -> float:
    """Gate-3 metric ([VQ3R page] §3.1): ||W - W_hat||_F / ||W||_F, fp64 sums."""
    w = np.asarray(w, dtype=np.float64)
    d = w - np.asarray(w_hat, dtype=np.float64)
    return float(np.sqrt(np.sum(d * d) / np.sum(w * w)))


def error_sums(w: np.ndarray, w_hat: np.ndarray):
    """(sum (w - w_hat)^2, sum w^2) in fp64."""
    w = np.asarray(w, dtype=np.float64)
    d = w - np.asarray(w_hat, dtype=np.float64)
    return float(np.sum(d * d)), float(np.sum(w * w))


def gemv_ref(w_hat: np.ndarray, x: np.ndarray):
    """y = W_hat x in fp64, plus the condition scale sum_k |w_hat_k x_k| per output."""
    W = np.asarray(w_hat, dtype=np.float64)
    xv = np.asarray(x, dtype=np.float64)
    return W @ xv, np.abs(W) @ np.abs(xv)


# ------------------------------------------------------------------ RTN
def rtn(w: np.ndarray, bits: int, group: int | None):
    """Round-to-nearest baseline rtn{bits}-g{group} ([VQ3R page] §3.1 table).
    Reading: symmetric absmax per group of `group` contiguous weights along the
    row (group=None: the whole row), levels -(2^(b-1)-1) .. 2^(b-1)-1, one fp16
    scale per group and no zero point (the table's bits/weight column, 2.25 and
    3.25 at g64 and 4.01 per row, is b + 16/group).
    sc = fp16(amax / qmax) (fp32 division, then round to nearest even);
    q = clamp(rint(w / sc), -qmax, qmax) with ties to even; w_hat = sc * q;
    a zero scale gives w_hat = 0. Returns (w_hat fp32, bits_per_weight)."""
    w = _f32(w)
    rows, cols = w.shape
    G = cols if group is None else int(group)
    assert cols % G == 0
    qmax = np.float32(2 ** (bits - 1) - 1)
    g = w.reshape(rows, cols // G, G)
    amax = np.max(np.abs(g), axis=2, keepdims=True)
    sc = (amax / qmax).astype(np.float32).astype(np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(g / sc), -qmax, qmax)
    w_hat = np.where(sc == 0, np.float32(0), (sc * q).astype(np.float32))
    return w_hat.reshape(rows, cols).astype(np.float32), bits + 16.0 / G


# ------------------------------------------------------------------ MXFP4
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def e2m1_round(a: np.ndarray) -> np.ndarray:
    """Round |v| to the FP4 E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}, nearest with
    ties to the even encoding, saturating at 6 (OCP MX v1.0 conversion)."""
    a = np.asarray(a, dtype=np.float32)
    q = np.where(a < 2, np.rint(2 * a) / 2, np.where(a < 4, np.rint(a), 2 * np.rint(a / 2)))
    return np.minimum(q, 6).astype(np.float32)


def mxfp4_qdq(w: np.ndarray) -> np.ndarray:
    """Quantize to MXFP4 and decode back to fp32 (the K3 experts' native format,
    [VQ3R page] §3.2). Blocks of 32 contiguous elements along the row share one
    E8M0 scale X = 2^(floor(log2 amax) - 2) (2 = exponent of the largest E2M1
    value), clamped to [2^-127, 2^127]; elements are E2M1(w / X); a zero block
    decodes to zeros."""
    w = _f32(w)
    rows, cols = w.shape
    assert cols % 32 == 0
    if not np.all(np.isfinite(w)):
        raise OracleError("non-finite input")
    b = w.reshape(rows, cols // 32, 32)
    amax = np.max(np.abs(b), axis=2, keepdims=True)
    _, ex = np.frexp(amax)  # amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
    xe = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)
    X = np.ldexp(np.float32(1), xe).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(amax == 0, np.float32(0), (b / X).astype(np.float32))
    q = np.sign(v) * e2m1_round(np.abs(v))
    out = np.where(amax == 0, np.float32(0), (X * q).astype(np.float32))
    return out.reshape(rows, cols).astype(np.float32)
