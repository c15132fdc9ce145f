"""MI355X-native residual vector quantization (VQ3R / VQ4P) of MoE expert weights.

Thin ctypes binding over libvq.so (include/vq.h). Every step of the method
runs in the library's HIP kernels; this module only marshals arguments:
PyTorch tensors provide device memory and the current HIP stream.

[VQ3R page] = the page "3比特逼近4比特精度？WARP残差向量量化VQ3R的完整测量实验":
  §2 VQ3R recipe (3 x 256-entry codebooks, 8-dim vectors, FP16 row scale),
  §3 relative Frobenius error, §4 encoder / codebook fit, §5 VQ4P.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "VQError", "lib", "FORMATS", "ENGINES", "stages_entries",
    "encode", "decode", "fit_codebooks", "gemv_pack", "dequant_gemv", "dequant_gemv_packed", "error_sums",
    "rel_errors", "mxfp4_qdq", "encode_workspace", "fit_workspace", "gemv_workspace", "gemv_packed_workspace",
    "error_workspace", "read_status",
    "container_layout", "crc32", "write_container", "container_info", "read_container", "load_container",
    "verify_container", "convert_layer", "dequant_gemm", "gemm_workspace",
    "ttp_quantize", "ttp_dequantize", "ttp_error_sums", "stream_read",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvq.so")

FORMATS = {"vq3r": 0, "vq4p": 1}
ENGINES = {"auto": 0, "mfma_f16x": 1, "mfma_f32": 2, "valu_f32": 3, "exact": 4}
STATUS = {0: "ok", 1: "invalid argument", 2: "size out of range", 3: "workspace", 4: "HIP runtime error",
          5: "data error flagged on the device", 6: "container file I/O failed",
          7: "container file malformed or corrupt"}


def stages_entries(fmt: str):
    return (3, 256) if fmt == "vq3r" else (4, 64)


class VQError(RuntimeError):
    def __init__(self, status: int, where: str, flags: int = 0):
        self.status = status
        self.flags = flags
        msg = "%s: %s" % (where, STATUS.get(status, "status %d" % status))
        if flags:
            msg += " (device flags 0x%x)" % flags
        super().__init__(msg)


_lib = None


def lib():
    """Loads libvq.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libvq.so is not built (%s); run residual_vector_quantization_amd.build_lib" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I, L64, SZ, U32P = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    sig = {
        "vq_status_string": ([I], ctypes.c_char_p),
        "vq_version": ([], I),
        "vq_read_status": ([P, P, U32P], I),
        "vq_read_device_status": ([P, P], I),
        "vq_clear_status": ([P, P], I),
        "vq_encode_workspace_size": ([I, L64, L64], SZ),
        "vq_encode": ([I, I, P, I, L64, L64, P, P, P, P, SZ, P], I),
        "vq3r_encode": ([P, I, L64, L64, P, P, P, P, SZ, P], I),
        "vq4p_encode": ([P, I, L64, L64, P, P, P, P, SZ, P], I),
        "vq_fit_workspace_size": ([I, L64, L64, L64], SZ),
        "vq_fit_codebooks": ([I, P, I, L64, L64, L64, ctypes.c_int32, P, P, P, SZ, I, P], I),
        "vq_forgy_init": ([L64, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64, P], I),
        "vq_fit_codebooks_seeded": ([I, P, I, L64, L64, L64, ctypes.c_int32, ctypes.c_uint64, P, P, SZ, I, P], I),
        "vq_decode": ([I, P, P, P, L64, L64, ctypes.c_int32, P, P], I),
        "vq3r_decode": ([P, P, P, L64, L64, P, P], I),
        "vq4p_decode": ([P, P, P, L64, L64, P, P], I),
        "vq_gemv_packed_size": ([I, L64, L64], SZ),
        "vq_gemv_pack": ([I, P, L64, L64, L64, P, P], I),
        "vq_gemv_workspace_size": ([I, L64, L64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32], SZ),
        "vq_gemv_packed_workspace_size": ([I, L64, L64, ctypes.c_int32, ctypes.c_int32], SZ),
        "vq_dequant_gemv": ([I, P, L64, P, L64, P, L64, L64, ctypes.c_int32, P, ctypes.c_int32, P,
                             ctypes.c_int32, P, P, SZ, P], I),
        "vq_dequant_gemv_packed": ([I, P, L64, P, L64, P, L64, L64, ctypes.c_int32, P, ctypes.c_int32, P,
                                    ctypes.c_int32, P, P, SZ, P], I),
        "vq_dequant_gemv_packed_noalloc": ([I, P, L64, P, L64, P, L64, L64, ctypes.c_int32, P, ctypes.c_int32,
                                            P, ctypes.c_int32, P, P, P], I),
        "vq3r_dequant_gemv": ([P, L64, P, L64, P, L64, L64, ctypes.c_int32, P, ctypes.c_int32, P,
                               ctypes.c_int32, P, P, SZ, P], I),
        "vq4p_dequant_gemv": ([P, L64, P, L64, P, L64, L64, ctypes.c_int32, P, ctypes.c_int32, P,
                               ctypes.c_int32, P, P, SZ, P], I),
        "vq_dequant_gemm_workspace_size": ([I, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32], SZ),
        "vq_dequant_gemm": ([I, P, L64, P, L64, P, L64, L64, ctypes.c_int32, P, ctypes.c_int32, P,
                             ctypes.c_int32, P, P, SZ, P], I),
        "vq_ttp_quantize": ([P, I, L64, L64, P, P, P, SZ, P], I),
        "vq_ttp_dequantize": ([P, P, L64, L64, P, P], I),
        "vq_ttp_error_workspace_size": ([L64, L64, L64], SZ),
        "vq_ttp_error": ([P, I, P, P, L64, L64, L64, P, P, SZ, P], I),
        "vq_error_workspace_size": ([I, L64, L64, L64], SZ),
        "vq_error": ([I, P, I, P, P, P, L64, L64, L64, P, P, P, P, SZ, P], I),
        "vq_mxfp4_qdq": ([P, I, L64, L64, P, P, SZ, P], I),
        "vq_mxfp4_qdq_bf16": ([P, I, L64, L64, P, P, SZ, P], I),
        "vq_stream_read": ([P, SZ, P, P], I),
        "vqc_layout": ([I, L64, L64, L64, P, P, P], ctypes.c_uint64),
        "vqc_crc32": ([ctypes.c_uint32, P, SZ], ctypes.c_uint32),
        "vqc_create": ([ctypes.c_char_p, I, L64, L64, L64, P], I),
        "vqc_write_records": ([ctypes.c_char_p, L64, L64, P, P, P], I),
        "vqc_info": ([ctypes.c_char_p, P, P, P, P], I),
        "vqc_read_codebooks": ([ctypes.c_char_p, P], I),
        "vqc_read_records": ([ctypes.c_char_p, L64, L64, P, P, P], I),
        "vqc_load_records": ([ctypes.c_char_p, L64, L64, P, P, P, P, SZ, P], I),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
    if t.dtype not in m:
        raise TypeError("weights must be float32, bfloat16 or float16, got %s" % t.dtype)
    return m[t.dtype]


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


def _call(where, st, workspace=None, check=False):
    if st != 0:
        raise VQError(st, where)
    if check and workspace is not None:
        read_status(workspace, where)


def read_status(workspace, where="vq_read_status"):
    """Synchronizes the current stream and raises VQError if the last call that
    used `workspace` flagged a data error on the device."""
    flags = ctypes.c_uint32(0)
    st = lib().vq_read_status(_ptr(workspace), _stream(), ctypes.byref(flags))
    if st != 0:
        raise VQError(st, where, flags.value)
    return flags.value


def _workspace(nbytes, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ encode
def encode_workspace(fmt, rows, cols, device="cuda"):
    n = lib().vq_encode_workspace_size(FORMATS[fmt], rows, cols)
    if n == 0:
        raise VQError(1, "vq_encode_workspace_size")
    return _workspace(n, device)


def encode(W, codebooks, fmt="vq3r", engine="auto", idx=None, scales=None, workspace=None, check=True):
    """Greedy residual encode ([VQ3R page] §2, §4). W [rows, cols] (fp32/bf16/fp16),
    codebooks fp32 [stages, entries, 8]. Returns (idx uint8 [rows, cols/8, 3],
    scales fp16 [rows])."""
    torch = _torch()
    rows, cols = W.shape
    _check_cuda(W, codebooks)
    if idx is None:
        idx = torch.empty((rows, cols // 8, 3), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float16, device=W.device)
    if workspace is None:
        workspace = encode_workspace(fmt, rows, cols, W.device)
    st = lib().vq_encode(FORMATS[fmt], ENGINES[engine], _ptr(W), _dtype_code(W), rows, cols, _ptr(codebooks),
                         _ptr(idx), _ptr(scales), _ptr(workspace), workspace.numel(), _stream())
    _call("vq_encode", st, workspace, check and rows > 0)
    return idx, scales


# ------------------------------------------------------------------ decode
def decode(idx, scales, codebooks, fmt="vq3r", stages_used=None, out=None):
    """W_hat = s * (C1[i1] + C2[i2] + ...) ([VQ3R page] §2), fp32 [rows, cols]."""
    torch = _torch()
    rows, V, _ = idx.shape
    _check_cuda(idx, scales, codebooks)
    S, _ = stages_entries(fmt)
    if out is None:
        out = torch.empty((rows, V * 8), dtype=torch.float32, device=idx.device)
    st = lib().vq_decode(FORMATS[fmt], _ptr(idx), _ptr(scales), _ptr(codebooks), rows, V * 8,
                         S if stages_used is None else stages_used, _ptr(out), _stream())
    _call("vq_decode", st)
    return out


# ------------------------------------------------------------------ fit
def fit_workspace(fmt, n_mats, rows, cols, device="cuda"):
    n = lib().vq_fit_workspace_size(FORMATS[fmt], n_mats, rows, cols)
    if n == 0:
        raise VQError(1, "vq_fit_workspace_size")
    return _workspace(n, device)


def forgy_init(n_vectors, fmt="vq3r", seed=0):
    """The library's seeded Forgy init (vq_forgy_init): int64 [stages, entries]
    distinct training-vector indices. Host-only."""
    S, K = stages_entries(fmt)
    out = np.zeros((S, K), dtype=np.int64)
    _call("vq_forgy_init", lib().vq_forgy_init(int(n_vectors), K, S, int(seed) & ((1 << 64) - 1),
                                               out.ctypes.data_as(ctypes.c_void_p)))
    return out


def fit_codebooks(mats, init_idx=None, fmt="vq3r", iters=20, engine="auto", codebooks=None, workspace=None,
                  check=True, seed=None):
    """Lloyd codebook fit over the vectors of `mats` ([VQ3R page] §2, §4).
    init_idx: int64 [stages, entries] distinct training-vector indices; or
    init_idx=None and seed=s: the library draws them (vq_fit_codebooks_seeded)."""
    torch = _torch()
    rows, cols = mats[0].shape
    for m in mats:
        _check_cuda(m)
        if m.shape != (rows, cols) or m.dtype != mats[0].dtype:
            raise ValueError("all matrices must share shape and dtype")
    S, K = stages_entries(fmt)
    if (init_idx is None) == (seed is None):
        raise ValueError("give exactly one of init_idx and seed")
    if codebooks is None:
        codebooks = torch.empty((S, K, 8), dtype=torch.float32, device=mats[0].device)
    if workspace is None:
        workspace = fit_workspace(fmt, len(mats), rows, cols, mats[0].device)
    ptrs = (ctypes.c_void_p * len(mats))(*[m.data_ptr() for m in mats])
    if seed is not None:
        st = lib().vq_fit_codebooks_seeded(FORMATS[fmt], ptrs, _dtype_code(mats[0]), len(mats), rows, cols,
                                           int(iters), int(seed) & ((1 << 64) - 1), _ptr(codebooks), _ptr(workspace),
                                           workspace.numel(), ENGINES[engine], _stream())
        _call("vq_fit_codebooks_seeded", st, workspace, check)
        return codebooks
    init = np.ascontiguousarray(init_idx, dtype=np.int64).reshape(S, K)
    st = lib().vq_fit_codebooks(FORMATS[fmt], ptrs, _dtype_code(mats[0]), len(mats), rows, cols, int(iters),
                                init.ctypes.data_as(ctypes.c_void_p), _ptr(codebooks), _ptr(workspace),
                                workspace.numel(), ENGINES[engine], _stream())
    _call("vq_fit_codebooks", st, workspace, check)
    return codebooks


# ------------------------------------------------------------------ GEMV
def gemv_workspace(fmt, rows, cols, ntok, topk, n_experts, device="cuda"):
    """Workspace of the stored-record GEMV (dequant_gemv)."""
    n = lib().vq_gemv_workspace_size(FORMATS[fmt], rows, cols, ntok, topk, n_experts)
    if n == 0:
        raise VQError(1, "vq_gemv_workspace_size")
    return _workspace(n, device)


def gemv_packed_workspace(fmt, rows, cols, ntok, topk, device="cuda"):
    """Workspace of the packed-layout GEMV (dequant_gemv_packed)."""
    n = lib().vq_gemv_packed_workspace_size(FORMATS[fmt], rows, cols, ntok, topk)
    if n == 0:
        raise VQError(1, "vq_gemv_packed_workspace_size")
    return _workspace(n, device)


def gemv_pack(idx, fmt="vq3r", out=None):
    """Repacks stored records idx [E, rows, cols/8, 3] into the GEMV runtime
    layout (uint8 [E, packed_size])."""
    torch = _torch()
    E, rows, V, _ = idx.shape
    _check_cuda(idx)
    n = lib().vq_gemv_packed_size(FORMATS[fmt], rows, V * 8)
    if n == 0:
        raise VQError(1, "vq_gemv_packed_size")
    if out is None:
        out = torch.empty((E, n), dtype=torch.uint8, device=idx.device)
    st = lib().vq_gemv_pack(FORMATS[fmt], _ptr(idx), rows, V * 8, E, _ptr(out), _stream())
    _call("vq_gemv_pack", st)
    return out


def _gemv_io(x, route, rows, device, y):
    torch = _torch()
    if x.dtype != torch.float16 or route.dtype != torch.int32:
        raise TypeError("x must be float16 and route int32")
    ntok, topk = route.shape
    if y is None:
        y = torch.empty((ntok, topk, rows), dtype=torch.float32, device=device)
    return ntok, topk, y


def dequant_gemv(idx, scales, codebooks, x, route, fmt="vq3r", y=None, workspace=None, check=False):
    """y[b][k] = W_hat_{route[b][k]} x_b from the stored records idx uint8
    [E, rows, cols/8, 3] and scales fp16 [E, rows]; x fp16 [ntok, cols], route
    int32 [ntok, topk] -> y fp32 [ntok, topk, rows] ([VQ3R page] §1)."""
    E, rows, V, _ = idx.shape
    _check_cuda(idx, scales, codebooks, x, route)
    ntok, topk, y = _gemv_io(x, route, rows, idx.device, y)
    if workspace is None:
        workspace = gemv_workspace(fmt, rows, V * 8, ntok, topk, E, idx.device)
    st = lib().vq_dequant_gemv(FORMATS[fmt], _ptr(idx), rows * V * 3, _ptr(scales), scales.shape[-1],
                               _ptr(codebooks), rows, V * 8, E, _ptr(x), ntok, _ptr(route), topk, _ptr(y),
                               _ptr(workspace), workspace.numel(), _stream())
    _call("vq_dequant_gemv", st, workspace, check)
    return y


def dequant_gemv_packed(packed, scales, codebooks, x, route, rows, cols, fmt="vq3r", y=None, workspace=None,
                        check=False):
    """The same from experts packed by gemv_pack (uint8 [E, packed_size])."""
    E = packed.shape[0]
    _check_cuda(packed, scales, codebooks, x, route)
    ntok, topk, y = _gemv_io(x, route, rows, packed.device, y)
    if workspace is None:
        workspace = gemv_packed_workspace(fmt, rows, cols, ntok, topk, packed.device)
    st = lib().vq_dequant_gemv_packed(FORMATS[fmt], _ptr(packed), packed.shape[1], _ptr(scales), scales.shape[-1],
                                      _ptr(codebooks), rows, cols, E, _ptr(x), ntok, _ptr(route), topk, _ptr(y),
                                      _ptr(workspace), workspace.numel(), _stream())
    _call("vq_dequant_gemv_packed", st, workspace, check)
    return y


def dequant_gemv_packed_noalloc(packed, scales, codebooks, x, route, rows, cols, fmt="vq3r", y=None, status=None):
    """dequant_gemv_packed without a workspace (the library's static device
    scratch holds the partial sums; calls that overlap on one GPU race).
    status: optional 256-byte uint8 device tensor that receives the status word
    (read it with read_status)."""
    E = packed.shape[0]
    _check_cuda(packed, scales, codebooks, x, route)
    ntok, topk, y = _gemv_io(x, route, rows, packed.device, y)
    st = lib().vq_dequant_gemv_packed_noalloc(FORMATS[fmt], _ptr(packed), packed.shape[1], _ptr(scales),
                                              scales.shape[-1], _ptr(codebooks), rows, cols, E, _ptr(x), ntok,
                                              _ptr(route), topk, _ptr(y), _ptr(status) if status is not None else None,
                                              _stream())
    _call("vq_dequant_gemv_packed_noalloc", st)
    return y


# ------------------------------------------------------------------ prefill GEMM
def gemm_workspace(fmt, n_experts, ntok, topk, device="cuda"):
    n = lib().vq_dequant_gemm_workspace_size(FORMATS[fmt], n_experts, ntok, topk)
    if n == 0:
        raise VQError(1, "vq_dequant_gemm_workspace_size")
    return _workspace(n, device)


def dequant_gemm(idx, scales, codebooks, x, route, fmt="vq3r", y=None, workspace=None, check=False):
    """Batched dequant-GEMM for many tokens per expert ([VQ3R page] §1, §2):
    y[b][k] = W_hat_{route[b][k]} x_b from the stored records idx uint8
    [E, rows, cols/8, 3] and scales fp16 [E, rows]; x fp16 [ntok, cols], route
    int32 [ntok, topk] -> y fp32 [ntok, topk, rows]."""
    torch = _torch()
    E, rows, V, _ = idx.shape
    ntok, topk = route.shape
    _check_cuda(idx, scales, codebooks, x, route)
    if x.dtype != torch.float16 or route.dtype != torch.int32:
        raise TypeError("x must be float16 and route int32")
    if y is None:
        y = torch.empty((ntok, topk, rows), dtype=torch.float32, device=idx.device)
    if workspace is None:
        workspace = gemm_workspace(fmt, E, ntok, topk, idx.device)
    st = lib().vq_dequant_gemm(FORMATS[fmt], _ptr(idx), rows * V * 3, _ptr(scales), scales.shape[-1], _ptr(codebooks),
                               rows, V * 8, E, _ptr(x), ntok, _ptr(route), topk, _ptr(y), _ptr(workspace),
                               workspace.numel(), _stream())
    _call("vq_dequant_gemm", st, workspace, check)
    return y


# ------------------------------------------------------------------ Tied Trit-Planes
def ttp_quantize(W, codes=None, scales=None, workspace=None, check=True):
    """Tied Trit-Planes 9-level codec ([TTP page]: two ternary planes tied by a
    factor of 3, 4.0625 bits per weight). W [rows, cols] (cols % 256 == 0) ->
    (codes uint8 [rows, cols/2], scales fp16 [rows, cols/256])."""
    torch = _torch()
    rows, cols = W.shape
    _check_cuda(W)
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((rows, cols // 256), dtype=torch.float16, device=W.device)
    if workspace is None:
        workspace = _workspace(256, W.device)
    st = lib().vq_ttp_quantize(_ptr(W), _dtype_code(W), rows, cols, _ptr(codes), _ptr(scales), _ptr(workspace),
                               workspace.numel(), _stream())
    _call("vq_ttp_quantize", st, workspace, check and rows > 0)
    return codes, scales


def ttp_dequantize(codes, scales, out=None):
    torch = _torch()
    rows, half = codes.shape
    _check_cuda(codes, scales)
    if out is None:
        out = torch.empty((rows, half * 2), dtype=torch.float32, device=codes.device)
    _call("vq_ttp_dequantize", lib().vq_ttp_dequantize(_ptr(codes), _ptr(scales), rows, half * 2, _ptr(out),
                                                       _stream()))
    return out


def ttp_error_sums(W, codes, scales, n_mats=1, sums=None, workspace=None, check=True):
    """fp64 [n_mats, 2]: sum (w - w_hat)^2 and sum w^2 per matrix."""
    torch = _torch()
    total_rows, cols = W.shape
    rows = total_rows // n_mats
    _check_cuda(W, codes, scales)
    if sums is None:
        sums = torch.empty((n_mats, 2), dtype=torch.float64, device=W.device)
    if workspace is None:
        n = lib().vq_ttp_error_workspace_size(n_mats, rows, cols)
        if n == 0:
            raise VQError(1, "vq_ttp_error_workspace_size")
        workspace = _workspace(n, W.device)
    st = lib().vq_ttp_error(_ptr(W), _dtype_code(W), _ptr(codes), _ptr(scales), n_mats, rows, cols, _ptr(sums),
                            _ptr(workspace), workspace.numel(), _stream())
    _call("vq_ttp_error", st, workspace, check)
    return sums


# ------------------------------------------------------------------ error
def error_workspace(fmt, n_mats, rows, cols, device="cuda"):
    n = lib().vq_error_workspace_size(FORMATS[fmt], n_mats, rows, cols)
    if n == 0:
        raise VQError(1, "vq_error_workspace_size")
    return _workspace(n, device)


def error_sums(W, idx, scales, codebooks, fmt="vq3r", n_mats=1, sums=None, workspace=None, check=True, rel=None,
               rel_all=None):
    """fp64 [n_mats, stages+1]: sum (w - w_hat_t)^2 after t = 1..stages, then sum w^2
    ([VQ3R page] §3.1). W is [n_mats*rows, cols] (matrices stacked by rows).
    rel / rel_all (optional fp64 [n_mats, stages] / [stages] device tensors)
    receive the library's relative Frobenius errors per matrix / over all."""
    torch = _torch()
    total_rows, cols = W.shape
    rows = total_rows // n_mats
    S, _ = stages_entries(fmt)
    _check_cuda(W, idx, scales, codebooks)
    if sums is None:
        sums = torch.empty((n_mats, S + 1), dtype=torch.float64, device=W.device)
    if workspace is None:
        workspace = error_workspace(fmt, n_mats, rows, cols, W.device)
    st = lib().vq_error(FORMATS[fmt], _ptr(W), _dtype_code(W), _ptr(idx), _ptr(scales), _ptr(codebooks), n_mats,
                        rows, cols, _ptr(sums), _ptr(rel) if rel is not None else None,
                        _ptr(rel_all) if rel_all is not None else None, _ptr(workspace), workspace.numel(),
                        _stream())
    _call("vq_error", st, workspace, check)
    return sums


def rel_errors(W, idx, scales, codebooks, fmt="vq3r", n_mats=1, workspace=None, check=True):
    """Relative Frobenius errors computed by the library ([VQ3R page] §3.1):
    (per matrix fp64 [n_mats, stages], over all matrices fp64 [stages], the
    sums of error_sums)."""
    torch = _torch()
    S, _ = stages_entries(fmt)
    rel = torch.empty((n_mats, S), dtype=torch.float64, device=W.device)
    rel_all = torch.empty(S, dtype=torch.float64, device=W.device)
    sums = error_sums(W, idx, scales, codebooks, fmt=fmt, n_mats=n_mats, workspace=workspace, check=check, rel=rel,
                      rel_all=rel_all)
    return rel, rel_all, sums


# ------------------------------------------------------------------ MXFP4
def mxfp4_qdq(W, out=None, workspace=None, check=True):
    """MXFP4 quantize-dequantize ([VQ3R page] §3.2 source format) -> [rows, cols], fp32 by default or bf16
    when `out` is a bfloat16 tensor (exact: vq_mxfp4_qdq_bf16)."""
    torch = _torch()
    rows, cols = W.shape
    _check_cuda(W)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=W.device)
    _check_cuda(out)
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (rows, cols) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 or bf16 tensor of shape %s" % ((rows, cols),))
    if workspace is None:
        workspace = _workspace(256, W.device)
    name = "vq_mxfp4_qdq_bf16" if out.dtype == torch.bfloat16 else "vq_mxfp4_qdq"
    st = getattr(lib(), name)(_ptr(W), _dtype_code(W), rows, cols, _ptr(out), _ptr(workspace), workspace.numel(),
                              _stream())
    _call(name, st, workspace, check)
    return out


# ------------------------------------------------------------------ read reference
def stream_read(buf, out):
    """Plain streaming read of a device buffer (the GEMV's bandwidth reference);
    out: one-element int32 device tensor."""
    _check_cuda(buf)
    _call("vq_stream_read", lib().vq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), _stream()))


# ------------------------------------------------------------------ container
# Expert records on disk (include/vq_container.h; [VQ3R page] §1 experts
# streamed from disk, §4 codebooks stored with the container and record-by-
# record verification against the source weights, §5 VQ4P records).
def _host(a, dtype):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a).view(dtype) if np.asarray(a).dtype != dtype else np.asarray(a))


def _path(path):
    return os.fsencode(os.fspath(path))


def container_layout(fmt, rows, cols, n_records):
    """Byte layout of a container: total size, table and records offsets, record stride."""
    t, r, s = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    total = lib().vqc_layout(FORMATS[fmt], rows, cols, n_records, ctypes.byref(t), ctypes.byref(r), ctypes.byref(s))
    if total == 0:
        raise VQError(1, "vqc_layout")
    return {"bytes": int(total), "table_offset": t.value, "records_offset": r.value, "record_stride": s.value}


def crc32(data, crc=0):
    """CRC-32 (IEEE, as zlib) of a bytes-like object, computed by the library."""
    b = np.frombuffer(bytes(data), dtype=np.uint8)
    return int(lib().vqc_crc32(crc, b.ctypes.data_as(ctypes.c_void_p), b.size))


def write_container(path, fmt, codebooks, idx, scales, rel_err=None):
    """Writes a container of n records: codebooks fp32 [stages, entries, 8],
    idx uint8 [n, rows, cols/8, 3], scales fp16 [n, rows] (torch tensors on any
    device, or numpy), rel_err optional f64 [n, stages] (the measured relative
    error after each stage, stored for verify_container)."""
    cb = _host(codebooks, np.float32)
    ix = _host(idx, np.uint8)
    sc = _host(scales, np.uint16)
    n, rows, V = ix.shape[0], ix.shape[1], ix.shape[2]
    if ix.shape[3:] != (3,) or sc.shape != (n, rows) or cb.shape != stages_entries(fmt) + (8,):
        raise ValueError("write_container: shapes do not match")
    st = lib().vqc_create(_path(path), FORMATS[fmt], rows, V * 8, n, cb.ctypes.data_as(ctypes.c_void_p))
    _call("vqc_create", st)
    re = None
    if rel_err is not None:
        re = np.full((n, 4), np.nan)
        r = np.asarray(rel_err.detach().cpu() if hasattr(rel_err, "detach") else rel_err, dtype=np.float64)
        re[:, :r.shape[1]] = r
    st = lib().vqc_write_records(_path(path), 0, n, sc.ctypes.data_as(ctypes.c_void_p),
                                 ix.ctypes.data_as(ctypes.c_void_p),
                                 re.ctypes.data_as(ctypes.c_void_p) if re is not None else None)
    _call("vqc_write_records", st)


def container_info(path):
    """{'fmt', 'rows', 'cols', 'n_records'} from a validated header."""
    f, r, c, n = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    st = lib().vqc_info(_path(path), ctypes.byref(f), ctypes.byref(r), ctypes.byref(c), ctypes.byref(n))
    _call("vqc_info", st)
    fmt = {v: k for k, v in FORMATS.items()}[f.value]
    return {"fmt": fmt, "rows": r.value, "cols": c.value, "n_records": n.value}


def _range(info, first, count):
    if count is None:
        count = info["n_records"] - first
    return first, count


def read_container(path, first=0, count=None):
    """Host (numpy) read with CRC checks: (codebooks f32, idx u8 [count, rows, V, 3],
    scales fp16 bits u16 [count, rows], rel_err f64 [count, stages])."""
    info = container_info(path)
    first, count = _range(info, first, count)
    S, K = stages_entries(info["fmt"])
    rows, V = info["rows"], info["cols"] // 8
    cb = np.empty((S, K, 8), dtype=np.float32)
    _call("vqc_read_codebooks", lib().vqc_read_codebooks(_path(path), cb.ctypes.data_as(ctypes.c_void_p)))
    ix = np.empty((count, rows, V, 3), dtype=np.uint8)
    sc = np.empty((count, rows), dtype=np.uint16)
    re = np.empty((count, 4), dtype=np.float64)
    st = lib().vqc_read_records(_path(path), first, count, sc.ctypes.data_as(ctypes.c_void_p),
                                ix.ctypes.data_as(ctypes.c_void_p), re.ctypes.data_as(ctypes.c_void_p))
    _call("vqc_read_records", st)
    return cb, ix, sc, re[:, :S]


def load_container(path, first=0, count=None, device="cuda", staging_bytes=256 << 20):
    """Streams records into device memory (vqc_load_records) through a pinned
    staging buffer: (codebooks f32 [S, K, 8], idx u8 [count, rows, V, 3],
    scales fp16 [count, rows], rel_err f64 numpy [count, stages]), all tensors on `device`."""
    torch = _torch()
    info = container_info(path)
    first, count = _range(info, first, count)
    S, K = stages_entries(info["fmt"])
    rows, V = info["rows"], info["cols"] // 8
    stride = container_layout(info["fmt"], rows, info["cols"], info["n_records"])["record_stride"]
    nbytes = max(int(staging_bytes), 2 * stride)
    raw = torch.empty(nbytes + 4096, dtype=torch.uint8, pin_memory=True)
    off = (-raw.data_ptr()) % 4096
    cbh = np.empty((S, K, 8), dtype=np.float32)
    _call("vqc_read_codebooks", lib().vqc_read_codebooks(_path(path), cbh.ctypes.data_as(ctypes.c_void_p)))
    cb = torch.from_numpy(cbh).to(device)
    ix = torch.empty((count, rows, V, 3), dtype=torch.uint8, device=device)
    sc = torch.empty((count, rows), dtype=torch.float16, device=device)
    re = np.empty((count, 4), dtype=np.float64)
    st = lib().vqc_load_records(_path(path), first, count, _ptr(sc), _ptr(ix), re.ctypes.data_as(ctypes.c_void_p),
                                ctypes.c_void_p(raw.data_ptr() + off), nbytes, _stream())
    _call("vqc_load_records", st)
    return cb, ix, sc, re[:, :S]


def verify_container(path, sources, first=0):
    """Dequantizes each record of the container on the GPU and compares it with
    its source matrix (sources[r] is the [rows, cols] weight tensor of record
    first + r): returns {'stored': f64 [n, stages] errors stored at conversion,
    'measured': the same errors recomputed from the container's bytes,
    'match': stored == measured for every record that stored them}."""
    info = container_info(path)
    n = len(sources)
    cb, ix, sc, stored = load_container(path, first, n, device=sources[0].device)
    measured = np.empty_like(stored)
    for r in range(n):
        measured[r] = rel_errors(sources[r], ix[r], sc[r], cb, fmt=info["fmt"])[0][0].cpu().numpy()
    have = ~np.isnan(stored)
    match = bool(np.array_equal(stored[have], measured[have]))
    return {"stored": stored, "measured": measured, "match": match}


# ------------------------------------------------------------------ layer conversion
def convert_layer(weights, inits, sample, fmt="vq3r", iters=20, engine="auto", out_dir=None):
    """Converts the expert matrices of one MoE layer ([VQ3R page] §2 and §4:
    per layer and per matrix family, codebooks fit with k-means on sampled
    experts, then every expert encoded; §3.2 reports the w1 and w2 errors
    separately).

    weights: {name: tensor [E, rows, cols]} on the GPU, e.g. w1 and w3
             [E, 2048, 7168] and w2 [E, 7168, 2048] (fp32, bf16 or fp16);
    inits:   {name: int64 [stages, entries]} Forgy indices into the training
             vectors of the sampled experts of that matrix family;
    sample:  the expert ids whose matrices train the codebooks.
    Returns {name: {"codebooks", "idx" [E, rows, cols/8, 3], "scales" [E, rows],
    "rel_err" f64 [E, stages] (per expert, after each stage), "rel_err_all"
    f64 [stages] (over the whole family)}}. With out_dir, each family is also
    written to out_dir/<name>.vqc with its per-expert errors."""
    torch = _torch()
    out = {}
    for name, Wn in weights.items():
        E, rows, cols = Wn.shape
        mats = [Wn[e] for e in sample]
        cb = fit_codebooks(mats, inits[name], fmt=fmt, iters=iters, engine=engine)
        flat = Wn.reshape(E * rows, cols)
        idx, sc = encode(flat, cb, fmt=fmt, engine=engine)
        rel, rel_all, _ = rel_errors(flat, idx, sc, cb, fmt=fmt, n_mats=E)
        res = {"codebooks": cb, "idx": idx.view(E, rows, cols // 8, 3), "scales": sc.view(E, rows),
               "rel_err": rel, "rel_err_all": rel_all}
        if out_dir is not None:
            os.makedirs(out_dir, exist_ok=True)
            write_container(os.path.join(out_dir, name + ".vqc"), fmt, cb, res["idx"], res["scales"],
                            rel_err=res["rel_err"])
        out[name] = res
    torch.cuda.current_stream().synchronize()
    return out

