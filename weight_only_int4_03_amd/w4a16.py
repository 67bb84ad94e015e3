"""Thin ctypes binding over libw4a16.so (the C ABI in include/w4a16.h).

Argument marshalling only: every step runs in the library's HIP kernels (or,
for ``pack_host``, its C++ host code).  PyTorch supplies device memory and
the current stream.  The library must have been built
(``python -m weight_only_int4_03_amd.build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libw4a16.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "w4a16.h")

OK = 0
ERR_INVALID = -1
ERR_UNSUPPORTED = -2
ERR_NONFINITE = -3
ERR_HIP = -4
ERR_WORKSPACE = -5

PATH_AUTO = 0
PATH_DECODE = 1
PATH_PREFILL = 2
PATH_DENSE = 3
PATHS = {"auto": PATH_AUTO, "decode": PATH_DECODE, "prefill": PATH_PREFILL, "dense": PATH_DENSE}
FLAG_SWIGLU = 0x10
FLAG_BF16 = 0x20
FLAG_ZP = 0x40
FLAG_INT8 = 0x80
G = 128


class W4A16Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("w4a16 error %d: %s" % (code, message))
        self.code = code


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int

_SIGNATURES = {
    "w4a16_pack": ([_p, _i64, _i64, _int, _p, _p, _p], _int),
    "w4a16_pack_host": ([_p, _i64, _i64, _int, _p, _p, _int], _int),
    "w4a16_pack_gain": ([_p, _p, _i64, _i64, _int, _p, _p, _p], _int),
    "w4a16_gemm_rowscale": ([_p, _i64, _i64, _p, _p, _i64, _int, _p, _p, _int, _p, _i64, _p],
                            _int),
    "w4a16_rms_rowscale": ([_p, _i64, _i64, ctypes.c_float, _int, _p, _p], _int),
    "w4a16_repacked_weight_bytes": ([_i64, _i64, _int], _i64),
    "w4a16_repacked_scale_bytes": ([_i64, _i64, _int], _i64),
    "w4a16_repack": ([_p, _p, _i64, _i64, _int, _p, _p, _p], _int),
    "w4a16_unrepack": ([_p, _p, _i64, _i64, _int, _p, _p, _p], _int),
    "w4a16_dequant": ([_p, _p, _i64, _i64, _int, _p, _p], _int),
    "w4a16_dequant_bf16": ([_p, _p, _i64, _i64, _int, _p, _p], _int),
    "w4a16_zero_rows": ([_p, _p, _i64, _i64, _int, _p, _p], _int),
    "w4a16_pack_int8": ([_p, _i64, _i64, _int, _p, _p, _p], _int),
    "w4a16_repacked_weight_bytes_int8": ([_i64, _i64, _int], _i64),
    "w4a16_repack_int8": ([_p, _p, _i64, _i64, _int, _p, _p, _p], _int),
    "w4a16_unrepack_int8": ([_p, _p, _i64, _i64, _int, _p, _p, _p], _int),
    "w4a16_dequant_int8": ([_p, _p, _i64, _i64, _int, _int, _p, _p], _int),
    "w4a16_gemm_int8": ([_p, _i64, _i64, _p, _p, _i64, _int, _p, _p, _int, _p, _i64, _p], _int),
    "w4a16_dequant_zp": ([_p, _p, _p, _i64, _i64, _int, _int, _p, _p], _int),
    "w4a16_gemm_zp": ([_p, _i64, _i64, _p, _p, _p, _i64, _int, _p, _p, _int, _p, _i64, _p],
                      _int),
    "w4a16_gemm": ([_p, _i64, _i64, _p, _p, _i64, _int, _p, _p], _int),
    "w4a16_gemm_swiglu": ([_p, _i64, _i64, _p, _p, _i64, _int, _p, _p], _int),
    "w4a16_gemm_ex": ([_p, _i64, _i64, _p, _p, _i64, _int, _p, _int, _p, _i64, _p], _int),
    "w4a16_gemm_noalloc": ([_p, _i64, _i64, _p, _p, _i64, _int, _p, _int, _p], _int),
    "w4a16_noalloc_scratch_bytes": ([], _i64),
    "w4a16_gemm_workspace_bytes": ([_i64, _i64, _i64, _int, _int], _i64),
    "w4a16_select_path": ([_i64, _i64, _i64, _int, _int], _int),
    "w4a16_describe": ([_i64, _i64, _i64, _int, _int, _p, _i64], _int),
    "w4a16_probe_stream_read": ([_p, _i64, _p, _p], _int),
    "w4a16_probe_mfma": ([_i64, _i64, _p, _p, _p], _int),
    "w4a16_reserve_workspace": ([_i64], _int),
    "w4a16_workspace_reserved": ([], _i64),
    "w4a16_release_workspace": ([], _int),
    "w4a16_last_fallback": ([], ctypes.c_char_p),
    "w4a16_last_error": ([], ctypes.c_char_p),
    "w4a16_version": ([], ctypes.c_char_p),
}

_lib = None


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions include/w4a16.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError("libw4a16.so is not built: run python -m weight_only_int4_03_amd.build")
        # torch ships its own HIP runtime; loading it first makes the library
        # bind to that same runtime (a second runtime in the process would not
        # see torch's device memory, streams or device).
        _torch()
        L = ctypes.CDLL(LIBRARY)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def last_error() -> str:
    return lib().w4a16_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise W4A16Error(rc, last_error())
    return rc


def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


# -- host pack -----------------------------------------------------------------

def pack_host(W: np.ndarray, G: int = G, nthreads: int = 0):
    """Quantize + pack on the host: (packed int32 [K/8,N], scales uint16 [K/G,N])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    K, N = W.shape
    packed = np.empty((K // 8, N), np.int32)
    scales = np.empty((K // G, N), np.uint16)
    _check(lib().w4a16_pack_host(W.ctypes.data, K, N, G, packed.ctypes.data,
                                 scales.ctypes.data, nthreads))
    return packed, scales


# -- device calls ------------------------------------------------------------------

def pack(W, G: int = G, stream=None, gamma=None):
    """Quantize + pack a device fp32 [K,N] tensor: (packed int32 [K/8,N], scales int16 [K/G,N]).
    With gamma (device fp32 [K]), the folded-gain weights gamma[k] * W[k,n] are packed."""
    torch = _torch()
    assert W.is_cuda and W.dtype == torch.float32 and W.is_contiguous()
    K, N = W.shape
    packed = torch.empty((K // 8, N), dtype=torch.int32, device=W.device)
    scales = torch.empty((K // G, N), dtype=torch.int16, device=W.device)
    if gamma is None:
        _check(lib().w4a16_pack(_ptr(W), K, N, G, _ptr(packed), _ptr(scales), _stream(stream)))
    else:
        assert gamma.is_cuda and gamma.dtype == torch.float32 and gamma.numel() == K
        _check(lib().w4a16_pack_gain(_ptr(W), _ptr(gamma), K, N, G, _ptr(packed), _ptr(scales),
                                     _stream(stream)))
    return packed, scales


class RepackedWeight:
    """Repacked device buffers of one [K,N] weight (built by :func:`repack`;
    rz: prescaled zero rows of asymmetric weights, see :func:`zero_rows`)."""

    def __init__(self, rw, rs, K: int, N: int, G: int = G, rz=None, bits: int = 4):
        self.rw, self.rs, self.K, self.N, self.G, self.rz = rw, rs, K, N, G, rz
        self.bits = bits  # 4: INT4 codes; 8: INT8 codes (see repack_int8)

    def clone(self) -> "RepackedWeight":
        return RepackedWeight(self.rw.clone(), self.rs.clone(), self.K, self.N, self.G,
                              None if self.rz is None else self.rz.clone(), self.bits)

    @property
    def nbytes(self) -> int:
        return self.rw.numel() + self.rs.numel() + (0 if self.rz is None else self.rz.numel())


def repacked_bytes(K: int, N: int, G: int = G):
    return (_check(lib().w4a16_repacked_weight_bytes(K, N, G)),
            _check(lib().w4a16_repacked_scale_bytes(K, N, G)))


def repack(packed, scales, G: int = G, stream=None) -> RepackedWeight:
    """Canonical device (packed [K/8,N] int32, scales [K/G,N] fp16 bits) -> repacked."""
    torch = _torch()
    assert packed.is_cuda and packed.dtype == torch.int32 and packed.is_contiguous()
    assert scales.is_cuda and scales.element_size() == 2 and scales.is_contiguous()
    K, N = packed.shape[0] * 8, packed.shape[1]
    wb, sb = repacked_bytes(K, N, G)
    rw = torch.empty(wb, dtype=torch.uint8, device=packed.device)
    rs = torch.empty(sb, dtype=torch.uint8, device=packed.device)
    _check(lib().w4a16_repack(_ptr(packed), _ptr(scales), K, N, G, _ptr(rw), _ptr(rs),
                              _stream(stream)))
    return RepackedWeight(rw, rs, K, N, G)


def unrepack(w: RepackedWeight, G: int | None = None, stream=None):
    """Canonical device (packed, scales) of repacked weights (INT8 weights:
    packed [K/4,N])."""
    torch = _torch()
    G = w.G if G is None else G
    per = 4 if w.bits == 8 else 8
    packed = torch.empty((w.K // per, w.N), dtype=torch.int32, device=w.rw.device)
    scales = torch.empty((w.K // G, w.N), dtype=torch.int16, device=w.rw.device)
    fn = lib().w4a16_unrepack_int8 if w.bits == 8 else lib().w4a16_unrepack
    _check(fn(_ptr(w.rw), _ptr(w.rs), w.K, w.N, G, _ptr(packed), _ptr(scales), _stream(stream)))
    return packed, scales


def pack_int8(W, G: int = G, stream=None):
    """Quantize + pack a device fp32 [K,N] tensor to INT8 codes:
    (packed int32 [K/4,N], scales int16 [K/G,N])."""
    torch = _torch()
    assert W.is_cuda and W.dtype == torch.float32 and W.is_contiguous()
    K, N = W.shape
    packed = torch.empty((K // 4, N), dtype=torch.int32, device=W.device)
    scales = torch.empty((K // G, N), dtype=torch.int16, device=W.device)
    _check(lib().w4a16_pack_int8(_ptr(W), K, N, G, _ptr(packed), _ptr(scales), _stream(stream)))
    return packed, scales


def repack_int8(packed, scales, G: int = G, stream=None) -> RepackedWeight:
    """Canonical INT8 device (packed [K/4,N] int32, scales [K/G,N] fp16 bits) -> repacked."""
    torch = _torch()
    assert packed.is_cuda and packed.dtype == torch.int32 and packed.is_contiguous()
    assert scales.is_cuda and scales.element_size() == 2 and scales.is_contiguous()
    K, N = packed.shape[0] * 4, packed.shape[1]
    wb = _check(lib().w4a16_repacked_weight_bytes_int8(K, N, G))
    sb = _check(lib().w4a16_repacked_scale_bytes(K, N, G))
    rw = torch.empty(wb, dtype=torch.uint8, device=packed.device)
    rs = torch.empty(sb, dtype=torch.uint8, device=packed.device)
    _check(lib().w4a16_repack_int8(_ptr(packed), _ptr(scales), K, N, G, _ptr(rw), _ptr(rs),
                                   _stream(stream)))
    return RepackedWeight(rw, rs, K, N, G, bits=8)


def zero_rows(w: RepackedWeight, scales, zeros, stream=None) -> RepackedWeight:
    """Attach AWQ zero points to repacked weights: builds the prescaled zero
    rows fp16((8 - zp) s) from the canonical scales [K/G,N] (fp16 bits) and the
    zero points [K/G,N] (uint8), both device tensors.  Returns the weight with rz."""
    torch = _torch()
    assert scales.is_cuda and scales.element_size() == 2 and scales.is_contiguous()
    assert zeros.is_cuda and zeros.dtype == torch.uint8 and zeros.is_contiguous()
    assert tuple(zeros.shape) == tuple(scales.shape) == (w.K // w.G, w.N)
    rz = torch.empty(repacked_bytes(w.K, w.N, w.G)[1], dtype=torch.uint8, device=w.rw.device)
    _check(lib().w4a16_zero_rows(_ptr(scales), _ptr(zeros), w.K, w.N, w.G, _ptr(rz),
                                 _stream(stream)))
    return RepackedWeight(w.rw, w.rs, w.K, w.N, w.G, rz)


def dequant(w: RepackedWeight, G: int | None = None, stream=None, bf16: bool = False):
    """fp16 (or, with bf16, bf16) [K,N] dequantized weights (canonical row-major),
    with the zero rows when the weight has them."""
    torch = _torch()
    G = w.G if G is None else G
    W = torch.empty((w.K, w.N), dtype=torch.bfloat16 if bf16 else torch.float16,
                    device=w.rw.device)
    if w.bits == 8:
        _check(lib().w4a16_dequant_int8(_ptr(w.rw), _ptr(w.rs), w.K, w.N, G,
                                        FLAG_BF16 if bf16 else 0, _ptr(W), _stream(stream)))
        return W
    if w.rz is not None:
        _check(lib().w4a16_dequant_zp(_ptr(w.rw), _ptr(w.rs), _ptr(w.rz), w.K, w.N, G,
                                      FLAG_BF16 if bf16 else 0, _ptr(W), _stream(stream)))
        return W
    fn = lib().w4a16_dequant_bf16 if bf16 else lib().w4a16_dequant
    _check(fn(_ptr(w.rw), _ptr(w.rs), w.K, w.N, G, _ptr(W), _stream(stream)))
    return W


def _flags(path, swiglu: bool, bf16: bool, zp: bool = False, int8: bool = False) -> int:
    return ((PATHS[path] if isinstance(path, str) else int(path)) | (FLAG_SWIGLU if swiglu else 0)
            | (FLAG_BF16 if bf16 else 0) | (FLAG_ZP if zp else 0) | (FLAG_INT8 if int8 else 0))


def gemm(A, w: RepackedWeight, swiglu: bool = False, path: str | int = "auto", out=None,
         workspace=None, G: int | None = None, stream=None, rowscale=None):
    """C = A * dequant(W) ([M,N] in A's dtype, fp16 or bf16); with swiglu,
    Z = silu(C[:, :N/2]) * C[:, N/2:].  Weights with zero rows (w.rz) go
    through w4a16_gemm_zp."""
    torch = _torch()
    G = w.G if G is None else G
    assert A.is_cuda and A.dtype in (torch.float16, torch.bfloat16) and A.is_contiguous()
    bf16 = A.dtype == torch.bfloat16
    M, K = A.shape
    if K != w.K:
        raise ValueError("A has K=%d, weight has K=%d" % (K, w.K))
    ncols = w.N // 2 if swiglu else w.N
    if out is None:
        out = torch.empty((M, ncols), dtype=A.dtype, device=A.device)
    assert out.dtype == A.dtype
    flags = _flags(path, swiglu, bf16)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if rowscale is not None:
        assert rowscale.is_cuda and rowscale.dtype == torch.float32 and rowscale.numel() == M
    if w.bits == 8:
        _check(lib().w4a16_gemm_int8(_ptr(A), M, K, _ptr(w.rw), _ptr(w.rs), w.N, G,
                                     _ptr(rowscale), _ptr(out), flags, _ptr(workspace), ws_bytes,
                                     _stream(stream)))
    elif w.rz is not None:
        _check(lib().w4a16_gemm_zp(_ptr(A), M, K, _ptr(w.rw), _ptr(w.rs), _ptr(w.rz), w.N, G,
                                   _ptr(rowscale), _ptr(out), flags, _ptr(workspace), ws_bytes,
                                   _stream(stream)))
    elif rowscale is None:
        _check(lib().w4a16_gemm_ex(_ptr(A), M, K, _ptr(w.rw), _ptr(w.rs), w.N, G, _ptr(out),
                                   flags, _ptr(workspace), ws_bytes, _stream(stream)))
    else:
        _check(lib().w4a16_gemm_rowscale(_ptr(A), M, K, _ptr(w.rw), _ptr(w.rs), w.N, G,
                                         _ptr(rowscale), _ptr(out), flags, _ptr(workspace),
                                         ws_bytes, _stream(stream)))
    return out


def gemm_noalloc(A, w: RepackedWeight, swiglu: bool = False, path: str | int = "auto", out=None,
                 G: int | None = None, stream=None):
    """w4a16_gemm_noalloc: as :func:`gemm` (fp16 or bf16 INT4 weights without
    zero points or row factor) with the split-K partials in the library's
    fixed per-GPU scratch; makes no allocation."""
    torch = _torch()
    G = w.G if G is None else G
    assert A.is_cuda and A.dtype in (torch.float16, torch.bfloat16) and A.is_contiguous()
    assert w.bits == 4 and w.rz is None
    M, K = A.shape
    if out is None:
        out = torch.empty((M, w.N // 2 if swiglu else w.N), dtype=A.dtype, device=A.device)
    _check(lib().w4a16_gemm_noalloc(_ptr(A), M, K, _ptr(w.rw), _ptr(w.rs), w.N, G, _ptr(out),
                                    _flags(path, swiglu, A.dtype == torch.bfloat16),
                                    _stream(stream)))
    return out


def rms_rowscale(A, eps: float = 1e-5, stream=None):
    """RMSNorm row factors rho[m] = (mean_k A[m,k]^2 + eps)^(-1/2) of an fp16 or
    bf16 device tensor, as fp32 [M]."""
    torch = _torch()
    assert A.is_cuda and A.dtype in (torch.float16, torch.bfloat16) and A.is_contiguous()
    M, K = A.shape
    rho = torch.empty((M,), dtype=torch.float32, device=A.device)
    flags = FLAG_BF16 if A.dtype == torch.bfloat16 else 0
    _check(lib().w4a16_rms_rowscale(_ptr(A), M, K, eps, flags, _ptr(rho), _stream(stream)))
    return rho


def gemm_plain(A, w: RepackedWeight, out=None, G: int | None = None, stream=None):
    """w4a16_gemm (automatic path, library workspace)."""
    torch = _torch()
    M, K = A.shape
    if out is None:
        out = torch.empty((M, w.N), dtype=torch.float16, device=A.device)
    G = w.G if G is None else G
    _check(lib().w4a16_gemm(_ptr(A), M, K, _ptr(w.rw), _ptr(w.rs), w.N, G, _ptr(out),
                            _stream(stream)))
    return out


def gemm_swiglu(A, w: RepackedWeight, out=None, G: int | None = None, stream=None):
    """w4a16_gemm_swiglu (automatic path, library workspace)."""
    torch = _torch()
    M, K = A.shape
    if out is None:
        out = torch.empty((M, w.N // 2), dtype=torch.float16, device=A.device)
    G = w.G if G is None else G
    _check(lib().w4a16_gemm_swiglu(_ptr(A), M, K, _ptr(w.rw), _ptr(w.rs), w.N, G, _ptr(out),
                                   _stream(stream)))
    return out


def workspace_bytes(M: int, K: int, N: int, swiglu: bool = False, path: str | int = "auto",
                    G: int = G, bf16: bool = False, zp: bool = False, int8: bool = False) -> int:
    return _check(lib().w4a16_gemm_workspace_bytes(M, K, N, G,
                                                   _flags(path, swiglu, bf16, zp, int8)))


def select_path(M: int, K: int, N: int, swiglu: bool = False, G: int = G,
                int8: bool = False) -> str:
    code = _check(lib().w4a16_select_path(M, K, N, G, _flags(0, swiglu, False, False, int8)))
    return {v: k for k, v in PATHS.items()}[code]


def describe(M: int, K: int, N: int, swiglu: bool = False, path: str | int = "auto",
             G: int = G, bf16: bool = False, zp: bool = False, int8: bool = False) -> str:
    """The kernel launches (profiler names and grids) a GEMM of this shape makes."""
    buf = ctypes.create_string_buffer(1024)
    _check(lib().w4a16_describe(M, K, N, G, _flags(path, swiglu, bf16, zp, int8),
                                ctypes.addressof(buf), len(buf)))
    return buf.value.decode()


def reserve_workspace(nbytes: int) -> None:
    """Grow the current device's library workspace to at least nbytes (a
    load-time call: it may synchronise the device)."""
    _check(lib().w4a16_reserve_workspace(int(nbytes)))


def workspace_reserved() -> int:
    return _check(lib().w4a16_workspace_reserved())


def release_workspace() -> None:
    _check(lib().w4a16_release_workspace())


def last_fallback() -> str:
    return lib().w4a16_last_fallback().decode()


def probe_stream_read(buf, sink, stream=None) -> None:
    """Enqueue one streaming read of every byte of the device tensor `buf`
    (sink: a device tensor of at least 4 bytes)."""
    _check(lib().w4a16_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                         _stream(stream)))


def probe_mfma(iterations: int, workgroups: int, sink, stream=None) -> int:
    """Enqueue the dense fp16 MFMA loop; returns the FLOPs it performs."""
    flops = ctypes.c_int64(0)
    _check(lib().w4a16_probe_mfma(iterations, workgroups, _ptr(sink), ctypes.byref(flops),
                                  _stream(stream)))
    return flops.value


def load_weight(W_host: np.ndarray, device="cuda", G: int = G, gamma=None) -> RepackedWeight:
    """Host fp32 W -> device, quantize+pack on the GPU (gain gamma folded in
    when given, host fp32 [K]), repack.  (Load-time path.)"""
    torch = _torch()
    Wd = torch.from_numpy(np.ascontiguousarray(W_host, dtype=np.float32)).to(device)
    gd = None if gamma is None else torch.from_numpy(
        np.ascontiguousarray(gamma, dtype=np.float32)).to(device)
    packed, scales = pack(Wd, G, gamma=gd)
    del Wd
    return repack(packed, scales, G)


def load_weight_int8(W_host: np.ndarray, device="cuda", G: int = G) -> RepackedWeight:
    """Host fp32 W -> device, INT8 quantize+pack on the GPU, repack."""
    torch = _torch()
    Wd = torch.from_numpy(np.ascontiguousarray(W_host, dtype=np.float32)).to(device)
    packed, scales = pack_int8(Wd, G)
    del Wd
    return repack_int8(packed, scales, G)
