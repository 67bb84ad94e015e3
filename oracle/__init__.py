"""W4A16 oracle: ctypes wrapper around the plain C reference in w4a16_oracle.c.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``weight_only_int4_03_amd``) and imports nothing from it.

Every function follows the page "GPU Kernels for INT4 Inference, in depth"
(aicassindra.com), sections "The job, stated precisely" and "The data
contract", except ``swiglu_f64``, which follows the SwiGLU line of the block
equations in FuTransformer (arXiv 2610.23796), section 2.1, the RMSNorm
folding helpers (FuTransformer, section 3.2.2), and the zero-point functions
(``zero_rows``, ``dequant_zp``), which follow the Swordfish page
(blog.alpindale.net), section "The packed format", and the INT8 functions
(``quantize8`` ... ``gemm8_f64``), which follow the same section and "Making a
Single GPU Go Fast" (arunshar.com), section 9.3.2.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "w4a16_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_w4a16.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]

OK = 0
ERR_SHAPE = -1
ERR_NONFINITE = -3


def build(source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle with gcc (no fast-math; IEEE fp32 division)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_p = ctypes.c_void_p
_i64 = ctypes.c_int64


class Oracle:
    """Bindings to one build of the oracle library (a path to a .so)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_dequant_bf16.argtypes = [_p, _p, _i64, _i64, ctypes.c_int, _p]
        lib.oracle_fold_gain.argtypes = [_p, _p, _i64, _i64, _p]
        lib.oracle_rms_rowscale_f64.argtypes = [_p, _i64, _i64, ctypes.c_int, ctypes.c_double, _p]
        lib.oracle_scale_rows.argtypes = [_p, _i64, _i64, _p, _p]
        lib.oracle_zero_rows.argtypes = [_p, _p, _i64, _i64, _p]
        lib.oracle_dequant_zp.argtypes = [_p, _p, _p, _i64, _i64, ctypes.c_int, ctypes.c_int, _p]
        lib.oracle_gemm_wb_f64.argtypes = [_p, _i64, _i64, _p, _i64, _p, ctypes.c_int]
        lib.oracle_quantize8.argtypes = [_p, _i64, _i64, ctypes.c_int, _p, _p]
        lib.oracle_pack8.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_unpack8.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_dequant8.argtypes = [_p, _p, _i64, _i64, ctypes.c_int, ctypes.c_int, _p]
        lib.oracle_gemm8_f64.argtypes = [_p, _i64, _i64, _p, _p, _i64, ctypes.c_int, ctypes.c_int,
                                         _p, ctypes.c_int]
        lib.oracle_gemm_bf16_f64.argtypes = [_p, _i64, _i64, _p, _p, _i64, ctypes.c_int, _p,
                                             ctypes.c_int]
        lib.oracle_quantize.argtypes = [_p, _i64, _i64, ctypes.c_int, _p, _p]
        lib.oracle_pack.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_unpack.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_dequant.argtypes = [_p, _p, _i64, _i64, ctypes.c_int, _p]
        lib.oracle_gemm_f64.argtypes = [_p, _i64, _i64, _p, _p, _i64, ctypes.c_int, _p,
                                        ctypes.c_int]
        lib.oracle_gemm_w16_f64.argtypes = [_p, _i64, _i64, _p, _i64, _p, ctypes.c_int]
        lib.oracle_swiglu_f64.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_max_threads.argtypes = []
        for name in ("oracle_quantize", "oracle_pack", "oracle_unpack", "oracle_dequant",
                     "oracle_dequant_bf16", "oracle_gemm_f64", "oracle_gemm_bf16_f64",
                     "oracle_gemm_w16_f64", "oracle_swiglu_f64", "oracle_max_threads",
                     "oracle_fold_gain", "oracle_rms_rowscale_f64", "oracle_scale_rows"):
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib
        self.path = path

    # -- binary16 ---------------------------------------------------------
    def f16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        b = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
        return np.array([self.lib.oracle_f16_to_f64(int(x)) for x in b]).reshape(np.shape(bits))

    def f64_to_f16(self, values: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(values, dtype=np.float64).ravel()
        return np.array([self.lib.oracle_f64_to_f16(float(x)) for x in v],
                        dtype=np.uint16).reshape(np.shape(values))

    # -- bfloat16 ---------------------------------------------------------
    def bf16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        b = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
        return np.array([self.lib.oracle_bf16_to_f64(int(x)) for x in b]).reshape(np.shape(bits))

    def f64_to_bf16(self, values: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(values, dtype=np.float64).ravel()
        return np.array([self.lib.oracle_f64_to_bf16(float(x)) for x in v],
                        dtype=np.uint16).reshape(np.shape(values))

    # -- format -----------------------------------------------------------
    def quantize(self, W: np.ndarray, G: int = 128):
        """Return (u [K,N] uint8 nibble values, s16 [K/G,N] fp16 bits)."""
        W = np.ascontiguousarray(W, dtype=np.float32)
        K, N = W.shape
        u = np.empty((K, N), np.uint8)
        s16 = np.empty((max(K // G, 0), N), np.uint16)
        rc = self.lib.oracle_quantize(W.ctypes.data, K, N, G, u.ctypes.data, s16.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_quantize failed with status %d" % rc)
        return u, s16

    def pack(self, u: np.ndarray) -> np.ndarray:
        u = np.ascontiguousarray(u, dtype=np.uint8)
        K, N = u.shape
        packed = np.empty((K // 8, N), np.int32)
        rc = self.lib.oracle_pack(u.ctypes.data, K, N, packed.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_pack failed with status %d" % rc)
        return packed

    def unpack(self, packed: np.ndarray) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        R, N = packed.shape
        u = np.empty((8 * R, N), np.uint8)
        rc = self.lib.oracle_unpack(packed.ctypes.data, 8 * R, N, u.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_unpack failed with status %d" % rc)
        return u

    def quantize_pack(self, W: np.ndarray, G: int = 128):
        """The data contract's quantize_pack: (packed int32 [K/8,N], s16 bits [K/G,N])."""
        u, s16 = self.quantize(W, G)
        return self.pack(u), s16

    def dequant(self, packed: np.ndarray, s16: np.ndarray, G: int = 128) -> np.ndarray:
        """fp16 bits [K,N] of (u-8)*s16, rounded once to fp16."""
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        s16 = np.ascontiguousarray(s16, dtype=np.uint16)
        R, N = packed.shape
        W16 = np.empty((8 * R, N), np.uint16)
        rc = self.lib.oracle_dequant(packed.ctypes.data, s16.ctypes.data, 8 * R, N, G,
                                     W16.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_dequant failed with status %d" % rc)
        return W16

    def dequant_bf16(self, packed: np.ndarray, s16: np.ndarray, G: int = 128) -> np.ndarray:
        """bf16 bits [K,N] of (u-8)*s16, rounded once to bf16."""
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        s16 = np.ascontiguousarray(s16, dtype=np.uint16)
        R, N = packed.shape
        Wb = np.empty((8 * R, N), np.uint16)
        rc = self.lib.oracle_dequant_bf16(packed.ctypes.data, s16.ctypes.data, 8 * R, N, G,
                                          Wb.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_dequant_bf16 failed with status %d" % rc)
        return Wb

    # -- INT8 weights (Swordfish, "The packed format"; "Making a Single GPU
    #    Go Fast", section 9.3.2) ------------------------------------------
    def quantize8(self, W: np.ndarray, G: int = 128):
        """(u uint8 [K,N] = q + 128, s16 bits [K/G,N]) with s = max|W|/127."""
        W = np.ascontiguousarray(W, dtype=np.float32)
        K, N = W.shape
        u = np.empty((K, N), np.uint8)
        s16 = np.empty((K // G, N), np.uint16)
        rc = self.lib.oracle_quantize8(W.ctypes.data, K, N, G, u.ctypes.data, s16.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_quantize8 failed with status %d" % rc)
        return u, s16

    def pack8(self, u: np.ndarray) -> np.ndarray:
        """int32 [K/4,N]: byte k at bits 8(k mod 4)."""
        u = np.ascontiguousarray(u, dtype=np.uint8)
        K, N = u.shape
        packed = np.empty((K // 4, N), np.int32)
        rc = self.lib.oracle_pack8(u.ctypes.data, K, N, packed.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_pack8 failed with status %d" % rc)
        return packed

    def unpack8(self, packed: np.ndarray) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        R, N = packed.shape
        u = np.empty((4 * R, N), np.uint8)
        rc = self.lib.oracle_unpack8(packed.ctypes.data, 4 * R, N, u.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_unpack8 failed with status %d" % rc)
        return u

    def quantize_pack8(self, W: np.ndarray, G: int = 128):
        u, s16 = self.quantize8(W, G)
        return self.pack8(u), s16

    def dequant8(self, packed: np.ndarray, s16: np.ndarray, G: int = 128,
                 bf16: bool = False) -> np.ndarray:
        """fp16 (or bf16) bits [K,N] of (u - 128) * s16, rounded once."""
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        s16 = np.ascontiguousarray(s16, dtype=np.uint16)
        R, N = packed.shape
        W = np.empty((4 * R, N), np.uint16)
        rc = self.lib.oracle_dequant8(packed.ctypes.data, s16.ctypes.data, 4 * R, N, G,
                                      int(bf16), W.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_dequant8 failed with status %d" % rc)
        return W

    def gemm8_f64(self, A: np.ndarray, packed: np.ndarray, s16: np.ndarray, G: int = 128,
                  bf16: bool = False, nthreads: int = 0) -> np.ndarray:
        """C = A * W for INT8 weights in fp64 (A fp16, or bf16 bits with bf16)."""
        A = np.ascontiguousarray(np.asarray(A).view(np.uint16))
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        s16 = np.ascontiguousarray(s16, dtype=np.uint16)
        M, K = A.shape
        R, N = packed.shape
        if 4 * R != K:
            raise ValueError("A has K=%d but packed has %d rows" % (K, R))
        C = np.empty((M, N), np.float64)
        rc = self.lib.oracle_gemm8_f64(A.ctypes.data, M, K, packed.ctypes.data, s16.ctypes.data,
                                       N, G, int(bf16), C.ctypes.data, nthreads)
        if rc != OK:
            raise ValueError("oracle_gemm8_f64 failed with status %d" % rc)
        return C

    # -- zero points (Swordfish page, section "The packed format") ---------
    def zero_rows(self, s16: np.ndarray, zp: np.ndarray) -> np.ndarray:
        """fp16 bits [K/G,N] of the prescaled zero rows fp16((8 - zp) * s16)."""
        s16 = np.ascontiguousarray(s16, dtype=np.uint16)
        zp = np.ascontiguousarray(zp, dtype=np.uint8)
        if zp.shape != s16.shape:
            raise ValueError("zero points and scales differ in shape")
        KG, N = s16.shape
        z16 = np.empty((KG, N), np.uint16)
        rc = self.lib.oracle_zero_rows(s16.ctypes.data, zp.ctypes.data, KG, N, z16.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_zero_rows failed with status %d" % rc)
        return z16

    def dequant_zp(self, packed: np.ndarray, s16: np.ndarray, z16: np.ndarray, G: int = 128,
                   bf16: bool = False) -> np.ndarray:
        """fp16 (or bf16) bits [K,N] of (u-8)*s16 + z16, rounded once."""
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        s16 = np.ascontiguousarray(s16, dtype=np.uint16)
        z16 = np.ascontiguousarray(z16, dtype=np.uint16)
        if z16.shape != s16.shape:
            raise ValueError("zero rows and scales differ in shape")
        R, N = packed.shape
        W = np.empty((8 * R, N), np.uint16)
        rc = self.lib.oracle_dequant_zp(packed.ctypes.data, s16.ctypes.data, z16.ctypes.data,
                                        8 * R, N, G, int(bf16), W.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_dequant_zp failed with status %d" % rc)
        return W

    # -- products ---------------------------------------------------------
    def gemm_f64(self, A16: np.ndarray, packed: np.ndarray, s16: np.ndarray, G: int = 128,
                 nthreads: int = 0) -> np.ndarray:
        """C = A * dequant(W) in fp64 with the exact dequantized weights.

        A16 is fp16 bits (uint16) or float16 [M,K]; returns float64 [M,N].
        """
        A16 = np.ascontiguousarray(np.asarray(A16).view(np.uint16))
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        s16 = np.ascontiguousarray(s16, dtype=np.uint16)
        M, K = A16.shape
        R, N = packed.shape
        if 8 * R != K:
            raise ValueError("A has K=%d but packed has %d rows" % (K, R))
        C = np.empty((M, N), np.float64)
        rc = self.lib.oracle_gemm_f64(A16.ctypes.data, M, K, packed.ctypes.data,
                                      s16.ctypes.data, N, G, C.ctypes.data, nthreads)
        if rc != OK:
            raise ValueError("oracle_gemm_f64 failed with status %d" % rc)
        return C

    def gemm_bf16_f64(self, Ab: np.ndarray, packed: np.ndarray, s16: np.ndarray, G: int = 128,
                      nthreads: int = 0) -> np.ndarray:
        """C = A * dequant_bf16(W) in fp64, A as bf16 bits (uint16) [M,K];
        returns float64 [M,N]."""
        Ab = np.ascontiguousarray(np.asarray(Ab).view(np.uint16))
        packed = np.ascontiguousarray(packed, dtype=np.int32)
        s16 = np.ascontiguousarray(s16, dtype=np.uint16)
        M, K = Ab.shape
        R, N = packed.shape
        if 8 * R != K:
            raise ValueError("A has K=%d but packed has %d rows" % (K, R))
        C = np.empty((M, N), np.float64)
        rc = self.lib.oracle_gemm_bf16_f64(Ab.ctypes.data, M, K, packed.ctypes.data,
                                           s16.ctypes.data, N, G, C.ctypes.data, nthreads)
        if rc != OK:
            raise ValueError("oracle_gemm_bf16_f64 failed with status %d" % rc)
        return C

    def gemm_w16_f64(self, A16: np.ndarray, W16: np.ndarray, nthreads: int = 0) -> np.ndarray:
        """A times the fp16-rounded dequantized weights, summed in fp64."""
        A16 = np.ascontiguousarray(np.asarray(A16).view(np.uint16))
        W16 = np.ascontiguousarray(np.asarray(W16).view(np.uint16))
        M, K = A16.shape
        K2, N = W16.shape
        if K != K2:
            raise ValueError("shape mismatch")
        C = np.empty((M, N), np.float64)
        self.lib.oracle_gemm_w16_f64(A16.ctypes.data, M, K, W16.ctypes.data, N,
                                     C.ctypes.data, nthreads)
        return C

    def gemm_wb_f64(self, Ab: np.ndarray, Wb: np.ndarray, nthreads: int = 0) -> np.ndarray:
        """bf16 activations times given bf16 weights (both bits), summed in fp64."""
        Ab = np.ascontiguousarray(np.asarray(Ab).view(np.uint16))
        Wb = np.ascontiguousarray(np.asarray(Wb).view(np.uint16))
        M, K = Ab.shape
        K2, N = Wb.shape
        if K != K2:
            raise ValueError("shape mismatch")
        C = np.empty((M, N), np.float64)
        self.lib.oracle_gemm_wb_f64(Ab.ctypes.data, M, K, Wb.ctypes.data, N, C.ctypes.data,
                                    nthreads)
        return C

    def fold_gain(self, W: np.ndarray, gamma: np.ndarray) -> np.ndarray:
        """W'[k,n] = fp32(gamma[k] * W[k,n]) (FuTransformer, section 3.2.2)."""
        W = np.ascontiguousarray(W, dtype=np.float32)
        gamma = np.ascontiguousarray(gamma, dtype=np.float32)
        K, N = W.shape
        if gamma.shape != (K,):
            raise ValueError("gamma must have K entries")
        Wf = np.empty_like(W)
        self.lib.oracle_fold_gain(W.ctypes.data, gamma.ctypes.data, K, N, Wf.ctypes.data)
        return Wf

    def rms_rowscale_f64(self, A: np.ndarray, eps: float, bf16: bool = False) -> np.ndarray:
        """rho[m] = (sum_k A[m,k]^2 / K + eps)^(-1/2) in fp64 (A: fp16 values or
        fp16 bits; bf16 bits with bf16=True)."""
        A = np.ascontiguousarray(np.asarray(A).view(np.uint16))
        M, K = A.shape
        rho = np.empty((M,), np.float64)
        rc = self.lib.oracle_rms_rowscale_f64(A.ctypes.data, M, K, int(bf16), float(eps),
                                              rho.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_rms_rowscale_f64 failed with status %d" % rc)
        return rho

    def scale_rows(self, C: np.ndarray, rho: np.ndarray) -> np.ndarray:
        """out[m,n] = rho[m] * C[m,n]."""
        C = np.ascontiguousarray(C, dtype=np.float64)
        rho = np.ascontiguousarray(rho, dtype=np.float64)
        M, N = C.shape
        out = np.empty_like(C)
        self.lib.oracle_scale_rows(C.ctypes.data, M, N, rho.ctypes.data, out.ctypes.data)
        return out

    def swiglu_f64(self, C: np.ndarray) -> np.ndarray:
        """Z[m,j] = silu(C[m,j]) * C[m,j+N/2] for a [M,N] gate|up product."""
        C = np.ascontiguousarray(C, dtype=np.float64)
        M, N = C.shape
        Z = np.empty((M, N // 2), np.float64)
        rc = self.lib.oracle_swiglu_f64(C.ctypes.data, M, N, Z.ctypes.data)
        if rc != OK:
            raise ValueError("oracle_swiglu_f64 failed with status %d" % rc)
        return Z

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        if (not os.path.exists(LIBRARY)
                or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        _default = Oracle(LIBRARY)
    return _default
