"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws numbers and builds shapes: it holds none of the W4A16
arithmetic (no quantizer, no packing, no dequantization, no product), so the
oracle and the GPU path can both be fed from it without sharing any of the
method's code.

Recipe (numpy PCG64):
  * weights W [K,N] fp32 = standard_normal * 0.02, generator seeded with ``seed``;
  * activations A [M,K]: standard_normal fp32 from a generator seeded with
    ``seed + 1``; for the outlier batches, round(0.01 K) channels drawn as
    ``permutation(K)[:n]`` from the same generator after A are scaled by 20 in
    fp32; then A is cast to fp16 (round to nearest even).
The shapes are those of Llama-8B / 70B projections: QKV, O, fused gate/up
(with a SwiGLU epilogue, output width N/2) and down.
"""
from __future__ import annotations

import numpy as np

G = 128

# Projection shapes (K, N, swiglu) per model.
LLAMA_8B = {
    "qkv": (4096, 6144, False),
    "o": (4096, 4096, False),
    "gate_up": (4096, 28672, True),
    "down": (14336, 4096, False),
}
LLAMA_70B = {
    "qkv": (8192, 10240, False),
    "o": (8192, 8192, False),
    "gate_up": (8192, 57344, True),
    "down": (28672, 8192, False),
}

# The five workloads: name -> list of (label, M, K, N, swiglu, outliers).
CONFIGS = {
    "gemv": [("gemv", 1, 4096, 4096, False, False)],
    "decode_8b": [("8b_%s_m%d" % (p, m), m, k, n, sw, False)
                  for m in (1, 8, 16, 32) for p, (k, n, sw) in LLAMA_8B.items()],
    "decode_70b": [("70b_%s_m%d" % (p, m), m, k, n, sw, False)
                   for m in (1, 4, 16, 32) for p, (k, n, sw) in LLAMA_70B.items()],
    "transition": [("trans_%s_m%d" % (p, m), m, k, n, False, True)
                   for m in (64, 128, 256)
                   for p, (k, n) in (("up", (4096, 28672)), ("down", (14336, 4096)))],
    "prefill": [("prefill_%s_m%d" % (p, m), m, k, n, sw, False)
                for m in (4096, 8191)
                for p, (k, n, sw) in (("gate_up", (4096, 28672, True)),
                                      ("down", (14336, 4096, False)))],
    "fallback": [("fallback_%s_m%d" % (p, m), m, k, n, sw, False)
                 for m in (16384,)
                 for p, (k, n, sw) in (("gate_up", (4096, 28672, True)),
                                       ("down", (14336, 4096, False)))],
}

# Shapes of the page's shape-parametrised test (M, K, N).
PAGE_TEST_SHAPES = [(1, 4096, 4096), (7, 4096, 11008), (33, 11008, 4096),
                    (512, 4096, 4096), (1, 4096, 4160)]


def weights(K: int, N: int, seed: int = 0) -> np.ndarray:
    """W [K,N] fp32 ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((K, N), dtype=np.float32)
    W *= np.float32(0.02)
    return W


def activations(M: int, K: int, seed: int = 0, outliers: bool = False) -> np.ndarray:
    """A [M,K] fp16 ~ N(0,1), optionally with 1% of K-channels scaled by 20."""
    rng = np.random.default_rng(seed + 1)
    A = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        idx = outlier_channels(K, rng)
        A[:, idx] *= np.float32(20.0)
    return A.astype(np.float16)


def activations_bf16(M: int, K: int, seed: int = 0, outliers: bool = False) -> np.ndarray:
    """The same draw as ``activations`` cast to bf16 (nearest even) instead of
    fp16; returned as the uint16 bit patterns."""
    rng = np.random.default_rng(seed + 1)
    A = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        idx = outlier_channels(K, rng)
        A[:, idx] *= np.float32(20.0)
    import torch
    return torch.from_numpy(A).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def outlier_channels(K: int, rng: np.random.Generator) -> np.ndarray:
    n_out = int(round(0.01 * K))
    return rng.permutation(K)[:n_out]


# -- structured inputs for exact-result tests ------------------------------

def grid_weights(K: int, N: int, p: int = 6, seed: int = 0, group: int = G) -> np.ndarray:
    """W = j * 2^-p with integer j in [-7, 7], and one entry of every
    (group, column) set to +-7 * 2^-p, so that each group's maximum is exactly
    7 * 2^-p (its scale is then 2^-p and the quantization is lossless).
    ``group`` is the group size the property is built for."""
    rng = np.random.default_rng(seed)
    j = rng.integers(-7, 8, size=(K, N)).astype(np.float32)
    rows = np.arange(0, K, group)[:, None] + rng.integers(0, group, size=(K // group, N))
    sign = np.where(rng.integers(0, 2, size=(K // group, N)) == 0, -7.0, 7.0).astype(np.float32)
    j[rows, np.arange(N)[None, :]] = sign
    return j * np.float32(2.0 ** -p)


def grid_weights8(K: int, N: int, p: int = 10, seed: int = 0, group: int = G) -> np.ndarray:
    """The 8-bit counterpart of ``grid_weights``: W = j * 2^-p with integer j in
    [-127, 127] and one entry of every (group, column) set to +-127 * 2^-p, so
    that each group's scale is exactly 2^-p and 8-bit quantization is lossless."""
    rng = np.random.default_rng(seed)
    j = rng.integers(-127, 128, size=(K, N)).astype(np.float32)
    rows = np.arange(0, K, group)[:, None] + rng.integers(0, group, size=(K // group, N))
    sign = np.where(rng.integers(0, 2, size=(K // group, N)) == 0, -127.0, 127.0).astype(np.float32)
    j[rows, np.arange(N)[None, :]] = sign
    return j * np.float32(2.0 ** -p)


def random_bytes(K: int, N: int, seed: int = 0, group: int = G) -> tuple[np.ndarray, np.ndarray]:
    """Arbitrary 8-bit codes (every value 0..255, including 0, which the
    quantizer never emits) packed four per int32 along K (byte k at bits
    8(k mod 4)), with positive fp16 scales in [2^-12, 2^-8), one per ``group``
    rows."""
    rng = np.random.default_rng(seed + 6)
    packed = rng.integers(0, 2 ** 32, size=(K // 4, N), dtype=np.uint64).astype(np.uint32)
    scales = (rng.random((K // group, N), dtype=np.float32) * np.float32(2.0 ** -8 - 2.0 ** -12)
              + np.float32(2.0 ** -12)).astype(np.float16)
    return packed.view(np.int32), scales.view(np.uint16)


def onehot_activations(M: int, K: int, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """A[m, k(m)] = 1, zero elsewhere; returns (A fp16, k(m))."""
    rng = np.random.default_rng(seed + 2)
    ks = rng.integers(0, K, size=M)
    A = np.zeros((M, K), np.float16)
    A[np.arange(M), ks] = 1.0
    return A, ks


def ternary_activations(M: int, K: int, density: float = 1.0, seed: int = 0) -> np.ndarray:
    """A in {-1, 0, +1} (fp16), nonzero with probability ``density``."""
    rng = np.random.default_rng(seed + 3)
    vals = rng.choice(np.array([-1.0, 1.0], np.float32), size=(M, K))
    keep = rng.random((M, K)) < density
    return np.where(keep, vals, 0.0).astype(np.float16)


def zero_points(KG: int, N: int, seed: int = 0) -> np.ndarray:
    """Zero points [KG, N] (uint8) of asymmetric 4-bit weights: mostly near
    the middle of 0..15, as min/max quantization of roughly centred groups
    gives, with every value 0..15 present."""
    rng = np.random.default_rng(seed + 5)
    z = np.clip(np.rint(rng.normal(7.5, 2.5, (KG, N))), 0, 15).astype(np.uint8)
    flat = z.reshape(-1)
    flat[: min(16, flat.size)] = np.arange(min(16, flat.size), dtype=np.uint8)
    return z


def random_words(K: int, N: int, seed: int = 0, group: int = G) -> tuple[np.ndarray, np.ndarray]:
    """Arbitrary packed words (every nibble 0..15, including 0, which the RTN
    quantizer never emits) with positive fp16 scales in [2^-9, 2^-5), one per
    `group` rows."""
    rng = np.random.default_rng(seed + 4)
    packed = rng.integers(0, 2 ** 32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32)
    scales = (rng.random((K // group, N), dtype=np.float32) * np.float32(2.0 ** -5 - 2.0 ** -9)
              + np.float32(2.0 ** -9)).astype(np.float16)
    return packed.view(np.int32), scales.view(np.uint16)
