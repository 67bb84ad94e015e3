"""Comparison rules for GPU results against the oracle.

Floating-point GEMM outputs (fp16) are compared, as float64, with the oracle's
fp64 value (never with its fp16 rounding):
  * elementwise |C - ref| <= max(2e-2, one fp16 ulp of ref)  -- the 2e-2
    max-abs bound, widened to one ulp where fp16 output rounding alone can
    exceed it (|ref| >= 32: half an ulp is already 0.0156 .. 0.031);
  * relative L2 error ||C - ref|| / ||ref|| <= 1e-3;
  * the page's test ratio max|C - ref| / max|ref| < 2e-3;
  * every output finite.
Integer, byte and index results are compared bit for bit.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = 2e-2
REL_L2 = 1e-3
PAGE_RATIO = 2e-3


def fp16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of fp16 values at |x| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.exp2(e - 10)


def compare(out_fp16: np.ndarray, ref: np.ndarray) -> dict:
    g = np.asarray(out_fp16).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    finite = bool(np.isfinite(g).all())
    err = np.abs(g - ref)
    bound = np.maximum(MAX_ABS, fp16_ulp(ref))
    ok_elem = bool((err <= bound).all()) if finite else False
    denom = np.linalg.norm(ref)
    rel_l2 = float(np.linalg.norm(g - ref) / denom) if denom > 0 else float(np.linalg.norm(g))
    page = float(err.max() / np.abs(ref).max()) if np.abs(ref).max() > 0 else float(err.max())
    return {
        "finite": finite,
        "elementwise": ok_elem,
        "max_abs": float(err.max()) if err.size else 0.0,
        "ulp_arm_used": int(((err > MAX_ABS) & (err <= bound)).sum()),
        "rel_l2": rel_l2,
        "page_ratio": page,
        "max_ref": float(np.abs(ref).max()) if ref.size else 0.0,
    }


def assert_close(out_fp16: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    s = compare(out_fp16, ref)
    assert s["finite"], "%s: non-finite output" % what
    assert s["elementwise"], "%s: elementwise bound exceeded %s" % (what, s)
    assert s["rel_l2"] <= REL_L2, "%s: relative L2 %s" % (what, s)
    assert s["page_ratio"] < PAGE_RATIO, "%s: page ratio %s" % (what, s)
    return s


# bf16 outputs.  The pages fix no tolerance for bf16; the bound comes from the
# arithmetic.  A bf16 output has 8 significant bits, so its one rounding alone
# moves an element by up to half an ulp (2^-8 relative, 2^-9 at the top of a
# binade) and the relative L2 error of a rounded matrix is about 2^-8/sqrt(3)
# ~ 2.3e-3 at worst; FP32 accumulation adds ~1e-6.  So, against the fp64
# oracle (whose weights are the same bf16 values):
#   * elementwise |C - ref| <= max(2e-2, one bf16 ulp of ref);
#   * relative L2 <= 4e-3;  page ratio max|C - ref| / max|ref| < 8e-3
#     (one bf16 ulp at the largest element is up to 2^-7 of it).
REL_L2_BF16 = 4e-3
PAGE_RATIO_BF16 = 8e-3


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^-133 in the subnormal range)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_close_bf16(out_bits: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    g = bf16_bits_to_f64(out_bits)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    finite = bool(np.isfinite(g).all())
    err = np.abs(g - ref)
    ok = bool((err <= np.maximum(MAX_ABS, bf16_ulp(ref))).all()) if finite else False
    denom = np.linalg.norm(ref)
    rel_l2 = float(np.linalg.norm(g - ref) / denom) if denom > 0 else float(np.linalg.norm(g))
    page = float(err.max() / np.abs(ref).max()) if np.abs(ref).max() > 0 else float(err.max())
    s = {"finite": finite, "elementwise": ok, "max_abs": float(err.max()) if err.size else 0.0,
         "rel_l2": rel_l2, "page_ratio": page}
    assert finite, "%s: non-finite output" % what
    assert ok, "%s: elementwise bound exceeded %s" % (what, s)
    assert rel_l2 <= REL_L2_BF16, "%s: relative L2 %s" % (what, s)
    assert page < PAGE_RATIO_BF16, "%s: page ratio %s" % (what, s)
    return s
