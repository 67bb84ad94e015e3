"""Pins for the oracle: each check ties one oracle function to something other
than the oracle itself (a value the pages print, a closed form, an invariant,
a library routine on a special case, or brute force on tiny inputs).

Every check takes an ``oracle.Oracle`` instance and raises AssertionError on a
mismatch, so the same checks run against the real oracle and against copies of
it with a planted mistake (which must fail at least one check).
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy import integrate, special

from weight_only_int4_03_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _word(nibbles):
    """int32 value of a word whose nibble i (bits 4i..4i+3) is nibbles[i],
    built from its hexadecimal spelling (most significant nibble first)."""
    v = int("".join("%X" % x for x in reversed(nibbles)), 16)
    return v - (1 << 32) if v >= (1 << 31) else v


# -- IEEE binary16 ---------------------------------------------------------

def check_f16_decode(o):
    """Every binary16 bit pattern decodes as numpy's float16 does."""
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint32).astype(np.uint16)
    bits = np.concatenate([bits, np.array([0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF,
                                           0x7C00, 0x8001, 0xFBFF, 0xFC00], np.uint16)])
    ours = o.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isinf(ours), np.isinf(ref))


def check_f16_encode(o):
    """Rounding to binary16 agrees with numpy's correctly rounded cast,
    including exact ties (to even), subnormals and the overflow threshold."""
    rng = np.random.default_rng(7)
    vals = np.arange(0, 0x7C00, 37, dtype=np.uint32).astype(np.uint16).view(np.float16)
    vals = vals.astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0                         # exact ties
    offs = vals[:-1] + (vals[1:] - vals[:-1]) * rng.random(len(vals) - 1)
    specials = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24,
                         2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, 1e-8,
                         np.float64(np.float32(1e-8)), 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11])
    x = np.concatenate([vals, mids, offs, -mids, specials, -specials])
    ours = o.f64_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


# -- bfloat16 ------------------------------------------------------------------

def _torch_bf16_bits(x64):
    """torch's float32 -> bfloat16 cast (round to nearest even) of values
    that are exact in float32, as uint16 bits."""
    import torch
    t = torch.from_numpy(np.asarray(x64, np.float64).astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def check_bf16_decode(o):
    """Every sampled bfloat16 bit pattern decodes as the upper half of the
    binary32 with those bits (numpy's float32)."""
    bits = np.arange(0, 1 << 16, 61, dtype=np.uint32).astype(np.uint16)
    bits = np.concatenate([bits, np.array([0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x7F7F,
                                           0x7F80, 0x8001, 0xFF7F, 0xFF80], np.uint16)])
    ours = o.bf16_to_f64(bits)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isinf(ours), np.isinf(ref))
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def check_bf16_encode(o):
    """Rounding to bfloat16 agrees with torch's cast on float32-exact values:
    exact ties (to even), values between neighbours, subnormals, overflow."""
    rng = np.random.default_rng(17)
    bits = np.arange(0, 0x7F80, 41, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0                         # exact ties, fp32-exact
    frac = np.floor(rng.random(len(vals) - 1) * 65536) / 65536  # fp32-exact offsets
    offs = vals[:-1] + (vals[1:] - vals[:-1]) * frac
    specials = np.array([0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 3.0e38,
                         float(np.float32(3.39e38)), 2.0 ** -133, 2.0 ** -134,
                         3 * 2.0 ** -135, 2.0 ** -126 - 2.0 ** -134, 65504.0, 1e-8])
    x = np.concatenate([vals, mids, offs, -mids, specials, -specials])
    x = x[np.float32(x).astype(np.float64) == x]                  # keep fp32-exact inputs
    ours = o.f64_to_bf16(x)
    ref = _torch_bf16_bits(x)
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


# -- packing ------------------------------------------------------------------

def check_pack_worked_words(o):
    """Worked words fixed by the data contract (value k at bits 4(k mod 8))."""
    g = _golden("packed_words.json")
    cases = g["cases"]
    u = np.array([c["nibbles"] for c in cases], np.uint8).T      # [8, ncases]
    packed = o.pack(u)
    assert packed.shape == (1, len(cases))
    for i, c in enumerate(cases):
        assert int(packed[0, i]) == c["int32"], (c, int(packed[0, i]))
        assert int(packed[0, i]) == _word(c["nibbles"])
        assert (int(packed[0, i]) < 0) == (c["nibbles"][7] >= 8)


def check_pack_roundtrip(o):
    """unpack(pack(u)) == u for every nibble value at every position."""
    u = np.zeros((8 * 16, 8), np.uint8)
    for pos in range(8):
        for val in range(16):
            u[8 * val + pos, pos] = val
    rng = np.random.default_rng(3)
    u = np.concatenate([u, rng.integers(0, 16, size=(8 * 16, 8)).astype(np.uint8)], axis=1)
    assert np.array_equal(o.unpack(o.pack(u)), u)


def check_unpack_sign_words(o):
    """Words with a top nibble >= 8 (negative int32) unpack to 0..15 values."""
    rng = np.random.default_rng(11)
    nibs = rng.integers(0, 16, size=(64, 8))
    nibs[:, 7] = rng.integers(8, 16, size=64)
    words = np.array([[_word(list(r)) for r in nibs]], np.int32)  # [1, 64]
    assert (words < 0).all()
    u = o.unpack(words)
    assert np.array_equal(u.T, nibs.astype(np.uint8))


# -- quantizer ------------------------------------------------------------------

def check_quantize_group_max(o):
    """RTN with s = amax/7: the group's largest |w| maps to q = +-7 and no
    nibble 0 (q = -8) appears; every nibble lies in 1..15."""
    W = synth.weights(512, 24, seed=5)
    u, s16 = o.quantize(W)
    for g in range(512 // 128):
        blk = W[128 * g:128 * (g + 1)]
        kmax = np.abs(blk).argmax(axis=0)
        got = u[128 * g + kmax, np.arange(24)].astype(int) - 8
        assert np.array_equal(np.abs(got), np.full(24, 7))
        assert np.array_equal(np.sign(got), np.sign(blk[kmax, np.arange(24)]).astype(int))
    assert u.min() >= 1 and u.max() <= 15


def check_quantize_grid_roundtrip(o):
    """W = j * 2^-p with a +-7 entry in every group: scale is 2^-p exactly and
    dequantization gives W back bit for bit."""
    for p in (4, 6, 9):
        W = synth.grid_weights(256, 16, p=p, seed=p)
        u, s16 = o.quantize(W)
        assert np.array_equal(s16, np.full_like(s16, np.float16(2.0 ** -p).view(np.uint16)))
        assert np.array_equal(u.astype(np.float32) - 8, W * np.float32(2.0 ** p))
        W16 = o.dequant(o.pack(u), s16)
        assert np.array_equal(W16, W.astype(np.float16).view(np.uint16))


def check_quantize_ties_to_even(o):
    """With group maximum 7.0 the scale is exactly 1.0, so w/s is w itself and
    x.5 values are exact ties: round-half-to-even decides them."""
    col = np.zeros(128, np.float32)
    col[0] = 7.0
    vals = [2.5, -2.5, 0.5, -0.5, 1.5, 3.5, -3.5, 6.5, 5.5, 4.5, 2.4, 2.6]
    expect_q = [2, -2, 0, 0, 2, 4, -4, 6, 6, 4, 2, 3]
    col[1:1 + len(vals)] = vals
    u, s16 = o.quantize(col[:, None])
    assert int(s16[0, 0]) == 0x3C00                        # fp16 1.0
    assert u[0, 0] == 15
    assert [int(x) - 8 for x in u[1:1 + len(vals), 0]] == expect_q


def check_quantize_scale_value(o):
    """The stored scale is fp16(fl32(amax / 7)), here for amax in {1, 0.02}."""
    for amax in (1.0, 0.02, 3.0):
        col = np.zeros((128, 1), np.float32)
        col[17, 0] = -np.float32(amax)
        _, s16 = o.quantize(col)
        expect = (np.float32(amax) / np.float32(7.0)).astype(np.float16).view(np.uint16)
        assert int(s16[0, 0]) == int(expect)


def check_quantize_zero_group(o):
    """An all-zero group: scale max(0, 1e-8) rounds to fp16 zero, nibbles 8."""
    W = synth.weights(256, 4, seed=9)
    W[128:, 2] = 0.0
    u, s16 = o.quantize(W)
    assert int(s16[1, 2]) == 0
    assert (u[128:, 2] == 8).all()
    assert (s16[0] != 0).all()


def _expected_max_sq(n=128):
    """E[max^2] of n iid half-normal variables (numerical integral)."""
    f = lambda x: x * x * n * special.erf(x / np.sqrt(2)) ** (n - 1) * np.sqrt(2 / np.pi) \
        * np.exp(-x * x / 2)
    return integrate.quad(f, 0, 12)[0]


def check_quantization_error_closed_form(o):
    """Relative RMS quantization error of Gaussian weights at G=128:
    sqrt(E[max^2] / (12 * 49) * 127/128) (uniform rounding error of width
    s = max/7 on the 127 non-maximal entries)."""
    W = synth.weights(1024, 512, seed=1)
    u, s16 = o.quantize(W)
    W16 = o.dequant(o.pack(u), s16).view(np.float16).astype(np.float64)
    rel = np.sqrt(np.mean((W16 - W) ** 2)) / np.sqrt(np.mean(W.astype(np.float64) ** 2))
    theory = np.sqrt(_expected_max_sq() / (12 * 49) * 127 / 128)
    assert abs(theory - 0.1173) < 5e-4, theory
    assert abs(rel - theory) < 2.5e-3, (rel, theory)


def check_quantize_other_group_sizes(o):
    """G = 32, 64, 256 and channelwise (G = K): each group's scale is numpy's
    fp16(fl32(amax / 7)), its largest |w| lands on q = +-7, and the product
    equals numpy's float64 matmul of the exact weights."""
    rng = np.random.default_rng(31)
    K, N = 512, 12
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    A = rng.standard_normal((2, K)).astype(np.float16)
    for G in (32, 64, 256, K):
        packed, s16 = o.quantize_pack(W, G)
        assert s16.shape == (K // G, N)
        amax = np.abs(W.reshape(K // G, G, N)).max(axis=1)
        assert np.array_equal(s16, (amax / np.float32(7.0)).astype(np.float16).view(np.uint16))
        u = o.unpack(packed).reshape(K // G, G, N)
        at = np.abs(W.reshape(K // G, G, N)).argmax(axis=1)
        for g in range(K // G):
            for n in range(N):
                assert u[g, at[g, n], n] in (1, 15)
        Wx = (o.unpack(packed).astype(np.float64) - 8) * np.repeat(
            s16.view(np.float16).astype(np.float64), G, axis=0)
        assert np.allclose(o.gemm_f64(A, packed, s16, G), np.matmul(A.astype(np.float64), Wx),
                           rtol=1e-12, atol=1e-12)


# -- dequantization ------------------------------------------------------------

def check_dequant_special_values(o):
    """u = 8 gives +0; u = 0 gives -8 s exactly; u = 15 gives 7 s (exact for a
    power-of-two scale)."""
    u = np.full((128, 3), 8, np.uint8)
    u[5, 1] = 0
    u[6, 2] = 15
    s = np.array([[np.float16(0.3).view(np.uint16), np.float16(2.0 ** -7).view(np.uint16),
                   np.float16(2.0 ** -7).view(np.uint16)]], np.uint16)
    W16 = o.dequant(o.pack(u), s)
    assert (W16[:, 0] == 0).all()
    assert W16[5, 1] == np.float16(-8 * 2.0 ** -7).view(np.uint16)
    assert W16[6, 2] == np.float16(7 * 2.0 ** -7).view(np.uint16)


def check_dequant_rounds_once(o):
    """For an arbitrary fp16 scale the result is fp16 of the exact product,
    compared here with numpy's correctly rounded float64 -> float16 cast."""
    packed, s16 = synth.random_words(256, 16, seed=4)
    u = o.unpack(packed).astype(np.float64)
    s = s16.view(np.float16).astype(np.float64)
    exact = (u - 8) * np.repeat(s, 128, axis=0)
    W16 = o.dequant(packed, s16)
    assert np.array_equal(W16, exact.astype(np.float16).view(np.uint16))


def check_dequant_bf16_rounds_once(o):
    """bf16 weights are bf16 of the exact product (fp32-exact: at most 15
    significant bits), compared with torch's cast."""
    packed, s16 = synth.random_words(256, 16, seed=14)
    u = o.unpack(packed).astype(np.float64)
    s = s16.view(np.float16).astype(np.float64)
    exact = (u - 8) * np.repeat(s, 128, axis=0)
    Wb = o.dequant_bf16(packed, s16)
    assert np.array_equal(Wb, _torch_bf16_bits(exact))
    # u = 8 gives +0, power-of-two scales are exact.
    assert (Wb[(o.unpack(packed) == 8)] == 0).all()


# -- zero points (Swordfish page, section "The packed format") -------------------

def _f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def check_zero_rows(o):
    """z = fp16((8 - zp) s): zp = 8 gives +0, zp = 0 gives 8 s exactly,
    power-of-two scales are exact, z(16 - zp) = -z(zp) (round to nearest even
    is odd-symmetric), and arbitrary scales round as numpy's correctly rounded
    float64 -> float16 cast of the exact product."""
    rng = np.random.default_rng(31)
    s16 = _f16(rng.random((4, 24)) * 0.05 + 1e-3)
    zp = rng.integers(0, 16, (4, 24)).astype(np.uint8)
    s = s16.view(np.float16).astype(np.float64)
    z = o.zero_rows(s16, zp)
    assert np.array_equal(z, _f16((8.0 - zp) * s))
    assert (o.zero_rows(s16, np.full_like(zp, 8)) == 0).all()
    assert np.array_equal(o.zero_rows(s16, np.zeros_like(zp)), _f16(8.0 * s))
    p2 = _f16(np.exp2(rng.integers(-14, -2, (4, 24))))
    assert np.array_equal(o.zero_rows(p2, zp).view(np.float16).astype(np.float64),
                          (8.0 - zp) * p2.view(np.float16).astype(np.float64))
    inner = (zp >= 1) & (zp <= 15)
    mirrored = o.zero_rows(s16, np.where(inner, 16 - zp, zp).astype(np.uint8))
    f = lambda b: b.view(np.float16).astype(np.float64)
    assert np.array_equal(f(mirrored[inner]), -f(z[inner]))


def check_dequant_zp_worked_examples(o):
    """The hand-worked binary16 cases of tests/golden/zero_point_examples.json
    (a single rounding of (q - 8) s + z, with z itself rounded)."""
    for c in _golden("zero_point_examples.json")["cases"]:
        u = np.full((128, 1), 8, np.uint8)
        u[0, 0] = c["q"]
        s16 = np.array([[int(c["s_bits"], 16)]], np.uint16)
        z = o.zero_rows(s16, np.array([[c["zp"]]], np.uint8))
        assert z[0, 0] == int(c["z_bits"], 16)
        packed = o.pack(u)
        assert o.dequant_zp(packed, s16, z)[0, 0] == int(c["w_f16_bits"], 16)
        assert o.dequant_zp(packed, s16, z, bf16=True)[0, 0] == int(c["w_bf16_bits"], 16)


def check_dequant_zp_reduces_to_symmetric(o):
    """zp = 8 makes every zero row +0, and the weights are then the symmetric
    format's, fp16 and bf16, for any group size."""
    for G in (32, 128):
        packed, s16 = synth.random_words(256, 16, seed=32 + G, group=G)
        z = o.zero_rows(s16, np.full(s16.shape, 8, np.uint8))
        assert np.array_equal(o.dequant_zp(packed, s16, z, G), o.dequant(packed, s16, G))
        assert np.array_equal(o.dequant_zp(packed, s16, z, G, bf16=True),
                              o.dequant_bf16(packed, s16, G))


def check_dequant_zp_power_of_two_exact(o):
    """Power-of-two scales make z and the weight exact: w = (q - zp) s, the
    textbook asymmetric dequantization, with the zero point of the right group
    and column."""
    rng = np.random.default_rng(33)
    K, N, G = 256, 16, 64
    u = rng.integers(0, 16, (K, N)).astype(np.uint8)
    zp = rng.integers(0, 16, (K // G, N)).astype(np.uint8)
    s16 = _f16(np.exp2(rng.integers(-12, -4, (K // G, N))))
    z = o.zero_rows(s16, zp)
    want = (u.astype(np.float64) - np.repeat(zp, G, axis=0)) * \
        np.repeat(s16.view(np.float16).astype(np.float64), G, axis=0)
    for bf16 in (False, True):
        W = o.dequant_zp(o.pack(u), s16, z, G, bf16=bf16)
        got = o.bf16_to_f64(W) if bf16 else W.view(np.float16).astype(np.float64)
        assert np.array_equal(got, want)


def check_dequant_zp_error_bound(o):
    """For arbitrary scales the weight is within half an fp16 ulp of z plus
    half an ulp of the result of the exact (q - zp) s."""
    rng = np.random.default_rng(34)
    K, N = 256, 24
    u = rng.integers(0, 16, (K, N)).astype(np.uint8)
    zp = rng.integers(0, 16, (K // 128, N)).astype(np.uint8)
    s16 = _f16(rng.random((K // 128, N)) * 0.02 + 1e-3)
    z = o.zero_rows(s16, zp)
    W = o.dequant_zp(o.pack(u), s16, z).view(np.float16).astype(np.float64)
    s = np.repeat(s16.view(np.float16).astype(np.float64), 128, axis=0)
    zf = np.repeat(z.view(np.float16).astype(np.float64), 128, axis=0)
    exact = (u.astype(np.float64) - np.repeat(zp, 128, axis=0)) * s
    ulp = lambda x: np.spacing(np.abs(x).astype(np.float16)).astype(np.float64)
    assert (np.abs(W - exact) <= ulp(zf) / 2 + ulp(W) / 2).all()
    assert np.array_equal(o.dequant_zp(o.pack(u), s16, z).view(np.float16).astype(np.float64),
                          W)


def check_gemm_wb_reference(o):
    """The bf16 given-weight product equals numpy's float64 matmul and, for
    the symmetric weights, the bf16 GEMM reference bit for bit."""
    rng = np.random.default_rng(35)
    packed, s16 = synth.random_words(256, 16, seed=35)
    Ab = _torch_bf16_bits(rng.standard_normal((3, 256)).astype(np.float32))
    Wb = o.dequant_bf16(packed, s16)
    C = o.gemm_wb_f64(Ab, Wb)
    assert np.array_equal(C, o.gemm_bf16_f64(Ab, packed, s16))
    ref = np.matmul(o.bf16_to_f64(Ab), o.bf16_to_f64(Wb))
    assert np.allclose(C, ref, rtol=1e-12, atol=1e-12)


# -- INT8 weights (Swordfish, "The packed format"; "Making a Single GPU Go
#    Fast", section 9.3.2) ----------------------------------------------------

def check_pack8_worked_words(o):
    """The hand-derived words of tests/golden/packed_bytes.json."""
    for c in _golden("packed_bytes.json")["cases"]:
        u = np.array(c["bytes"], np.uint8).reshape(4, 1)
        w = o.pack8(u)
        assert w.shape == (1, 1) and int(w[0, 0]) == c["int32"], c
        assert np.array_equal(o.unpack8(w)[:, 0], u[:, 0]), c


def check_pack8_roundtrip(o):
    """unpack8(pack8(u)) == u, and the packed words are numpy's little-endian
    view of the bytes taken four at a time along K."""
    rng = np.random.default_rng(41)
    u = rng.integers(0, 256, (64, 12)).astype(np.uint8)
    w = o.pack8(u)
    assert np.array_equal(o.unpack8(w), u)
    le = np.ascontiguousarray(u.reshape(16, 4, 12).transpose(0, 2, 1)).view("<u4")[..., 0]
    assert np.array_equal(w.view(np.uint32), le)


def check_quantize8_grid_roundtrip(o):
    """Grid weights j 2^-p with a +-127 2^-p entry per group quantize
    losslessly: scale 2^-p, codes j + 128, dequantized weights equal W."""
    for G in (128, 64):
        W = synth.grid_weights8(512, 16, p=10, seed=G, group=G)
        u, s16 = o.quantize8(W, G)
        assert (s16 == np.float16(2.0 ** -10).view(np.uint16)).all()
        assert np.array_equal(u.astype(np.int64) - 128, np.rint(W * 2.0 ** 10).astype(np.int64))
        Wd = o.dequant8(o.pack8(u), s16, G).view(np.float16).astype(np.float64)
        assert np.array_equal(Wd, W.astype(np.float64))


def check_quantize8_group_max_and_zero_group(o):
    """The group maximum maps to code 255 (or 1 for a negative maximum), the
    scale is fp16(max / 127); an all-zero group has scale fp16(1e-8) = 0 and
    codes 128."""
    W = np.zeros((256, 3), np.float32)
    W[5, 0], W[6, 0] = 0.3, -0.1
    W[130, 1] = -2.5
    u, s16 = o.quantize8(W)
    assert u[5, 0] == 255 and u[130, 1] == 1
    assert s16[0, 0] == np.float16(np.float32(0.3) / np.float32(127)).view(np.uint16)
    assert (s16[:, 2] == 0).all() and (u[:, 2] == 128).all()


def check_quantize8_ties_to_even(o):
    """Exact ties (k + 1/2) s round to the even k."""
    s = 2.0 ** -7
    W = np.zeros((128, 1), np.float32)
    W[0, 0] = 127 * s                                   # sets the scale to 2^-7
    W[1:6, 0] = np.array([0.5, 1.5, 2.5, -0.5, -3.5]) * s
    u, _ = o.quantize8(W)
    assert list(u[1:6, 0].astype(int) - 128) == [0, 2, 2, 0, -4]


def check_quantize8_error_bound(o):
    """|W - (u - 128) s| <= s / 2 with the quantizer's fp32 scale s (random
    Gaussian weights, no clamping at +-127 since |W| <= 127 s)."""
    rng = np.random.default_rng(42)
    W = (rng.standard_normal((256, 24)) * 0.02).astype(np.float32)
    u, _ = o.quantize8(W)
    amax = np.abs(W.reshape(2, 128, 24)).max(axis=1)
    s = np.repeat((amax / np.float32(127)).astype(np.float32), 128, axis=0).astype(np.float64)
    err = np.abs(W.astype(np.float64) - (u.astype(np.float64) - 128) * s)
    assert (err <= s / 2 * (1 + 1e-6)).all()


def check_dequant8_values(o):
    """Code 0 gives -128 s, 128 gives +0, 255 gives 127 s; arbitrary scales
    round once (numpy's correctly rounded cast of the exact product); bf16 as
    torch rounds."""
    packed, s16 = synth.random_bytes(256, 16, seed=43)
    u = o.unpack8(packed).astype(np.float64)
    s = np.repeat(s16.view(np.float16).astype(np.float64), 128, axis=0)
    exact = (u - 128) * s
    assert np.array_equal(o.dequant8(packed, s16), exact.astype(np.float16).view(np.uint16))
    assert np.array_equal(o.dequant8(packed, s16, bf16=True), _torch_bf16_bits(exact))
    p2 = np.full((128, 3), 128, np.uint8)
    p2[1, 0], p2[2, 1] = 0, 255
    s2 = np.array([[np.float16(2.0 ** -7).view(np.uint16)] * 3], np.uint16)
    W = o.dequant8(o.pack8(p2), s2).view(np.float16).astype(np.float64)
    assert W[1, 0] == -1.0 and W[2, 1] == 127 * 2.0 ** -7 and (W[:, 2] == 0).all()


def check_gemm8_bruteforce_and_exact(o):
    """Tiny shapes against numpy's float64 matmul of the exact weights (fp16
    activations) and of the bf16-rounded weights (bf16 activations); one-hot
    rows select weight rows exactly; grid weights with ternary activations
    give numpy's exact product."""
    rng = np.random.default_rng(44)
    for M, K, N, G in ((1, 128, 8, 128), (3, 256, 16, 64)):
        packed, s16 = synth.random_bytes(K, N, seed=M + K, group=G)
        Wx = (o.unpack8(packed).astype(np.float64) - 128) * np.repeat(
            s16.view(np.float16).astype(np.float64), G, axis=0)
        A = rng.standard_normal((M, K)).astype(np.float16)
        assert np.allclose(o.gemm8_f64(A, packed, s16, G), A.astype(np.float64) @ Wx,
                           rtol=1e-12, atol=1e-12)
        Ab = _torch_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        Wb = o.bf16_to_f64(_torch_bf16_bits(Wx))
        assert np.allclose(o.gemm8_f64(Ab, packed, s16, G, bf16=True), o.bf16_to_f64(Ab) @ Wb,
                           rtol=1e-12, atol=1e-12)
    packed, s16 = synth.random_bytes(256, 8, seed=45)
    A, ks = synth.onehot_activations(4, 256, seed=45)
    C = o.gemm8_f64(A, packed, s16)
    u = o.unpack8(packed).astype(np.float64)
    for m, k in enumerate(ks):
        assert np.array_equal(C[m], (u[k] - 128) * s16[k // 128].view(np.float16).astype(np.float64))
    W = synth.grid_weights8(512, 16, seed=46)
    p8, s8 = o.quantize_pack8(W)
    A = synth.ternary_activations(3, 512, density=0.5, seed=46)
    assert np.array_equal(o.gemm8_f64(A, p8, s8), A.astype(np.float64) @ W.astype(np.float64))


# -- GEMM ------------------------------------------------------------------------

def _exact_weights(o, packed, s16, G=128):
    u = o.unpack(packed).astype(np.float64)
    return (u - 8) * np.repeat(s16.view(np.float16).astype(np.float64), G, axis=0)


def check_gemm_bruteforce(o):
    """Tiny shapes against numpy's float64 matmul of the exact weights."""
    rng = np.random.default_rng(2)
    for M, K, N in ((1, 128, 8), (3, 256, 16), (2, 256, 8)):
        packed, s16 = synth.random_words(K, N, seed=M + K + N)
        A = rng.standard_normal((M, K)).astype(np.float16)
        C = o.gemm_f64(A, packed, s16)
        ref = np.matmul(A.astype(np.float64), _exact_weights(o, packed, s16))
        assert C.shape == (M, N)
        assert np.allclose(C, ref, rtol=1e-12, atol=1e-12)


def check_gemm_onehot(o):
    """One-hot rows of A select rows of the weight matrix exactly."""
    K, N = 384, 24
    packed, s16 = synth.random_words(K, N, seed=8)
    A, ks = synth.onehot_activations(5, K, seed=8)
    C = o.gemm_f64(A, packed, s16)
    u = o.unpack(packed).astype(np.float64)
    for m, k in enumerate(ks):
        row = (u[k] - 8) * s16[k // 128].view(np.float16).astype(np.float64)
        assert np.array_equal(C[m], row)


def check_gemm_integer_exact(o):
    """Ternary A with power-of-two scales: every partial sum is an exact
    multiple of 2^-p, so the product equals numpy's float64 matmul exactly."""
    K, N = 512, 16
    W = synth.grid_weights(K, N, p=4, seed=3)
    packed, s16 = o.quantize_pack(W)
    A = synth.ternary_activations(4, K, density=0.7, seed=3)
    C = o.gemm_f64(A, packed, s16)
    assert np.array_equal(C, np.matmul(A.astype(np.float64), W.astype(np.float64)))


def check_gemm_all_ones(o):
    """A = 1: C[n] = sum_g s16[g,n] * sum_{k in g} (u[k,n] - 8)."""
    K, N = 512, 8
    packed, s16 = synth.random_words(K, N, seed=6)
    u = o.unpack(packed).astype(np.int64) - 8
    group_sums = u.reshape(K // 128, 128, N).sum(axis=1)               # integers
    expect = (group_sums * s16.view(np.float16).astype(np.float64)).sum(axis=0)
    C = o.gemm_f64(np.ones((2, K), np.float16), packed, s16)
    assert np.allclose(C, np.broadcast_to(expect, (2, N)), rtol=1e-13, atol=0)


def check_gemm_w16_reference(o):
    """The fp16-rounded-weight reference equals numpy's matmul of W16."""
    rng = np.random.default_rng(12)
    packed, s16 = synth.random_words(256, 16, seed=12)
    A = rng.standard_normal((3, 256)).astype(np.float16)
    W16 = o.dequant(packed, s16)
    C = o.gemm_w16_f64(A, W16)
    ref = np.matmul(A.astype(np.float64), W16.view(np.float16).astype(np.float64))
    assert np.allclose(C, ref, rtol=1e-12, atol=1e-12)


def check_gemm_bf16_bruteforce(o):
    """bf16 activations on tiny shapes: numpy's float64 matmul of the bf16
    activations and torch's bf16 rounding of the exact weights."""
    rng = np.random.default_rng(15)
    for M, K, N in ((1, 128, 8), (3, 256, 16)):
        packed, s16 = synth.random_words(K, N, seed=M * 7 + K + N)
        Ab = _torch_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        C = o.gemm_bf16_f64(Ab, packed, s16)
        A = (Ab.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        Wb = _torch_bf16_bits(_exact_weights(o, packed, s16))
        W = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.allclose(C, np.matmul(A, W), rtol=1e-12, atol=1e-12)


def check_gemm_bf16_matches_fp16_when_exact(o):
    """Ternary activations and power-of-two scales are exact in both formats,
    so the bf16 product equals the fp16 product bit for bit."""
    K, N = 512, 16
    W = synth.grid_weights(K, N, p=4, seed=9)
    packed, s16 = o.quantize_pack(W)
    A = synth.ternary_activations(3, K, density=0.8, seed=9)     # fp16 values
    Ab = _torch_bf16_bits(A.astype(np.float64))
    assert np.array_equal(o.bf16_to_f64(Ab), A.astype(np.float64))
    assert np.array_equal(o.gemm_bf16_f64(Ab, packed, s16), o.gemm_f64(A, packed, s16))


# -- folded RMSNorm gain -------------------------------------------------------------

def check_fold_gain(o):
    """gamma = 1 leaves W; power-of-two gains scale exactly; any gain equals
    numpy's float32 multiply (IEEE, one rounding)."""
    rng = np.random.default_rng(21)
    W = rng.standard_normal((256, 24)).astype(np.float32)
    assert np.array_equal(o.fold_gain(W, np.ones(256, np.float32)), W)
    g2 = np.exp2(rng.integers(-3, 4, 256)).astype(np.float32)
    assert np.array_equal(o.fold_gain(W, g2), W * g2[:, None].astype(np.float64))
    g = (rng.random(256) * 2).astype(np.float32)
    assert np.array_equal(o.fold_gain(W, g), g[:, None] * W)


def check_rms_rowscale(o):
    """Constant rows give (c^2 + eps)^(-1/2); random fp16 and bf16 rows agree
    with numpy's mean of squares; eps enters once."""
    K = 512
    c = np.array([0.5, 2.0, -3.0], np.float16)
    A = np.repeat(c[:, None], K, axis=1)
    rho = o.rms_rowscale_f64(A, 1e-5)
    assert np.allclose(rho, 1.0 / np.sqrt(c.astype(np.float64) ** 2 + 1e-5), rtol=1e-15)
    rng = np.random.default_rng(22)
    A = rng.standard_normal((4, K)).astype(np.float16)
    x = A.astype(np.float64)
    assert np.allclose(o.rms_rowscale_f64(A, 1e-6), 1.0 / np.sqrt(np.mean(x * x, axis=1) + 1e-6),
                       rtol=1e-14)
    Ab = _torch_bf16_bits(rng.standard_normal((3, K)).astype(np.float32))
    xb = (Ab.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.allclose(o.rms_rowscale_f64(Ab, 0.0, bf16=True),
                       1.0 / np.sqrt(np.mean(xb * xb, axis=1)), rtol=1e-14)
    assert o.rms_rowscale_f64(np.zeros((1, K), np.float16), 0.25)[0] == 2.0


def check_scale_rows(o):
    """Row m is multiplied by rho[m] (and only by it)."""
    rng = np.random.default_rng(23)
    C = rng.standard_normal((3, 5))
    rho = np.array([2.0, 0.5, -1.0])
    assert np.array_equal(o.scale_rows(C, rho), C * rho[:, None])
    assert np.array_equal(o.scale_rows(C, np.ones(3)), C)


# -- SwiGLU ----------------------------------------------------------------------

def check_swiglu(o):
    """Z = g * expit(g) * up (scipy's logistic); silu(0) = 0; silu(x) -> x."""
    rng = np.random.default_rng(13)
    C = rng.standard_normal((3, 16)) * 4
    C[0, 0] = 0.0
    C[1, 1] = 40.0
    C[2, 2] = -40.0
    Z = o.swiglu_f64(C)
    ref = C[:, :8] * special.expit(C[:, :8]) * C[:, 8:]
    assert np.allclose(Z, ref, rtol=1e-14, atol=1e-300)
    assert Z[0, 0] == 0.0
    assert abs(Z[1, 1] / (40.0 * C[1, 9]) - 1) < 1e-15
    assert abs(Z[2, 2]) < 1e-15


# Checks cheap enough to run on every mutant of the oracle.
FAST_CHECKS = [
    check_f16_decode, check_f16_encode, check_pack_worked_words, check_pack_roundtrip,
    check_unpack_sign_words, check_quantize_group_max, check_quantize_grid_roundtrip,
    check_quantize_ties_to_even, check_quantize_scale_value, check_quantize_zero_group,
    check_quantization_error_closed_form, check_dequant_special_values,
    check_dequant_rounds_once, check_gemm_bruteforce, check_gemm_onehot,
    check_gemm_integer_exact, check_gemm_all_ones, check_gemm_w16_reference, check_swiglu,
    check_bf16_decode, check_bf16_encode, check_dequant_bf16_rounds_once,
    check_gemm_bf16_bruteforce, check_gemm_bf16_matches_fp16_when_exact,
    check_fold_gain, check_rms_rowscale, check_scale_rows, check_quantize_other_group_sizes,
    check_zero_rows, check_dequant_zp_worked_examples, check_dequant_zp_reduces_to_symmetric,
    check_dequant_zp_power_of_two_exact, check_dequant_zp_error_bound, check_gemm_wb_reference,
    check_pack8_worked_words, check_pack8_roundtrip, check_quantize8_grid_roundtrip,
    check_quantize8_group_max_and_zero_group, check_quantize8_ties_to_even,
    check_quantize8_error_bound, check_dequant8_values, check_gemm8_bruteforce_and_exact,
]
