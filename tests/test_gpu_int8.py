"""GPU parity for INT8 weights (W8A16): 8-bit codes offset by 128, four per
int32 along K, one fp16 scale per group (Swordfish page, blog.alpindale.net,
section "The packed format"; "Making a Single GPU Go Fast", arunshar.com,
section 9.3.2), against the oracle on the same seeded inputs: the packer, the
repacked layout, the dequantization and the GEMM on the decode path and the
dense tier."""
import numpy as np
import pytest

import parity
from gpuhelp import bf16_dev, bf16_out, fp16_out, orc, sample_indices, say, to_dev, torch
from weight_only_int4_03_amd import synth, w4a16

pytestmark = pytest.mark.gpu


def gemm8_case(M, K, N, G=128, swiglu=False, path="auto", bf16=False, seed=0, rows=None,
               cols=None, W=None, rowscale=False):
    say("int8 case M=%d K=%d N=%d G=%d swiglu=%s bf16=%s path=%s seed=%d" %
        (M, K, N, G, swiglu, bf16, path, seed))
    if W is None:
        W = synth.weights(K, N, seed)
    w = w4a16.load_weight_int8(W, G=G)
    rho = rho_d = None
    if rowscale:
        rho = (0.25 + 1.5 * np.random.default_rng(seed).random(M)).astype(np.float32)
        rho_d = torch().from_numpy(rho).cuda()
    if bf16:
        A = synth.activations_bf16(M, K, seed=seed)
        out = bf16_out(w4a16.gemm(bf16_dev(A), w, swiglu=swiglu, path=path, rowscale=rho_d))
    else:
        A = synth.activations(M, K, seed=seed)
        out = fp16_out(w4a16.gemm(to_dev(A), w, swiglu=swiglu, path=path, rowscale=rho_d))
    torch().cuda.synchronize()
    ncols = N // 2 if swiglu else N
    ocols = np.arange(ncols) if cols is None else np.asarray(cols)
    orows = np.arange(M) if rows is None else np.asarray(rows)
    wcols = np.concatenate([ocols, ocols + N // 2]) if swiglu else ocols
    o = orc()
    packed, s16 = o.quantize_pack8(np.ascontiguousarray(W[:, wcols]), G)
    C = o.gemm8_f64(np.ascontiguousarray(A[orows]), packed, s16, G, bf16=bf16)
    if rowscale:
        C = o.scale_rows(C, rho[orows].astype(np.float64))
    ref = o.swiglu_f64(C) if swiglu else C
    got = out[np.ix_(orows, ocols)]
    what = "int8 M=%d K=%d N=%d G=%d path=%s" % (M, K, N, G, path)
    stats = parity.assert_close_bf16(got, ref, what) if bf16 else parity.assert_close(got, ref, what)
    say("  ", {k: (round(v, 6) if isinstance(v, float) else v) for k, v in stats.items()})
    return stats


@pytest.mark.parametrize("K,N,G", [(128, 8, 128), (4096, 1064, 128), (2048, 72, 32),
                                   (1152, 1088, 1152), (11008, 264, 64)])
def test_pack_int8_bit_exact(K, N, G):
    """The GPU quantizer's codes and scales equal the oracle's (ties, zero
    groups and the group maximum included)."""
    W = synth.weights(K, N, seed=K + N)
    W[:, 3] = 0.0
    if K >= 256:
        W[:128, 5] = 0.0
        W[7, 5] = 127 * 2.0 ** -7
        W[8:13, 5] = np.array([0.5, 1.5, 2.5, -0.5, -3.5]) * 2.0 ** -7
    packed, scales = w4a16.pack_int8(to_dev(W), G)
    po, so = orc().quantize_pack8(W, G)
    assert np.array_equal(packed.cpu().numpy(), po)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), so)


@pytest.mark.parametrize("K,N,G", [(1024, 1064, 128), (2048, 72, 32), (1152, 40, 1152)])
def test_repack_int8_roundtrip(K, N, G):
    """Repack then unrepack returns the canonical words and scales bit for bit
    (arbitrary codes, ragged N)."""
    packed, s16 = synth.random_bytes(K, N, seed=K + G, group=G)
    w = w4a16.repack_int8(to_dev(packed), to_dev(s16.view(np.int16)), G)
    p2, s2 = w4a16.unrepack(w)
    assert np.array_equal(p2.cpu().numpy(), packed)
    assert np.array_equal(s2.cpu().numpy().view(np.uint16), s16)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("K,N,G", [(1024, 1064, 128), (2048, 136, 32), (2048, 1088, 2048)])
def test_dequant_int8_bit_exact(K, N, G, bf16):
    """round((q - 128) s) in fp16 and bf16, bit for bit, every code 0..255."""
    packed, s16 = synth.random_bytes(K, N, seed=K + N + bf16, group=G)
    w = w4a16.repack_int8(to_dev(packed), to_dev(s16.view(np.int16)), G)
    got = w4a16.dequant(w, bf16=bf16).view(torch().int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, orc().dequant8(packed, s16, G, bf16=bf16))


@pytest.mark.parametrize("path", ["decode", "prefill", "dense", "auto"])
@pytest.mark.parametrize("M,K,N,G,swiglu,bf16", [(1, 4096, 1064, 128, False, False),
                                                 (5, 4096, 2112, 128, True, False),
                                                 (16, 2048, 1088, 64, False, True),
                                                 (32, 1024, 2112, 32, True, True),
                                                 (20, 2048, 1088, 2048, False, False),
                                                 (3, 14336, 1024, 128, False, False),
                                                 (70, 2048, 2112, 128, True, False),
                                                 (300, 1024, 4160, 128, False, True)])
def test_int8_each_path(path, M, K, N, G, swiglu, bf16):
    """The decode and prefill kernels' 8-bit instances and the dense tier,
    fp16 and bf16, several group sizes (channelwise included), SwiGLU, ragged
    M and N."""
    gemm8_case(M, K, N, G=G, swiglu=swiglu, path=path, bf16=bf16, seed=M + N + G)


@pytest.mark.parametrize("half,ks", [(1, 1), (1, 2), (0, 1), (0, 3)])
def test_int8_decode_configs(monkeypatch, half, ks):
    """Half-strip and whole-strip workgroups, with and without split K."""
    monkeypatch.setenv("W4A16_DECODE_HALF", str(half))
    monkeypatch.setenv("W4A16_DECODE_KS", str(ks))
    d = w4a16.describe(8, 4096, 2048, path="decode", int8=True)
    assert d.split(">")[0].endswith("%s, 8" % ("true" if half else "false")) and "ks=%d" % ks in d, d
    gemm8_case(8, 4096, 2048, path="decode", seed=half + ks)
    gemm8_case(1, 2048, 1088, path="decode", seed=7 + ks, bf16=True)


@pytest.mark.parametrize("path", ["decode", "prefill", "dense"])
@pytest.mark.parametrize("bf16", [False, True])
def test_int8_onehot_rows_bit_exact(path, bf16):
    """One-hot activation rows return rows of the dequantized weights exactly."""
    K, N = 2048, 1088
    packed, s16 = synth.random_bytes(K, N, seed=11 + bf16)
    w = w4a16.repack_int8(to_dev(packed), to_dev(s16.view(np.int16)))
    Wo = orc().dequant8(packed, s16, bf16=bf16)
    for M in (3, 17 if path == "decode" else 40):
        A, ks = synth.onehot_activations(M, K, seed=M)
        if bf16:
            Ab = np.zeros((M, K), np.uint16)
            Ab[np.arange(M), ks] = 0x3F80
            got = bf16_out(w4a16.gemm(bf16_dev(Ab), w, path=path))
        else:
            got = fp16_out(w4a16.gemm(to_dev(A), w, path=path)).view(np.uint16)
        for m, k in enumerate(ks):
            same = (got[m] == Wo[k]) | (((got[m] | Wo[k]) & 0x7FFF) == 0)
            assert same.all(), (path, bf16, M, m, k)


@pytest.mark.parametrize("path", ["decode", "prefill", "dense"])
def test_int8_integer_exact_inputs(path):
    """Grid weights (lossless 8-bit codes, power-of-two scales) and sparse
    ternary activations: exact sums, the correctly rounded fp16 output."""
    o = orc()
    for M, K, N in [(4, 2048, 1088), (24, 4096, 2048)]:
        W = synth.grid_weights8(K, N, p=10, seed=M)
        A = synth.ternary_activations(M, K, density=0.25, seed=M)
        w = w4a16.load_weight_int8(W)
        out = fp16_out(w4a16.gemm(to_dev(A), w, path=path)).view(np.uint16)
        packed, s16 = o.quantize_pack8(W)
        assert np.array_equal(out, o.f64_to_f16(o.gemm8_f64(A, packed, s16))), (path, M)


def test_int8_with_rowscale():
    """INT8 weights with the RMSNorm row factor, decode, prefill and dense."""
    gemm8_case(9, 2048, 2112, swiglu=True, path="decode", seed=9, rowscale=True)
    gemm8_case(70, 2048, 1088, path="dense", seed=70, rowscale=True, bf16=True)
    gemm8_case(300, 2048, 2112, swiglu=True, path="prefill", seed=300, rowscale=True)


@pytest.mark.parametrize("wm", [2, 1])
@pytest.mark.parametrize("bm,tps,ks", [(64, 1, 1), (128, 2, 4), (256, 2, 1), (64, 2, 3)])
def test_int8_prefill_tiles(monkeypatch, wm, bm, tps, ks):
    """The fused kernel's 8-bit instances at each row tile, wave layout,
    pipeline step and K split."""
    if wm == 1 and bm == 256:
        pytest.skip("the 256-row tile keeps two waves along the rows")
    monkeypatch.setenv("W4A16_PREFILL_BM", str(bm))
    monkeypatch.setenv("W4A16_PREFILL_TPS", str(tps))
    monkeypatch.setenv("W4A16_PREFILL_KS", str(ks))
    monkeypatch.setenv("W4A16_PREFILL_WM", str(wm))
    d = w4a16.describe(200, 4096, 2112, swiglu=True, path="prefill", int8=True)
    assert d.startswith("prefill2_kernel<%d, %d, %d, %d" % (bm // (32 * wm), wm, 8 // wm, tps)), d
    assert d.split(">")[0].endswith(", 8") and ("ks=%d" % ks) in d, d
    gemm8_case(200, 4096, 2112, swiglu=True, path="prefill", seed=bm + ks + wm)


@pytest.mark.parametrize("M,K,N,swiglu", [(1, 4096, 28672, True), (16, 14336, 4096, False),
                                          (4096, 4096, 6144, False), (8191, 14336, 4096, False)])
def test_int8_full_size_sampled(M, K, N, swiglu):
    """Llama-3.1-8B projection sizes on the automatic path (decode, and the
    fused prefill kernel for 4096- and 8191-token prefills), checked on
    sampled rows and columns."""
    ncols = N // 2 if swiglu else N
    rows = sample_indices(M, 24, seed=M, edge=2) if M > 64 else None
    cols = sample_indices(ncols, 96, seed=N, edge=2)
    gemm8_case(M, K, N, swiglu=swiglu, seed=M + K, rows=rows, cols=cols)


@pytest.mark.parametrize("wm,ks", [(1, 3), (2, 2)])
def test_int8_prefill_split_bit_exact_integer_inputs(monkeypatch, wm, ks):
    """Split K with uneven slices on exact sums: the FP32 partials add up to
    the same integer multiple of 2^-10 in any order, so the fp16 output is the
    correctly rounded exact product."""
    monkeypatch.setenv("W4A16_PREFILL_BM", "64")
    monkeypatch.setenv("W4A16_PREFILL_KS", str(ks))
    monkeypatch.setenv("W4A16_PREFILL_WM", str(wm))
    o = orc()
    M, K, N = 130, 4608, 1088
    W = synth.grid_weights8(K, N, p=10, seed=ks)
    A = synth.ternary_activations(M, K, density=0.25, seed=ks)
    w = w4a16.load_weight_int8(W)
    d = w4a16.describe(M, K, N, path="prefill", int8=True)
    assert ("ks=%d" % ks) in d and d.split(">")[0].endswith(", 8"), d
    out = fp16_out(w4a16.gemm(to_dev(A), w, path="prefill")).view(np.uint16)
    packed, s16 = o.quantize_pack8(W)
    assert np.array_equal(out, o.f64_to_f16(o.gemm8_f64(A, packed, s16)))


@pytest.mark.parametrize("wc,wk,ks", [(1, 4, 1), (2, 4, 2), (4, 2, 1), (2, 2, 4), (4, 2, 4), (8, 1, 3),
                                      (1, 8, 1), (1, 8, 2)])
@pytest.mark.parametrize("M", [1, 7, 16, 24, 32])
@pytest.mark.parametrize("bf16", [False, True])
def test_int8_cooperative_decode(monkeypatch, wc, wk, ks, M, bf16):
    """The cooperative decode kernel's 8-bit instances (two 16-byte vectors
    per lane and unit) in several configurations, with K splits that leave
    partial rounds and gate/up with an odd number of strips (N = 2112)."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    monkeypatch.setenv("W4A16_COOP_WC", str(wc))
    monkeypatch.setenv("W4A16_COOP_WK", str(wk))
    monkeypatch.setenv("W4A16_COOP_KS", str(ks))
    swiglu = (wc + M) % 2 == 1
    K, N = (1152, 2112) if swiglu else (2560, 1064)
    d = w4a16.describe(M, K, N, swiglu, path="decode", bf16=bf16, int8=True)
    # At M > 16 some configurations need more LDS than a workgroup has, and
    # one column group with eight waves along K exists for plain projections
    # only: those fall back to the per-wave kernel.
    if M <= 16 and not (swiglu and (wc, wk) == (1, 8)):
        assert d.startswith("decode_coop_kernel") and d.split(">")[0].endswith(", 8"), d
    gemm8_case(M, K, N, swiglu=swiglu, path="decode", bf16=bf16, seed=wc * 100 + wk * 10 + ks + M)


def test_int8_cooperative_integer_exact(monkeypatch):
    """Grid weights and sparse ternary activations through the cooperative
    8-bit instances with K splits: the correctly rounded exact product."""
    o = orc()
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    K, N = 4096, 2048
    for (wc, wk, ks), M in [((2, 4, 2), 1), ((1, 4, 1), 16), ((4, 2, 4), 32)]:
        monkeypatch.setenv("W4A16_COOP_WC", str(wc))
        monkeypatch.setenv("W4A16_COOP_WK", str(wk))
        monkeypatch.setenv("W4A16_COOP_KS", str(ks))
        assert w4a16.describe(M, K, N, path="decode", int8=True).startswith("decode_coop_kernel")
        W = synth.grid_weights8(K, N, p=10, seed=M)
        A = synth.ternary_activations(M, K, density=0.25, seed=M)
        w = w4a16.load_weight_int8(W)
        out = fp16_out(w4a16.gemm(to_dev(A), w, path="decode")).view(np.uint16)
        packed, s16 = o.quantize_pack8(W)
        assert np.array_equal(out, o.f64_to_f16(o.gemm8_f64(A, packed, s16))), (wc, wk, ks, M)
