"""GPU parity for asymmetric (AWQ) weights with zero points: the prescaled
zero rows fp16((8 - zp) s) (Swordfish page, blog.alpindale.net, section "The
packed format"), the dequantization round((q - 8) s + z), and the GEMM on every
path against the oracle on the same seeded inputs."""
import numpy as np
import pytest

import parity
from gpuhelp import bf16_dev, bf16_out, fp16_out, orc, sample_indices, say, to_dev, torch
from weight_only_int4_03_amd import synth, w4a16

pytestmark = pytest.mark.gpu

PATHS = ["decode", "prefill", "dense"]


def zp_inputs(K, N, G, seed):
    """Seeded nibbles, scales and zero points (host) and the device weight."""
    packed, s16 = synth.random_words(K, N, seed=seed, group=G)
    zp = synth.zero_points(K // G, N, seed=seed)
    sd = to_dev(s16.view(np.int16))
    w = w4a16.zero_rows(w4a16.repack(to_dev(packed), sd, G), sd, to_dev(zp))
    return w, packed, s16, zp


def oracle_weights(packed, s16, zp, G, bf16, cols=None):
    o = orc()
    if cols is not None:
        packed, s16, zp = (np.ascontiguousarray(x[:, cols]) for x in (packed, s16, zp))
    return o.dequant_zp(packed, s16, o.zero_rows(s16, zp), G, bf16=bf16)


def zp_case(M, K, N, G=128, swiglu=False, path="auto", bf16=False, seed=0, rows=None,
            cols=None, rowscale=False):
    say("zp case M=%d K=%d N=%d G=%d swiglu=%s bf16=%s path=%s rowscale=%s seed=%d" %
        (M, K, N, G, swiglu, bf16, path, rowscale, seed))
    w, packed, s16, zp = zp_inputs(K, N, G, seed)
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
    Wo = oracle_weights(packed, s16, zp, G, bf16, wcols)
    Ao = np.ascontiguousarray(A[orows])
    C = o.gemm_wb_f64(Ao, Wo) if bf16 else o.gemm_w16_f64(Ao, Wo)
    if rowscale:
        C = o.scale_rows(C, rho[orows].astype(np.float64))
    ref = o.swiglu_f64(C) if swiglu else C
    got = out[np.ix_(orows, ocols)]
    what = "zp M=%d K=%d N=%d G=%d path=%s" % (M, K, N, G, path)
    stats = parity.assert_close_bf16(got, ref, what) if bf16 else parity.assert_close(got, ref, what)
    say("  ", {k: (round(v, 6) if isinstance(v, float) else v) for k, v in stats.items()})
    return stats


@pytest.mark.parametrize("G,K,N", [(32, 1024, 1064), (128, 2048, 1088), (1152, 1152, 72)])
def test_zero_rows_bit_exact(G, K, N):
    """The device's zero rows, read back in canonical order through the
    repack inverse, equal the oracle's fp16((8 - zp) s) bit for bit (N not a
    multiple of 32: padded columns)."""
    w, packed, s16, zp = zp_inputs(K, N, G, seed=G + N)
    _, z_dev = w4a16.unrepack(w4a16.RepackedWeight(w.rw, w.rz, K, N, G))
    assert np.array_equal(z_dev.cpu().numpy().view(np.uint16), orc().zero_rows(s16, zp))


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("G,K,N", [(32, 1024, 1064), (128, 2048, 1088), (2048, 2048, 136)])
def test_dequant_zp_bit_exact(G, K, N, bf16):
    """round((q - 8) s + z) in fp16 and bf16, bit for bit."""
    w, packed, s16, zp = zp_inputs(K, N, G, seed=G + K + bf16)
    W = w4a16.dequant(w, bf16=bf16)
    got = W.view(torch().int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle_weights(packed, s16, zp, G, bf16))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,K,N,G,swiglu,bf16", [(1, 2048, 1064, 128, False, False),
                                                 (5, 4096, 2112, 128, True, False),
                                                 (16, 2048, 1088, 64, False, True),
                                                 (32, 1024, 2112, 32, True, True),
                                                 (20, 2048, 1088, 2048, False, False),
                                                 (70, 2048, 2112, 128, True, False),
                                                 (130, 1152, 1088, 1152, False, True),
                                                 (300, 2048, 4160, 128, False, False),
                                                 (257, 1024, 2112, 32, True, True)])
def test_zp_each_path(path, M, K, N, G, swiglu, bf16):
    """Every path, fp16 and bf16, several group sizes (channelwise included),
    SwiGLU, ragged M and N."""
    zp_case(M, K, N, G=G, swiglu=swiglu, path=path, bf16=bf16, seed=M + N + G)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("bf16", [False, True])
def test_zp_onehot_rows_bit_exact(path, bf16):
    """One-hot activation rows select rows of the dequantized weights
    exactly: the product is bit-equal to the oracle's weights."""
    K, N, G = 2048, 1088, 64
    w, packed, s16, zp = zp_inputs(K, N, G, seed=7 + bf16)
    Wo = oracle_weights(packed, s16, zp, G, bf16)
    for M in (3, 40):
        A, ks = synth.onehot_activations(M, K, seed=M)
        if bf16:
            Ab = np.zeros((M, K), np.uint16)
            Ab[np.arange(M), ks] = 0x3F80                    # bf16 1.0
            out = bf16_out(w4a16.gemm(bf16_dev(Ab), w, path=path))
        else:
            out = fp16_out(w4a16.gemm(to_dev(A), w, path=path)).view(np.uint16)
        got = out.view(np.uint16)
        for m, k in enumerate(ks):
            want = Wo[k]
            same = (got[m] == want) | (((got[m] | want) & 0x7FFF) == 0)  # +0 == -0
            assert same.all(), (path, bf16, M, m, k)


@pytest.mark.parametrize("path", PATHS)
def test_zp_integer_exact_inputs(path):
    """Power-of-two scales make every weight (q - zp) s exact; sparse ternary
    activations keep every partial sum exact in FP32, so the fp16 output is
    the correctly rounded exact product, bit for bit, on every path."""
    o = orc()
    for M, K, N, G in [(4, 2048, 1088, 128), (90, 1024, 2048, 32)]:
        rng = np.random.default_rng(M)
        packed, _ = synth.random_words(K, N, seed=M, group=G)
        s16 = np.exp2(rng.integers(-6, -3, (K // G, N))).astype(np.float16).view(np.uint16)
        zp = synth.zero_points(K // G, N, seed=M)
        sd = to_dev(s16.view(np.int16))
        w = w4a16.zero_rows(w4a16.repack(to_dev(packed), sd, G), sd, to_dev(zp))
        A = synth.ternary_activations(M, K, density=0.1, seed=M)
        out = fp16_out(w4a16.gemm(to_dev(A), w, path=path)).view(np.uint16)
        C = o.gemm_w16_f64(A, o.dequant_zp(packed, s16, o.zero_rows(s16, zp), G))
        assert np.array_equal(out, o.f64_to_f16(C)), (path, M)


@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("bf16", [False, True])
def test_zp_with_rowscale(path, bf16):
    """Zero points and the RMSNorm row factor together (w4a16_gemm_zp with
    rowscale), with the SwiGLU epilogue."""
    M = 9 if path == "decode" else 140
    zp_case(M, 2048, 2112, swiglu=True, path=path, bf16=bf16, seed=M, rowscale=True)


@pytest.mark.parametrize("bm,tps,ks", [(64, 1, 1), (128, 2, 4), (256, 2, 1), (64, 2, 8),
                                       (256, 1, 2)])
def test_zp_prefill_tiles_and_k_slices(monkeypatch, bm, tps, ks):
    """The zero-point prefill instances at each row tile, pipeline depth and
    K split."""
    monkeypatch.setenv("W4A16_PREFILL_BM", str(bm))
    monkeypatch.setenv("W4A16_PREFILL_TPS", str(tps))
    monkeypatch.setenv("W4A16_PREFILL_KS", str(ks))
    d = w4a16.describe(200, 4096, 2112, swiglu=True, path="prefill", zp=True)
    assert "prefill2_kernel<%d, 2, 4, %d, false, true, false, true, 4>" % (bm // 64, tps) in d, d
    zp_case(200, 4096, 2112, swiglu=True, path="prefill", seed=bm + ks)


def test_zp_prefill_one_wave_kernel(monkeypatch):
    """The one-wave mainloop reads the zero rows at run time."""
    monkeypatch.setenv("W4A16_PREFILL_V2", "0")
    assert w4a16.describe(130, 1152, 2112, path="prefill", zp=True).startswith("prefill_kernel<")
    zp_case(130, 1152, 2112, swiglu=True, path="prefill", seed=3)
    zp_case(40, 1024, 1088, path="prefill", bf16=True, seed=4)


@pytest.mark.parametrize("M,K,N,swiglu", [(1, 4096, 28672, True), (16, 14336, 4096, False),
                                          (4096, 4096, 6144, False)])
def test_zp_full_size_sampled(M, K, N, swiglu):
    """Llama-3.1-8B projection sizes (gate/up with SwiGLU, down, and a
    4096-token prefill of the QKV projection) on the automatic path, checked on
    sampled rows and columns (the oracle computes those one by one)."""
    ncols = N // 2 if swiglu else N
    rows = sample_indices(M, 24, seed=M, edge=2) if M > 64 else None
    cols = sample_indices(ncols, 96, seed=N, edge=2)
    zp_case(M, K, N, swiglu=swiglu, seed=M + K, rows=rows, cols=cols)


@pytest.mark.parametrize("wc,wk,ks", [(1, 4, 1), (2, 4, 2), (4, 2, 1), (2, 2, 4), (4, 2, 4), (8, 1, 3),
                                      (1, 8, 1), (1, 8, 2)])
@pytest.mark.parametrize("M", [1, 7, 16, 24, 32])
@pytest.mark.parametrize("bf16", [False, True])
def test_zp_cooperative_decode(monkeypatch, wc, wk, ks, M, bf16):
    """The cooperative decode kernel's zero-row instances (zero rows staged in
    LDS beside the scales) in several configurations, with K splits that leave
    partial rounds, gate/up with an odd number of strips (N = 2112)."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    monkeypatch.setenv("W4A16_COOP_WC", str(wc))
    monkeypatch.setenv("W4A16_COOP_WK", str(wk))
    monkeypatch.setenv("W4A16_COOP_KS", str(ks))
    swiglu = (wc + M) % 2 == 1
    K, N = (1152, 2112) if swiglu else (2560, 1064)
    d = w4a16.describe(M, K, N, swiglu, path="decode", bf16=bf16, zp=True)
    # At M > 16 some configurations need more LDS than a workgroup has, and
    # one column group with eight waves along K exists for plain projections
    # only: those fall back to the per-wave kernel.
    if M <= 16 and not (swiglu and (wc, wk) == (1, 8)):
        assert d.startswith("decode_coop_kernel") and d.split(">")[0].endswith(", true, 4"), d
    zp_case(M, K, N, swiglu=swiglu, path="decode", bf16=bf16, seed=wc * 100 + wk * 10 + ks + M)


def test_zp_cooperative_integer_exact(monkeypatch):
    """Integer-exact inputs through the cooperative zero-row instances with a
    K split: the correctly rounded exact product, bit for bit."""
    o = orc()
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    for (wc, wk, ks), M in [((2, 4, 2), 1), ((2, 4, 2), 16), ((4, 2, 4), 32)]:
        monkeypatch.setenv("W4A16_COOP_WC", str(wc))
        monkeypatch.setenv("W4A16_COOP_WK", str(wk))
        monkeypatch.setenv("W4A16_COOP_KS", str(ks))
        K, N, G = 4096, 2048, 128
        rng = np.random.default_rng(M)
        packed, _ = synth.random_words(K, N, seed=M, group=G)
        s16 = np.exp2(rng.integers(-6, -3, (K // G, N))).astype(np.float16).view(np.uint16)
        zp = synth.zero_points(K // G, N, seed=M)
        sd = to_dev(s16.view(np.int16))
        w = w4a16.zero_rows(w4a16.repack(to_dev(packed), sd, G), sd, to_dev(zp))
        A = synth.ternary_activations(M, K, density=0.1, seed=M)
        assert w4a16.describe(M, K, N, path="decode", zp=True).startswith("decode_coop_kernel")
        out = fp16_out(w4a16.gemm(to_dev(A), w, path="decode")).view(np.uint16)
        C = o.gemm_w16_f64(A, o.dequant_zp(packed, s16, o.zero_rows(s16, zp), G))
        assert np.array_equal(out, o.f64_to_f16(C)), (wc, wk, ks, M)
