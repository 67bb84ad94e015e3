"""GPU parity of the transition-regime kernel (skinny row tiles whose waves
split K inside the workgroup) against the oracle on the same seeded inputs:
ragged row counts and column tails, both tile heights, split and unsplit K
(uneven slices, partial last rounds), the SwiGLU epilogue, bf16 activations,
zero points, INT8 weights, other group sizes and the row factor, the Stream-K
form and the four-wave workgroups (two per CU, also at full size on the
automatic path); one-hot and integer-exact inputs bit for bit."""
import numpy as np
import pytest

import parity
from gpuhelp import fp16_out, gemm_case, orc, sample_indices, say, to_dev
from test_gpu_int8 import gemm8_case
from test_gpu_zero_points import zp_case
from weight_only_int4_03_amd import synth, w4a16

pytestmark = pytest.mark.gpu


def _kernel(M, K, N, swiglu=False, **kw):
    d = w4a16.describe(M, K, N, swiglu=swiglu, path="prefill", **kw)
    assert d.startswith(("transition_kernel<", "transition_sk_kernel<")), d
    return d


@pytest.mark.parametrize("M", [33, 50, 64, 65, 100, 128, 129, 200, 256])
@pytest.mark.parametrize("N", [1088, 1064])
def test_transition_ragged_auto(M, N):
    """M = 33 .. 256 take the transition kernel on the automatic path; N = 1064
    leaves an 8-column tail strip (and an odd strip count: a half-empty strip
    pair), K = 1152 nine groups (a partial last round)."""
    d = _kernel(M, 1152, N)
    say(d)
    gemm_case(M, 1152, N, seed=M + N)


@pytest.mark.parametrize("mi", [2, 4])
@pytest.mark.parametrize("ks", [1, 2, 3, 5])
@pytest.mark.parametrize("M,K,N,swiglu", [(70, 2048, 2112, True), (130, 3072, 1064, False)])
def test_transition_tiles_and_slices(monkeypatch, mi, ks, M, K, N, swiglu):
    """Both tile heights (64 rows with four waves along K, 128 rows with two)
    and forced K slices, including uneven slices and slices shorter than a
    round; N = 2112 with SwiGLU gives 33 gate strips."""
    monkeypatch.setenv("W4A16_TRANSITION_MI", str(mi))
    monkeypatch.setenv("W4A16_TRANSITION_KS", str(ks))
    d = _kernel(M, K, N, swiglu)
    assert d.startswith("transition_kernel<%d, " % mi) and ("ks=%d" % ks) in d, d
    gemm_case(M, K, N, swiglu=swiglu, path="prefill", seed=M + K + ks)


@pytest.mark.parametrize("M", [1, 17, 32, 300])
def test_transition_forced_outside_its_range(monkeypatch, M):
    """Forced on, the kernel also takes row counts outside its default range
    (one row, a partial single tile, several 128-row tiles)."""
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    _kernel(M, 1024, 1088)
    gemm_case(M, 1024, 1088, path="prefill", seed=M)


@pytest.mark.parametrize("mi", [2, 4])
@pytest.mark.parametrize("M", [64, 130])
def test_transition_onehot_rows_bit_exact(monkeypatch, mi, M):
    """One-hot activation rows return dequantized weight rows bit for bit
    (every nibble value; pins the staged activation swizzle and the weight
    layout)."""
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    monkeypatch.setenv("W4A16_TRANSITION_MI", str(mi))
    K, N = 2048, 1056
    packed, scales = synth.random_words(K, N, seed=M + mi)
    w = w4a16.repack(to_dev(packed), to_dev(scales.view(np.int16)))
    A, ks = synth.onehot_activations(M, K, seed=M)
    _kernel(M, K, N)
    out = fp16_out(w4a16.gemm(to_dev(A), w, path="prefill"))
    want = orc().dequant(packed, scales)[ks].view(np.float16).astype(np.float64)
    assert np.array_equal(out.astype(np.float64), want)


@pytest.mark.parametrize("M,K,N,ks", [(256, 4096, 4096, 1), (64, 4096, 2048, 1),
                                      (128, 8192, 1024, 4), (96, 3072, 1088, 3)])
def test_transition_integer_exact(monkeypatch, M, K, N, ks):
    """Power-of-two scales and activations in {-1, 0, 1}: every partial sum is
    exact, so the output equals the oracle's bit for bit whatever the
    summation order, split K included."""
    monkeypatch.setenv("W4A16_TRANSITION_KS", str(ks))
    _kernel(M, K, N)
    W = synth.grid_weights(K, N, p=4, seed=M + K)
    A = synth.ternary_activations(M, K, density=0.5, seed=M)
    out = fp16_out(w4a16.gemm(to_dev(A), w4a16.load_weight(W)))
    packed_o, s16_o = orc().quantize_pack(W)
    C = orc().gemm_f64(A, packed_o, s16_o)
    assert np.abs(C).max() < 128, "inputs not fp16-exact"
    assert np.array_equal(out.astype(np.float64), C)


@pytest.mark.parametrize("M,swiglu", [(48, False), (100, True), (256, False)])
def test_transition_bf16(M, swiglu):
    _kernel(M, 2048, 2112, swiglu, bf16=True)
    gemm_case(M, 2048, 2112, swiglu=swiglu, seed=M, bf16=True)


@pytest.mark.parametrize("M,G,swiglu,bf16", [(64, 128, False, False), (100, 64, True, False),
                                             (200, 128, False, True), (40, 32, True, True)])
def test_transition_zero_points(M, G, swiglu, bf16):
    _kernel(M, 2048, 1088 if not swiglu else 2112, swiglu, zp=True, bf16=bf16)
    zp_case(M, 2048, 1088 if not swiglu else 2112, G=G, swiglu=swiglu, bf16=bf16, seed=M,
            rowscale=True)


@pytest.mark.parametrize("M,G,swiglu,bf16", [(64, 128, False, False), (100, 32, True, False),
                                             (256, 2048, False, True)])
def test_transition_int8(M, G, swiglu, bf16):
    _kernel(M, 2048, 2112, swiglu, int8=True)
    gemm8_case(M, 2048, 2112, G=G, swiglu=swiglu, bf16=bf16, seed=M, rowscale=True)


@pytest.mark.parametrize("G", [32, 64, 2048])
def test_transition_group_sizes(G):
    """Groups shorter than the 128-k round unit (scales per 64-k tile and lane
    half) and channelwise scales."""
    _kernel(100, 2048, 1088)
    gemm_case(100, 2048, 1088, seed=G, G=G)


SK_SHAPES = [(33, 1152, 1064, False), (64, 2048, 2112, True), (100, 3072, 1088, False),
             (200, 1152, 2112, True), (256, 1152, 8320, False)]


@pytest.mark.parametrize("mi", [2, 4])
@pytest.mark.parametrize("M,K,N,swiglu", SK_SHAPES)
def test_transition_stream_k(monkeypatch, mi, M, K, N, swiglu):
    """The Stream-K form: (tile, round) units dealt in equal runs to one
    workgroup per CU.  The shapes give tiles shared by up to four workgroups
    (their partial slices summed in order by the reduction kernel), tiles
    finished by the one workgroup that covers them (K = 1152 with 260 tiles),
    ragged rows and column tails, partial last rounds (nine groups) and the
    SwiGLU epilogue; two calls give the same bits."""
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    monkeypatch.setenv("W4A16_TRANSITION_SK", "1")
    monkeypatch.setenv("W4A16_TRANSITION_MI", str(mi))
    d = w4a16.describe(M, K, N, swiglu=swiglu, path="prefill")
    say(d)
    assert d.startswith("transition_sk_kernel<%d, " % mi) and "stream-k" in d, d
    W = synth.weights(K, N, seed=M + K)
    w = w4a16.load_weight(W)
    gemm_case(M, K, N, swiglu=swiglu, path="prefill", seed=M + N, W=W, weight=w)
    A = to_dev(synth.activations(M, K, seed=M + N))
    a = fp16_out(w4a16.gemm(A, w, swiglu=swiglu, path="prefill"))
    b = fp16_out(w4a16.gemm(A, w, swiglu=swiglu, path="prefill"))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("M,K,N", [(128, 4096, 2048), (64, 8192, 1024), (256, 1152, 8320)])
def test_transition_stream_k_integer_exact(monkeypatch, M, K, N):
    """Integer-exact inputs through the Stream-K form: the output equals the
    oracle's bit for bit, shared tiles included."""
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    monkeypatch.setenv("W4A16_TRANSITION_SK", "1")
    say(w4a16.describe(M, K, N, path="prefill"))
    W = synth.grid_weights(K, N, p=4, seed=M + K)
    A = synth.ternary_activations(M, K, density=0.5, seed=M)
    out = fp16_out(w4a16.gemm(to_dev(A), w4a16.load_weight(W), path="prefill"))
    packed_o, s16_o = orc().quantize_pack(W)
    C = orc().gemm_f64(A, packed_o, s16_o)
    assert np.abs(C).max() < 128, "inputs not fp16-exact"
    assert np.array_equal(out.astype(np.float64), C)


@pytest.mark.parametrize("M,swiglu,bf16", [(64, False, True), (200, True, True), (100, True, False)])
def test_transition_stream_k_bf16_rowscale(monkeypatch, M, swiglu, bf16):
    """bf16 activations and the row factor through the Stream-K form (the
    factor applied in the reduction kernel for shared tiles)."""
    from test_gpu_gemm import test_gemm_rowscale_each_path as rowscale_case
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    monkeypatch.setenv("W4A16_TRANSITION_SK", "1")
    assert w4a16.describe(M, 2048, 2112, swiglu=swiglu, path="prefill",
                          bf16=bf16).startswith("transition_sk_kernel<")
    gemm_case(M, 2048, 2112, swiglu=swiglu, path="prefill", seed=M, bf16=bf16)
    rowscale_case("prefill", M, 2048, 2112, swiglu, bf16)


def _random_transition_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        swiglu = bool(rng.integers(2))
        M = int(rng.integers(33, 257))
        K = 128 * int(rng.integers(4, 49))
        N = 64 * int(rng.integers(4, 64)) if swiglu else 8 * int(rng.integers(40, 600))
        out.append((M, K, N, swiglu, int(rng.choice([2, 4]))))
    return out


@pytest.mark.parametrize("M,K,N,swiglu,mi", _random_transition_cases(20, seed=77))
def test_transition_stream_k_random_shapes(monkeypatch, M, K, N, swiglu, mi):
    """Seeded random transition shapes through the Stream-K form (runs of
    units that start and end anywhere in a tile, tiles shared by several
    workgroups or finished by one): parity with the oracle."""
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    monkeypatch.setenv("W4A16_TRANSITION_SK", "1")
    monkeypatch.setenv("W4A16_TRANSITION_MI", str(mi))
    d = w4a16.describe(M, K, N, swiglu=swiglu, path="prefill")
    say("random stream-k:", d)
    assert d.startswith("transition_sk_kernel<"), d
    gemm_case(M, K, N, swiglu=swiglu, path="prefill", seed=M + K + N)


@pytest.mark.parametrize("ks", [0, 1, 3])
@pytest.mark.parametrize("M,K,N,swiglu,bf16", [(33, 1152, 1064, False, False), (64, 2048, 2112, True, False),
                                               (100, 3072, 1088, False, True), (256, 1152, 2112, True, False)])
def test_transition_four_waves(monkeypatch, ks, M, K, N, swiglu, bf16):
    """Four-wave workgroups (two along N, two along K, 64-row tiles), two of
    which share a CU: ragged rows and columns, partial rounds, the automatic
    K split for two slots per CU (ks = 0) and forced ones, SwiGLU, bf16."""
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    monkeypatch.setenv("W4A16_TRANSITION_WAVES", "4")
    if ks:
        monkeypatch.setenv("W4A16_TRANSITION_KS", str(ks))
    d = w4a16.describe(M, K, N, swiglu=swiglu, path="prefill", bf16=bf16)
    say(d)
    assert d.startswith("transition_kernel<2, 2, 2, ") and "threads=256" in d, d
    if ks:
        assert "ks=%d" % ks in d, d
    gemm_case(M, K, N, swiglu=swiglu, path="prefill", seed=M + ks, bf16=bf16)


@pytest.mark.parametrize("ks", [0, 3])
@pytest.mark.parametrize("M,G,swiglu,bf16", [(100, 128, True, False), (33, 32, False, True),
                                             (200, 2048, True, True)])
def test_transition_four_waves_int8_and_zero_points(monkeypatch, ks, M, G, swiglu, bf16):
    """The four-wave instances with INT8 weights and with zero rows: ragged
    rows and columns, group sizes 32 to 2048, SwiGLU, bf16, the row factor,
    automatic and forced K splits."""
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    monkeypatch.setenv("W4A16_TRANSITION_WAVES", "4")
    if ks:
        monkeypatch.setenv("W4A16_TRANSITION_KS", str(ks))
    N = 2112 if swiglu else 1064
    for kind in ("int8", "zp"):
        d = _kernel(M, 2048, N, swiglu, bf16=bf16, **{kind: True})
        say(kind, d)
        assert d.startswith("transition_kernel<2, 2, 2, ") and "threads=256" in d, d
        assert d.split(">")[0].endswith(", 8" if kind == "int8" else "true, 4"), d
        if kind == "int8":
            gemm8_case(M, 2048, N, G=G, swiglu=swiglu, bf16=bf16, seed=M + ks, rowscale=True)
        else:
            zp_case(M, 2048, N, G=G, swiglu=swiglu, bf16=bf16, seed=M + ks, rowscale=True)


def test_transition_four_waves_integer_exact(monkeypatch):
    monkeypatch.setenv("W4A16_TRANSITION", "1")
    monkeypatch.setenv("W4A16_TRANSITION_WAVES", "4")
    for M, K, N in [(64, 4096, 2048), (200, 2048, 1024)]:
        say(w4a16.describe(M, K, N, path="prefill"))
        W = synth.grid_weights(K, N, p=4, seed=M + K)
        A = synth.ternary_activations(M, K, density=0.5, seed=M)
        out = fp16_out(w4a16.gemm(to_dev(A), w4a16.load_weight(W), path="prefill"))
        packed_o, s16_o = orc().quantize_pack(W)
        C = orc().gemm_f64(A, packed_o, s16_o)
        assert np.abs(C).max() < 128, "inputs not fp16-exact"
        assert np.array_equal(out.astype(np.float64), C)


@pytest.mark.parametrize("M,K,N,swiglu", [(96, 4096, 28672, True), (128, 4096, 28672, True),
                                          (48, 8192, 57344, True), (64, 8192, 57344, False)])
def test_transition_four_waves_full_size(M, K, N, swiglu):
    """The automatic launch where the 64-row grid fits two workgroups per CU
    without a K split (Llama-8B gate/up at M = 96 and 128, Llama-70B gate/up
    at M = 48 and 64): four-wave workgroups at full size, 1% outlier
    activations, sampled columns with the edges.  The transition kernel
    multiplies by the fp16-rounded dequantized weight (the pages' dequantize),
    so the bound is taken against that reference, the one the INT4 kernels
    page's test builds; against the exact weight (q - 8) s the outlier
    channels' share of the weight rounding, amplified by SwiGLU, can pass the
    2e-2 elementwise bound, so there the relative L2 and page-ratio bounds
    apply and the distance is reported."""
    d = w4a16.describe(M, K, N, swiglu=swiglu)
    say("four-wave full size:", d)
    assert d.startswith("transition_kernel<2, 2, 2, ") and "threads=256 ks=1" in d, d
    W = synth.weights(K, N, seed=M)
    A = synth.activations(M, K, seed=M, outliers=True)
    out = fp16_out(w4a16.gemm(to_dev(A), w4a16.load_weight(W), swiglu=swiglu))
    ncols = N // 2 if swiglu else N
    cols = sample_indices(ncols, 64, seed=M, edge=8)
    wcols = np.concatenate([cols, cols + N // 2]) if swiglu else cols
    o = orc()
    packed_o, s16_o = o.quantize_pack(np.ascontiguousarray(W[:, wcols]))
    c16 = o.gemm_w16_f64(A, o.dequant(packed_o, s16_o))
    cx = o.gemm_f64(A, packed_o, s16_o)
    got = out[:, cols]
    stats = parity.assert_close(got, o.swiglu_f64(c16) if swiglu else c16,
                                "fp16-weight reference M=%d K=%d N=%d" % (M, K, N))
    exact = parity.compare(got, o.swiglu_f64(cx) if swiglu else cx)
    say("  fp16 weights", stats)
    say("  exact weights", exact)
    assert exact["finite"] and exact["rel_l2"] <= parity.REL_L2
    assert exact["page_ratio"] < parity.PAGE_RATIO
