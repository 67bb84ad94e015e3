"""GPU GEMM parity against the oracle on the same seeded inputs, at sizes the
oracle finishes in seconds, spanning several tiles and ragged tails, on every
path (decode, prefill, dense) and with the SwiGLU epilogue."""
import re

import numpy as np
import pytest

import parity
from gpuhelp import fp16_out, gemm_case, orc, sample_indices, say, to_dev, torch
from weight_only_int4_03_amd import synth, w4a16

pytestmark = pytest.mark.gpu

PATHS = ["decode", "prefill", "dense"]


@pytest.mark.parametrize("M,K,N", synth.PAGE_TEST_SHAPES)
def test_page_shapes_auto_path(M, K, N):
    """The page's shape-parametrised test: odd M exercises row masks, N = 4160
    column masks (against A times the dequantized weights, not the originals)."""
    cols = None
    if M * K * N > 2e9:
        from gpuhelp import sample_indices
        cols = sample_indices(N, 512, seed=M, edge=64)
    gemm_case(M, K, N, cols=cols)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 7, 16, 17, 32, 33, 100, 257])
@pytest.mark.parametrize("N", [1088, 1064])
def test_each_path_ragged(path, M, N):
    """Same inputs through every path; N = 1064 leaves an 8-column tail strip,
    N = 1088 a partial tile; K = 1152 is an odd number of 128-groups."""
    gemm_case(M, 1152, N, path=path, seed=M + N)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 5, 16, 32, 70, 300])
@pytest.mark.parametrize("N", [2048, 2112])
def test_swiglu_each_path(path, M, N):
    """Fused SwiGLU on a concatenated gate/up weight; N = 2112 gives an odd
    number (33) of gate strips."""
    gemm_case(M, 1024, N, swiglu=True, path=path, seed=3 * M + N)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 9, 32, 64, 130])
def test_onehot_rows_bit_exact(path, M):
    """One-hot activation rows select dequantized weight rows: every correct
    kernel returns them bit for bit, whatever its summation order or scale
    placement.  Pins layout and nibble-permutation mistakes."""
    K, N = 2048, 1056
    say("onehot M=%d path=%s" % (M, path))
    packed, scales = synth.random_words(K, N, seed=M)         # all nibbles 0..15
    w = w4a16.repack(to_dev(packed), to_dev(scales.view(np.int16)))
    A, ks = synth.onehot_activations(M, K, seed=M)
    out = fp16_out(w4a16.gemm(to_dev(A), w, path=path))
    W16 = orc().dequant(packed, scales)
    got = out.astype(np.float64)
    want = W16[ks].view(np.float16).astype(np.float64)
    assert np.array_equal(got, want)          # values (+0 and -0 compare equal)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,K,N,density", [(1, 4096, 4096, 1.0), (16, 4096, 6144, 1.0),
                                           (33, 14336, 1024, 0.2), (200, 8192, 2048, 0.5)])
def test_integer_exact_bit_exact(path, M, K, N, density):
    """Power-of-two scales and ternary activations: every partial sum is an
    exact multiple of 1/16 below 2^24, so any summation order gives the
    oracle's value exactly, and |C| < 128 makes its fp16 rounding exact."""
    say("integer-exact M=%d K=%d N=%d path=%s" % (M, K, N, path))
    W = synth.grid_weights(K, N, p=4, seed=M)
    A = synth.ternary_activations(M, K, density=density, seed=M)
    w = w4a16.load_weight(W)
    out = fp16_out(w4a16.gemm(to_dev(A), w, path=path))
    packed_o, s16_o = orc().quantize_pack(W)
    C = orc().gemm_f64(A, packed_o, s16_o)
    assert np.abs(C).max() < 128
    assert np.array_equal(out.astype(np.float64), C)


def test_all_ones_activation():
    """A = 1 sums each column: a closed form of the group sums and scales."""
    K, N = 1024, 512
    packed, scales = synth.random_words(K, N, seed=5)
    w = w4a16.repack(to_dev(packed), to_dev(scales.view(np.int16)))
    u = orc().unpack(packed).astype(np.int64) - 8
    expect = (u.reshape(K // 128, 128, N).sum(axis=1)
              * scales.view(np.float16).astype(np.float64)).sum(axis=0)
    for path in PATHS:
        out = fp16_out(w4a16.gemm(to_dev(np.ones((3, K), np.float16)), w, path=path))
        parity.assert_close(out, np.broadcast_to(expect, (3, N)), "all-ones " + path)


def test_nibble_zero_and_outliers():
    """Nibble 0 (q = -8, never produced by the RTN quantizer but legal in the
    format) and outlier activation channels, on every path."""
    K, N, M = 2048, 512, 48
    packed, scales = synth.random_words(K, N, seed=9)
    w = w4a16.repack(to_dev(packed), to_dev(scales.view(np.int16)))
    A = synth.activations(M, K, seed=9, outliers=True)
    ref = orc().gemm_f64(A, packed, scales)
    for path in PATHS:
        parity.assert_close(fp16_out(w4a16.gemm(to_dev(A), w, path=path)), ref, path)


def test_entry_points_and_determinism():
    """w4a16_gemm / w4a16_gemm_swiglu (library workspace) equal the explicit
    form with a caller workspace, and repeated calls are bit-identical."""
    t = torch()
    K, N = 4096, 2048
    W = synth.weights(K, N, seed=11)
    w = w4a16.load_weight(W)
    for M in (1, 8, 32, 300):
        A = to_dev(synth.activations(M, K, seed=M))
        c1 = w4a16.gemm_plain(A, w)
        z1 = w4a16.gemm_swiglu(A, w)
        nbytes = max(w4a16.workspace_bytes(M, K, N), w4a16.workspace_bytes(M, K, N, swiglu=True), 1)
        ws = t.zeros(nbytes, dtype=t.uint8, device="cuda")
        c2 = w4a16.gemm(A, w, workspace=ws)
        z2 = w4a16.gemm(A, w, swiglu=True, workspace=ws)
        runs = [w4a16.gemm(A, w) for _ in range(3)]
        t.cuda.synchronize()
        assert t.equal(c1, c2) and t.equal(z1, z2), M
        assert all(t.equal(r, c1) for r in runs), M


def test_empty_and_single_group():
    t = torch()
    W = synth.weights(128, 64, seed=2)
    w = w4a16.load_weight(W)
    empty = t.empty((0, 128), dtype=t.float16, device="cuda")
    assert w4a16.gemm(empty, w).shape == (0, 64)
    for path in PATHS:
        gemm_case(3, 128, 64, path=path, W=W, weight=w, seed=2)


COOP_CONFIGS = [(4, 1, 1), (8, 1, 1), (2, 2, 1), (4, 2, 1), (2, 4, 1), (1, 4, 1), (2, 4, 2), (1, 4, 3),
                (4, 2, 2), (4, 2, 4), (2, 2, 4), (1, 8, 1), (1, 8, 3)]


@pytest.mark.parametrize("wc,wk,ks", COOP_CONFIGS)
@pytest.mark.parametrize("M", [1, 7, 16, 24, 32])
@pytest.mark.parametrize("K,N,swiglu", [(1152, 1064, False), (1024, 2112, True), (2560, 4160, False)])
def test_decode_cooperative_forced(monkeypatch, wc, wk, ks, M, K, N, swiglu):
    """The cooperative decode kernel (activations and scales staged in LDS)
    in every configuration the library can run, on ragged shapes: a tail
    strip (N = 1064), an odd number of gate strips (N = 2112), K splits that
    leave partial rounds (K = 1152, 2560 with KS = 3)."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    monkeypatch.setenv("W4A16_COOP_WC", str(wc))
    monkeypatch.setenv("W4A16_COOP_WK", str(wk))
    monkeypatch.setenv("W4A16_COOP_KS", str(ks))
    desc = w4a16.describe(M, K, N, swiglu, path="decode")
    say("coop forced:", desc)
    # At M = 32 some configurations need more LDS than a workgroup has, and
    # one column group with eight waves along K exists for plain projections
    # only: those fall back to the per-wave kernel.
    if M <= 16 and not (swiglu and (wc, wk) == (1, 8)):
        assert desc.startswith("decode_coop_kernel"), desc
    gemm_case(M, K, N, swiglu=swiglu, path="decode", seed=wc * 100 + wk * 10 + ks + M)


def test_decode_cooperative_bit_exact_integer_inputs(monkeypatch):
    """Integer-exact inputs through the cooperative kernel with a K split:
    the result is the oracle's bit for bit."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    monkeypatch.setenv("W4A16_COOP_WC", "2")
    monkeypatch.setenv("W4A16_COOP_WK", "4")
    monkeypatch.setenv("W4A16_COOP_KS", "2")
    K, N = 4096, 2048
    for M in (1, 16):
        W = synth.grid_weights(K, N, p=4, seed=M)
        A = synth.ternary_activations(M, K, density=1.0, seed=M)
        w = w4a16.load_weight(W)
        out = fp16_out(w4a16.gemm(to_dev(A), w, path="decode"))
        packed_o, s16_o = orc().quantize_pack(W)
        C = orc().gemm_f64(A, packed_o, s16_o)
        assert np.array_equal(out.astype(np.float64), C)
    # 32-row tiles, four column groups per workgroup, four K slices.
    monkeypatch.setenv("W4A16_COOP_WC", "4")
    monkeypatch.setenv("W4A16_COOP_WK", "2")
    monkeypatch.setenv("W4A16_COOP_KS", "4")
    for M in (23, 32):
        assert w4a16.describe(M, K, N, path="decode").startswith("decode_coop_kernel<32, 1, 4, 2")
        W = synth.grid_weights(K, N, p=4, seed=M)
        A = synth.ternary_activations(M, K, density=1.0, seed=M)
        w = w4a16.load_weight(W)
        out = fp16_out(w4a16.gemm(to_dev(A), w, path="decode"))
        packed_o, s16_o = orc().quantize_pack(W)
        C = orc().gemm_f64(A, packed_o, s16_o)
        assert np.array_equal(out.astype(np.float64), C)


SPLIT_CASES = [  # forced configurations with K splits
    {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "2", "W4A16_COOP_WK": "4", "W4A16_COOP_KS": "2"},
    {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "4", "W4A16_COOP_KS": "3"},
    {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "4", "W4A16_COOP_WK": "2", "W4A16_COOP_KS": "4"},
    {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "8", "W4A16_COOP_KS": "2"},
    {"W4A16_DECODE_COOP": "0", "W4A16_DECODE_KS": "2", "W4A16_DECODE_HALF": "1"},
    {"W4A16_DECODE_COOP": "0", "W4A16_DECODE_KS": "3", "W4A16_DECODE_HALF": "0"},
]


@pytest.mark.parametrize("finish", ["auto", "exchange", "last"])
@pytest.mark.parametrize("case", range(len(SPLIT_CASES)))
@pytest.mark.parametrize("M,K,N,swiglu", [(1, 1152, 1064, False), (16, 1024, 2112, True),
                                          (7, 2560, 4160, False), (32, 1152, 1064, False),
                                          (24, 1024, 2112, True)])
def test_split_finish_in_launch(monkeypatch, finish, case, M, K, N, swiglu):
    """K splits finished inside the launch, against the reduction launch that
    a call with a caller's workspace runs.  By default (auto) a call on the
    library's workspace exchanges the partials of two splits when the output
    is small; W4A16_SPLIT_FINISH forces the exchange or the last-workgroup
    sum.  The last workgroup sums the partials in split order and the
    exchange adds two partials commutatively, so both equal the reduction
    launch bit for bit (the exchange with more splits adds in a fixed tree:
    compared with the oracle).  Three calls in a row (the second on another
    shape) check that every call leaves the slots and counters clear."""
    env = SPLIT_CASES[case]
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    t = torch()
    W = synth.weights(K, N, seed=case)
    w = w4a16.load_weight(W)
    A = to_dev(synth.activations(M, K, seed=M + case))
    monkeypatch.delenv("W4A16_SPLIT_FINISH", raising=False)
    ws = t.zeros(max(w4a16.workspace_bytes(M, K, N, swiglu, path="decode"), 256), dtype=t.uint8,
                 device="cuda")
    want = fp16_out(w4a16.gemm(A, w, swiglu=swiglu, path="decode", workspace=ws))
    if finish != "auto":
        monkeypatch.setenv("W4A16_SPLIT_FINISH", finish)
    desc = w4a16.describe(M, K, N, swiglu, path="decode")
    say("split finish:", desc)
    ks = int(re.search(r"ks=(\d+)", desc).group(1))  # a configuration that does not fit falls back
    in_launch = finish != "auto" or (ks == 2 and M * (N // 2 if swiglu else N) <= 16 * 8192)
    if ks > 1:
        assert ("finished in the launch" in desc) == in_launch, desc
        assert ("decode_reduce_kernel" in desc) == (not in_launch), desc
    W2 = synth.weights(K, 2 * N, seed=case + 1)
    w2 = w4a16.load_weight(W2)
    for rep in range(3):
        got = fp16_out(w4a16.gemm(A, w2 if rep == 1 else w, swiglu=swiglu, path="decode"))
        if rep == 1:
            continue
        if finish != "exchange" or ks <= 2:
            assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), (rep, desc)
    t.cuda.synchronize()
    gemm_case(M, K, N, swiglu=swiglu, path="decode", seed=M + case, W=W, weight=w)


@pytest.mark.parametrize("M,K,N", [(16, 4096, 4096), (16, 14336, 4096), (9, 14336, 4096)])
def test_split_layout_finished_in_launch(M, K, N):
    """Narrow decode GEMMs at M = 9-16 whose cooperative layout takes two K
    splits only because the launch can finish them (Llama-8B O and down): the
    library-workspace call (two splits, exchange) and the caller-workspace
    call (the unsplit layout) both match the oracle on sampled columns, and
    reruns of the library-workspace call are bit-identical."""
    t = torch()
    desc = w4a16.describe(M, K, N)
    say("split layout:", desc)
    assert desc.startswith("decode_coop_kernel<16, 1, 1, 8, 4, "), desc
    assert "ks=2; K splits finished in the launch (exchange)" in desc, desc
    W = synth.weights(K, N, seed=M + 3)
    w = w4a16.load_weight(W)
    A = synth.activations(M, K, seed=M + 3)
    dA = to_dev(A)
    ws = t.zeros(max(w4a16.workspace_bytes(M, K, N), 256), dtype=t.uint8, device="cuda")
    own = [fp16_out(w4a16.gemm(dA, w)) for _ in range(2)]
    caller = fp16_out(w4a16.gemm(dA, w, workspace=ws))
    assert np.array_equal(own[0].view(np.uint16), own[1].view(np.uint16))
    cols = sample_indices(N, 64, seed=M, edge=8)
    o = orc()
    packed_o, s16_o = o.quantize_pack(np.ascontiguousarray(W[:, cols]), 128)
    ref = o.gemm_f64(A, packed_o, s16_o, 128)
    for name, got in (("library workspace", own[0]), ("caller workspace", caller)):
        stats = parity.assert_close(got[:, cols], ref, "%s M=%d K=%d N=%d" % (name, M, K, N))
        say("  ", name, {k: (round(v, 6) if isinstance(v, float) else v) for k, v in stats.items()})


def test_split_exchange_full_size():
    """The shapes whose automatic configuration exchanges two K splits in the
    launch (Llama-8B down at M = 8, Llama-70B down at M = 4 and 16): the
    library-workspace call equals the caller-workspace call (reduction launch)
    bit for bit, and sampled columns match the oracle."""
    t = torch()
    for M, K, N in [(8, 14336, 4096), (4, 28672, 8192), (16, 28672, 8192)]:
        desc = w4a16.describe(M, K, N)
        say("exchange full size:", desc)
        assert "ks=2" in desc and "finished in the launch (exchange)" in desc, desc
        W = synth.weights(K, N, seed=M)
        w = w4a16.load_weight(W)
        A = to_dev(synth.activations(M, K, seed=M))
        ws = t.zeros(w4a16.workspace_bytes(M, K, N), dtype=t.uint8, device="cuda")
        ref = fp16_out(w4a16.gemm(A, w, workspace=ws))
        for _ in range(2):
            got = fp16_out(w4a16.gemm(A, w))
            assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), (M, K, N)
        gemm_case(M, K, N, seed=M, W=W, weight=w, cols=sample_indices(N, 64, seed=M, edge=8))


@pytest.mark.parametrize("path", ["prefill", "dense"])
@pytest.mark.parametrize("M,K,N,swiglu", [(257, 1152, 1088, False), (300, 1024, 2112, True),
                                          (600, 2048, 4160, False), (513, 1024, 4096, True)])
def test_prefill_two_waves_per_simd(monkeypatch, path, M, K, N, swiglu):
    """The 8-wave prefill mainloop (two waves per SIMD) on ragged shapes:
    partial row tiles, a tail strip, an odd number of gate strips."""
    monkeypatch.setenv("W4A16_PREFILL_V2", "1")
    gemm_case(M, K, N, swiglu=swiglu, path=path, seed=M + N)


@pytest.mark.parametrize("half,ks,waves,depth", [(1, 1, 8, 4), (1, 2, 8, 4), (1, 3, 4, 2),
                                                (1, 1, 4, 4), (0, 1, 8, 2), (0, 2, 8, 4)])
@pytest.mark.parametrize("M,K,N,swiglu", [(1, 2048, 1064, False), (5, 4096, 2112, True),
                                          (16, 1024, 1088, False), (12, 14336, 1024, False)])
def test_decode_half_strips(monkeypatch, half, ks, waves, depth, M, K, N, swiglu):
    """The per-wave decode kernel with each workgroup on one 16-column half of
    its strips (and on whole strips), with and without split K, at both wave
    counts and pipeline depths; ragged N (a partial last strip)."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "0")
    monkeypatch.setenv("W4A16_DECODE_HALF", str(half))
    monkeypatch.setenv("W4A16_DECODE_KS", str(ks))
    monkeypatch.setenv("W4A16_DECODE_WAVES", str(waves))
    monkeypatch.setenv("W4A16_DECODE_DEPTH", str(depth))
    d = w4a16.describe(M, K, N, swiglu=swiglu, path="decode")
    assert d.split(">")[0].endswith(("true" if half else "false") + ", 4"), d
    assert ("ks=%d" % ks) in d, d
    gemm_case(M, K, N, swiglu=swiglu, path="decode", seed=M + K + ks)


def test_decode_half_strips_bit_exact_integer_inputs(monkeypatch):
    """Half-strip workgroups with split K: ternary activations and power-of-two
    scales give exact sums, so both halves of every partial tile must land in
    place for the output to be bit-exact."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "0")
    monkeypatch.setenv("W4A16_DECODE_HALF", "1")
    for ks in (1, 2):
        monkeypatch.setenv("W4A16_DECODE_KS", str(ks))
        for M, K, N in [(3, 2048, 1088), (16, 4096, 2048)]:
            W = synth.grid_weights(K, N, p=4, seed=M)
            A = synth.ternary_activations(M, K, density=1.0, seed=M)
            w = w4a16.load_weight(W)
            out = fp16_out(w4a16.gemm(to_dev(A), w, path="decode"))
            packed_o, s16_o = orc().quantize_pack(W)
            assert np.array_equal(out.astype(np.float64), orc().gemm_f64(A, packed_o, s16_o))


@pytest.mark.parametrize("half,ks,waves,depth", [(1, 1, 4, 4), (1, 3, 4, 2), (0, 1, 8, 2),
                                                (0, 2, 8, 4), (1, 5, 8, 2)])
@pytest.mark.parametrize("K,N,swiglu", [(28672, 1088, False), (14336, 2112, True), (1152, 1064, False)])
def test_decode_one_row_lds_slices(monkeypatch, half, ks, waves, depth, K, N, swiglu):
    """M = 1 through the per-wave kernel, whose two-deep one-row instances
    stage each wave's K range of the activation row in LDS: the longest
    slices (K = 28672 unsplit, 56 KiB per workgroup), uneven slices (KS = 3,
    5), K ranges shorter than the pipeline (K = 1152), both wave counts, and
    the four-deep instances that load activations per group."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "0")
    monkeypatch.setenv("W4A16_DECODE_HALF", str(half))
    monkeypatch.setenv("W4A16_DECODE_KS", str(ks))
    monkeypatch.setenv("W4A16_DECODE_WAVES", str(waves))
    monkeypatch.setenv("W4A16_DECODE_DEPTH", str(depth))
    d = w4a16.describe(1, K, N, swiglu=swiglu, path="decode")
    assert d.startswith("decode_kernel<16, %d, %d, %d, 1, " % (2 if swiglu else 1, waves, depth)), d
    gemm_case(1, K, N, swiglu=swiglu, path="decode", seed=K + ks + waves)


@pytest.mark.parametrize("ks", [1, 2])
def test_decode_one_row_slices_beyond_lds(monkeypatch, ks):
    """M = 1 with K = 81920 unsplit: eight waves' activation slices (160 KiB)
    plus the reduction tile exceed a workgroup's LDS, so M = 1 runs the
    four-rows-per-lane instance (activations loaded per group); split in two
    it fits again and stages the row."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "0")
    monkeypatch.setenv("W4A16_DECODE_KS", str(ks))
    monkeypatch.setenv("W4A16_DECODE_WAVES", "8")
    K, N = 81920, 72
    d = w4a16.describe(1, K, N, path="decode")
    rpl = 4 if ks == 1 else 1
    assert d.startswith("decode_kernel<16, 1, 8, 4, %d, " % rpl), d
    gemm_case(1, K, N, path="decode", seed=ks)


@pytest.mark.parametrize("half,ks,waves,depth", [(1, 1, 4, 4), (1, 3, 4, 2), (0, 1, 8, 2),
                                                (0, 2, 8, 4)])
@pytest.mark.parametrize("M,K,N,swiglu", [(1, 2048, 1064, False), (5, 4096, 2112, True),
                                          (12, 14336, 1024, False), (32, 2560, 1088, False)])
def test_decode_stagger_per_wave_kernel(monkeypatch, half, ks, waves, depth, M, K, N, swiglu):
    """The per-wave decode kernel with its K order rotated per workgroup, on
    half and whole strips, with and without split K (uneven wave ranges at
    KS = 3), both wave counts and depths, ragged N."""
    monkeypatch.setenv("W4A16_DECODE_STAGGER", "1")
    monkeypatch.setenv("W4A16_DECODE_COOP", "0")
    monkeypatch.setenv("W4A16_DECODE_HALF", str(half))
    monkeypatch.setenv("W4A16_DECODE_KS", str(ks))
    monkeypatch.setenv("W4A16_DECODE_WAVES", str(waves))
    monkeypatch.setenv("W4A16_DECODE_DEPTH", str(depth))
    d = w4a16.describe(M, K, N, swiglu=swiglu, path="decode")
    assert d.startswith("decode_kernel<") and " stagger" in d, d
    gemm_case(M, K, N, swiglu=swiglu, path="decode", seed=M + K + ks + 7)


@pytest.mark.parametrize("wc,wk,ks", [(1, 4, 1), (2, 4, 2), (1, 4, 3), (4, 2, 4), (2, 2, 1), (8, 1, 1)])
@pytest.mark.parametrize("M", [1, 16, 32])
@pytest.mark.parametrize("K,N,swiglu", [(1152, 1064, False), (1024, 2112, True), (2560, 4160, False)])
def test_decode_stagger_cooperative(monkeypatch, wc, wk, ks, M, K, N, swiglu):
    """The cooperative decode kernel with its rounds rotated per workgroup:
    partial last rounds (K = 1152: nine groups in rounds of four or two; K
    slices of uneven length at KS = 3) stay last, ragged N."""
    monkeypatch.setenv("W4A16_DECODE_STAGGER", "1")
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    monkeypatch.setenv("W4A16_COOP_WC", str(wc))
    monkeypatch.setenv("W4A16_COOP_WK", str(wk))
    monkeypatch.setenv("W4A16_COOP_KS", str(ks))
    d = w4a16.describe(M, K, N, swiglu, path="decode")
    assert " stagger" in d, d
    gemm_case(M, K, N, swiglu=swiglu, path="decode", seed=wc * 100 + wk * 10 + ks + M + 3)


def test_decode_stagger_bit_exact_integer_inputs(monkeypatch):
    """Integer-exact inputs through both decode kernels with the rotated K
    order (the partial sums are exact, so only a lost, repeated or misplaced
    group could change the output): bit for bit the oracle's."""
    monkeypatch.setenv("W4A16_DECODE_STAGGER", "1")
    cases = [({"W4A16_DECODE_COOP": "0", "W4A16_DECODE_HALF": "1", "W4A16_DECODE_KS": "3"}, 3, 4608, 1088),
             ({"W4A16_DECODE_COOP": "0", "W4A16_DECODE_HALF": "0", "W4A16_DECODE_KS": "1"}, 16, 4096, 2048),
             ({"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "4",
               "W4A16_COOP_KS": "1"}, 1, 4736, 2048),
             ({"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "2", "W4A16_COOP_WK": "4",
               "W4A16_COOP_KS": "3"}, 16, 4736, 2048),
             ({"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "4", "W4A16_COOP_WK": "2",
               "W4A16_COOP_KS": "2"}, 32, 4224, 2048)]
    for env, M, K, N in cases:
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        d = w4a16.describe(M, K, N, path="decode")
        assert " stagger" in d, d
        W = synth.grid_weights(K, N, p=4, seed=M + K)
        A = synth.ternary_activations(M, K, density=1.0, seed=M)
        w = w4a16.load_weight(W)
        out = fp16_out(w4a16.gemm(to_dev(A), w, path="decode"))
        packed_o, s16_o = orc().quantize_pack(W)
        assert np.array_equal(out.astype(np.float64), orc().gemm_f64(A, packed_o, s16_o)), d


PREFILL2_CONFIGS = [(64, 1, 1), (128, 1, 4), (256, 1, 2), (64, 2, 2), (128, 2, 4), (256, 2, 1),
                    (64, 1, 8), (256, 2, 4)]


@pytest.mark.parametrize("wm", [2, 1])
@pytest.mark.parametrize("bm,tps,ks", PREFILL2_CONFIGS)
@pytest.mark.parametrize("M,K,N,swiglu", [(70, 2048, 1088, False), (200, 2048, 2112, True),
                                          (129, 4096, 4160, False)])
def test_prefill2_tiles_and_k_slices(monkeypatch, wm, bm, tps, ks, M, K, N, swiglu):
    """The 8-wave mainloop at each row tile (64/128/256), with the waves as
    2 x 4 (two waves share each weight fragment) or, for 64 and 128 rows,
    1 x 8 (each wave's fragments feed all the tile's rows); one or two 64-k
    tiles per pipeline step, and split K with the FP32 partial reduction;
    ragged M and N, odd step counts per slice where the split allows."""
    if wm == 1 and bm == 256:
        pytest.skip("the 256-row tile keeps two waves along the rows")
    monkeypatch.setenv("W4A16_PREFILL_BM", str(bm))
    monkeypatch.setenv("W4A16_PREFILL_TPS", str(tps))
    monkeypatch.setenv("W4A16_PREFILL_KS", str(ks))
    monkeypatch.setenv("W4A16_PREFILL_WM", str(wm))
    d = w4a16.describe(M, K, N, swiglu=swiglu, path="prefill")
    assert "prefill2_kernel<%d, %d, %d, %d" % (bm // (32 * wm), wm, 8 // wm, tps) in d, d
    assert ("ks=%d" % ks) in d, d
    gemm_case(M, K, N, swiglu=swiglu, path="prefill", seed=M + N + bm + ks)


def test_prefill2_one_wave_rows_bit_exact_integer_inputs(monkeypatch):
    """The 1 x 8 wave layout with split K on exact sums: every row block of
    every wave lands in place."""
    monkeypatch.setenv("W4A16_PREFILL_WM", "1")
    for bm, ks in ((64, 4), (128, 2), (128, 1)):
        monkeypatch.setenv("W4A16_PREFILL_BM", str(bm))
        monkeypatch.setenv("W4A16_PREFILL_KS", str(ks))
        for M, K, N in [(96, 2048, 2048), (150, 1024, 1088)]:
            W = synth.grid_weights(K, N, p=4, seed=M)
            A = synth.ternary_activations(M, K, density=1.0, seed=M)
            w = w4a16.load_weight(W)
            out = fp16_out(w4a16.gemm(to_dev(A), w, path="prefill"))
            packed_o, s16_o = orc().quantize_pack(W)
            assert np.array_equal(out.astype(np.float64), orc().gemm_f64(A, packed_o, s16_o))


@pytest.mark.parametrize("wm", [2, 1])
@pytest.mark.parametrize("ks", [2, 3, 4, 7])
def test_prefill2_uneven_k_slices_bit_exact(monkeypatch, wm, ks):
    """K slices that differ by one pipeline step (K = 1152: 9 steps of 128 k;
    K = 11008: 86 steps): exact sums, bit-exact output."""
    monkeypatch.setenv("W4A16_PREFILL_BM", "64")
    monkeypatch.setenv("W4A16_PREFILL_WM", str(wm))
    monkeypatch.setenv("W4A16_PREFILL_KS", str(ks))
    for M, K, N in [(70, 1152, 1088), (40, 11008, 1024)]:
        assert ("ks=%d" % ks) in w4a16.describe(M, K, N, path="prefill")
        W = synth.grid_weights(K, N, p=4, seed=M + ks)
        A = synth.ternary_activations(M, K, density=0.3 if K > 4096 else 1.0, seed=M)
        w = w4a16.load_weight(W)
        out = fp16_out(w4a16.gemm(to_dev(A), w, path="prefill"))
        packed_o, s16_o = orc().quantize_pack(W)
        assert np.array_equal(out.astype(np.float64), orc().gemm_f64(A, packed_o, s16_o)), (M, K)


def test_prefill2_split_k_bit_exact_integer_inputs(monkeypatch):
    """Split K sums FP32 partials in slice order; with small-integer inputs
    every partial and sum is exact, so the output is bit-exact."""
    monkeypatch.setenv("W4A16_PREFILL_BM", "64")
    monkeypatch.setenv("W4A16_PREFILL_KS", "4")
    for M, K, N in [(96, 2048, 2048), (80, 4096, 1024)]:
        W = synth.grid_weights(K, N, p=4, seed=M)
        A = synth.ternary_activations(M, K, density=1.0, seed=M)
        w = w4a16.load_weight(W)
        assert "ks=4" in w4a16.describe(M, K, N, path="prefill")
        out = fp16_out(w4a16.gemm(to_dev(A), w, path="prefill"))
        packed_o, s16_o = orc().quantize_pack(W)
        C = orc().gemm_f64(A, packed_o, s16_o)
        assert np.array_equal(out.astype(np.float64), C)


@pytest.mark.parametrize("path", ["prefill", "dense"])
@pytest.mark.parametrize("M,K,N,swiglu", [(40, 1024, 1088, False), (130, 1152, 2112, True),
                                          (300, 2048, 4096, False)])
def test_prefill_one_wave_kernel(monkeypatch, path, M, K, N, swiglu):
    """The one-wave-per-SIMD mainloop, which the fused path and the dense
    tier fall back to when an operand exceeds 32-bit buffer offsets (forced
    here)."""
    monkeypatch.setenv("W4A16_PREFILL_V2", "0")
    d = w4a16.describe(M, K, N, swiglu=swiglu, path=path)
    assert ("prefill_kernel<" if path == "prefill" else "; prefill_kernel<") in d, d
    gemm_case(M, K, N, swiglu=swiglu, path=path, seed=M + K)


def test_measurement_probes_run():
    """The ceiling probes run, report their work, and leave the sink alone."""
    T = torch()
    sink = T.zeros(4, dtype=T.int32, device="cuda")
    buf = T.arange(1 << 20, dtype=T.int32, device="cuda")
    w4a16.probe_stream_read(buf, sink)
    fl = w4a16.probe_mfma(16, 8, sink)
    T.cuda.synchronize()
    assert fl == 8 * 4 * 16 * 4 * 32768
    assert int(sink.abs().sum()) == 0



# -- bf16 activations -------------------------------------------------------------

@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,K,N,swiglu", [(1, 1024, 1064, False), (7, 2048, 2112, True),
                                          (32, 1152, 4160, False), (70, 2048, 1088, False),
                                          (300, 1024, 2112, True), (513, 2048, 4096, False)])
def test_bf16_each_path(path, M, K, N, swiglu):
    """bf16 activations and output on every path, ragged M and N, with and
    without the SwiGLU epilogue."""
    gemm_case(M, K, N, swiglu=swiglu, path=path, seed=M + K + N, bf16=True)


@pytest.mark.parametrize("wc,wk,ks", [(2, 4, 1), (1, 4, 1), (2, 2, 2), (4, 1, 1)])
@pytest.mark.parametrize("M", [1, 16, 32])
def test_bf16_decode_cooperative(monkeypatch, wc, wk, ks, M):
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    monkeypatch.setenv("W4A16_COOP_WC", str(wc))
    monkeypatch.setenv("W4A16_COOP_WK", str(wk))
    monkeypatch.setenv("W4A16_COOP_KS", str(ks))
    gemm_case(M, 2048, 2112, swiglu=True, path="decode", seed=wc + wk + ks + M, bf16=True)


@pytest.mark.parametrize("bm,ks", [(64, 1), (128, 4), (256, 2)])
def test_bf16_prefill_tiles(monkeypatch, bm, ks):
    monkeypatch.setenv("W4A16_PREFILL_BM", str(bm))
    monkeypatch.setenv("W4A16_PREFILL_KS", str(ks))
    gemm_case(200, 2048, 2112, swiglu=True, path="prefill", seed=bm + ks, bf16=True)


@pytest.mark.parametrize("path", PATHS)
def test_bf16_bit_exact_integer_inputs(path):
    """Ternary activations and power-of-two scales make every weight, product
    and partial sum exact in bf16 / FP32, so the bf16 output is the oracle's
    sum rounded once: bit-exact."""
    from gpuhelp import bf16_dev, bf16_out
    for M, K, N in [(5, 2048, 1088), (96, 2048, 2048)]:
        W = synth.grid_weights(K, N, p=4, seed=M)
        A = synth.ternary_activations(M, K, density=1.0, seed=M)
        Ab = orc().f64_to_bf16(A.astype(np.float64))
        w = w4a16.load_weight(W)
        out = bf16_out(w4a16.gemm(bf16_dev(Ab), w, path=path))
        packed_o, s16_o = orc().quantize_pack(W)
        C = orc().gemm_bf16_f64(Ab, packed_o, s16_o)
        assert np.array_equal(out, orc().f64_to_bf16(C)), (path, M, K, N)


def test_bf16_transition_with_outliers():
    """1% of K-channels scaled by 20 (the transition batches' activations)."""
    gemm_case(128, 4096, 4096, path="auto", seed=3, outliers=True, bf16=True)


# -- folded RMSNorm gain and the row-factor epilogue ----------------------------

def _rowscale(M, seed):
    """Seeded positive row factors, as an RMSNorm produces (inputs to both sides)."""
    rng = np.random.default_rng(seed)
    return (0.25 + 1.5 * rng.random(M)).astype(np.float32)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M,K,N,swiglu,bf16", [(1, 1024, 1064, False, False), (7, 2048, 2112, True, False),
                                               (40, 1152, 1088, False, True), (70, 2048, 2112, True, True),
                                               (300, 1024, 4096, False, False)])
def test_gemm_rowscale_each_path(path, M, K, N, swiglu, bf16):
    """out[m,:] = rho[m] * (A W)[m,:], the factor applied before SwiGLU, on
    every path (split-K reductions included), fp16 and bf16."""
    from gpuhelp import bf16_dev, bf16_out
    say("rowscale M=%d K=%d N=%d swiglu=%s bf16=%s path=%s" % (M, K, N, swiglu, bf16, path))
    W = synth.weights(K, N, seed=M + K)
    w = w4a16.load_weight(W)
    rho = _rowscale(M, M + N)
    rho_d = torch().from_numpy(rho).cuda()
    o = orc()
    packed_o, s16_o = o.quantize_pack(W)
    if bf16:
        A = synth.activations_bf16(M, K, seed=M)
        out = bf16_out(w4a16.gemm(bf16_dev(A), w, swiglu=swiglu, path=path, rowscale=rho_d))
        C = o.gemm_bf16_f64(A, packed_o, s16_o)
    else:
        A = synth.activations(M, K, seed=M)
        out = fp16_out(w4a16.gemm(to_dev(A), w, swiglu=swiglu, path=path, rowscale=rho_d))
        C = o.gemm_f64(A, packed_o, s16_o)
    C = o.scale_rows(C, rho.astype(np.float64))
    ref = o.swiglu_f64(C) if swiglu else C
    if bf16:
        parity.assert_close_bf16(out, ref, "rowscale bf16")
    else:
        parity.assert_close(out, ref, "rowscale")


def test_pack_gain_bit_exact():
    """w4a16_pack_gain packs fp32(gamma[k] W[k,n]) bit for bit as the oracle
    quantizes the folded weights."""
    for K, N in [(1024, 1064), (4096, 4096)]:
        W = synth.weights(K, N, seed=K)
        gamma = (0.5 + np.random.default_rng(K).random(K)).astype(np.float32)
        p_d, s_d = w4a16.pack(to_dev(W), gamma=to_dev(gamma))
        po, so = orc().quantize_pack(orc().fold_gain(W, gamma))
        assert np.array_equal(p_d.cpu().numpy(), po)
        assert np.array_equal(s_d.cpu().numpy().view(np.uint16), so)


@pytest.mark.parametrize("bf16", [False, True])
def test_rms_rowscale_matches_oracle(bf16):
    """rho in FP32 against the fp64 oracle (relative 1e-6), deterministic."""
    from gpuhelp import bf16_dev
    for M, K in [(1, 4096), (33, 14336), (257, 1024)]:
        if bf16:
            A = synth.activations_bf16(M, K, seed=K + M, outliers=True)
            Ad = bf16_dev(A)
        else:
            A = synth.activations(M, K, seed=K + M, outliers=True)
            Ad = to_dev(A)
        r1 = w4a16.rms_rowscale(Ad, eps=1e-5).cpu().numpy()
        r2 = w4a16.rms_rowscale(Ad, eps=1e-5).cpu().numpy()
        ref = orc().rms_rowscale_f64(A, 1e-5, bf16=bf16)
        assert np.array_equal(r1, r2)
        assert np.allclose(r1.astype(np.float64), ref, rtol=1e-6, atol=0), np.abs(r1 / ref - 1).max()


def test_rmsnorm_folded_projection_end_to_end():
    """The section's whole identity: raw x, gain folded into W before
    quantizing, rho from x, rho applied in the epilogue -- against the
    oracle's rho_m * sum_h x W' (W' quantized), with SwiGLU."""
    M, K, N = 24, 4096, 2112
    W = synth.weights(K, N, seed=11)
    gamma = (0.8 + 0.4 * np.random.default_rng(11).random(K)).astype(np.float32)
    A = synth.activations(M, K, seed=11, outliers=True)
    w = w4a16.load_weight(W, gamma=gamma)
    Ad = to_dev(A)
    rho = w4a16.rms_rowscale(Ad, eps=1e-6)
    out = fp16_out(w4a16.gemm(Ad, w, swiglu=True, rowscale=rho))
    o = orc()
    po, so = o.quantize_pack(o.fold_gain(W, gamma))
    C = o.scale_rows(o.gemm_f64(A, po, so), o.rms_rowscale_f64(A, 1e-6))
    parity.assert_close(out, o.swiglu_f64(C), "rmsnorm folded projection")


# -- group sizes other than 128 ---------------------------------------------------

@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("G,M,K,N,swiglu,bf16", [(32, 1, 1024, 1064, False, False),
                                                 (32, 24, 2048, 2112, True, False),
                                                 (64, 7, 2048, 1088, False, True),
                                                 (64, 300, 1024, 2112, True, False),
                                                 (256, 16, 4096, 1088, False, False),
                                                 (256, 130, 2048, 2112, True, True),
                                                 (1152, 5, 1152, 1064, False, False),
                                                 (1152, 70, 1152, 2112, True, False),
                                                 (2048, 33, 2048, 1088, False, True)])
def test_group_sizes_each_path(path, G, M, K, N, swiglu, bf16):
    """Every path with G = 32, 64, 256 and channelwise scales (one scale per
    column: G = K, including K = 1152, not a power of two)."""
    gemm_case(M, K, N, swiglu=swiglu, path=path, seed=G + M, bf16=bf16, G=G)


@pytest.mark.parametrize("G", [256, 2048])
def test_group_sizes_cooperative_decode(monkeypatch, G):
    """The cooperative decode kernel reads one scale per column and 128-k
    unit, so it takes G >= 128 (smaller groups use the per-wave kernel)."""
    monkeypatch.setenv("W4A16_DECODE_COOP", "1")
    assert w4a16.describe(16, 2048, 2112, swiglu=True, path="decode", G=G).startswith(
        "decode_coop_kernel")
    assert w4a16.describe(16, 2048, 2112, swiglu=True, path="decode", G=64).startswith(
        "decode_kernel")
    gemm_case(16, 2048, 2112, swiglu=True, path="decode", seed=G, G=G)


@pytest.mark.parametrize("path", PATHS)
def test_group_size_32_bit_exact_integer_inputs(path):
    """Ternary activations with power-of-two scales at G = 32: exact sums,
    bit-exact fp16 output."""
    for M, K, N in [(3, 1024, 1088), (90, 2048, 2048)]:
        W = synth.grid_weights(K, N, p=4, seed=M, group=32)
        A = synth.ternary_activations(M, K, density=1.0, seed=M)
        w = w4a16.load_weight(W, G=32)
        out = fp16_out(w4a16.gemm(to_dev(A), w, path=path))
        packed_o, s16_o = orc().quantize_pack(W, 32)
        assert np.array_equal(out.astype(np.float64), orc().gemm_f64(A, packed_o, s16_o, 32))


@pytest.mark.parametrize("half,waves,depth", [(1, 8, 2), (0, 8, 2), (1, 4, 4), (0, 4, 4)])
@pytest.mark.parametrize("K,N,swiglu", [(4096, 4096, False), (1152, 1064, False),
                                        (14336, 1024, False), (2048, 2112, True)])
def test_decode_dot_one_row(monkeypatch, half, waves, depth, K, N, swiglu):
    """The one-row instances without the matrix unit (v_dot2_f32_f16 per lane,
    ds_swizzle and v_permlane32_swap lane sums), forced, at both strip splits,
    wave counts and pipeline depths; ragged N and an odd group count."""
    monkeypatch.setenv("W4A16_DECODE_DOT", "1")
    monkeypatch.setenv("W4A16_DECODE_COOP", "0")
    monkeypatch.setenv("W4A16_DECODE_HALF", str(half))
    monkeypatch.setenv("W4A16_DECODE_WAVES", str(waves))
    monkeypatch.setenv("W4A16_DECODE_DEPTH", str(depth))
    d = w4a16.describe(1, K, N, swiglu=swiglu, path="decode")
    assert d.startswith("decode_kernel<16, %d, %d, %d, 0, " % (2 if swiglu else 1, waves, depth)), d
    gemm_case(1, K, N, swiglu=swiglu, path="decode", seed=K + N + half)


def test_decode_dot_one_row_bit_exact(monkeypatch):
    """Exact sums (ternary activations, power-of-two scales) and one-hot rows
    through the dot instances: bit for bit."""
    monkeypatch.setenv("W4A16_DECODE_DOT", "1")
    monkeypatch.setenv("W4A16_DECODE_COOP", "0")
    for K, N in ((4096, 6144), (14336, 4096)):
        W = synth.grid_weights(K, N, p=4, seed=K)
        A = synth.ternary_activations(1, K, density=0.5, seed=K)
        out = fp16_out(w4a16.gemm(to_dev(A), w4a16.load_weight(W), path="decode"))
        packed_o, s16_o = orc().quantize_pack(W)
        assert np.array_equal(out.astype(np.float64), orc().gemm_f64(A, packed_o, s16_o))
    K, N = 2048, 1056
    packed, scales = synth.random_words(K, N, seed=5)
    w = w4a16.repack(to_dev(packed), to_dev(scales.view(np.int16)))
    A, ks = synth.onehot_activations(1, K, seed=5)
    out = fp16_out(w4a16.gemm(to_dev(A), w, path="decode"))
    want = orc().dequant(packed, scales)[ks].view(np.float16).astype(np.float64)
    assert np.array_equal(out.astype(np.float64), want)


def _random_decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        swiglu = bool(rng.integers(2))
        M = int(rng.integers(1, 33))
        K = 128 * int(rng.integers(4, 41))
        N = 64 * int(rng.integers(4, 48)) if swiglu else 8 * int(rng.integers(40, 400))
        out.append((M, K, N, swiglu, int(rng.integers(2, 6)), bool(rng.integers(2))))
    return out


@pytest.mark.parametrize("M,K,N,swiglu,ks,coop", _random_decode_cases(24, seed=2026))
def test_split_exchange_random_shapes(monkeypatch, M, K, N, swiglu, ks, coop):
    """Seeded random decode shapes with K forced into 2-5 splits on either
    decode kernel, finished inside the launch by the exchange tree: parity
    with the oracle, and with two splits the same bits as the reduction
    launch that a caller's workspace gets."""
    monkeypatch.setenv("W4A16_SPLIT_FINISH", "exchange")
    if coop:
        monkeypatch.setenv("W4A16_DECODE_COOP", "1")
        monkeypatch.setenv("W4A16_COOP_KS", str(ks))
    else:
        monkeypatch.setenv("W4A16_DECODE_COOP", "0")
        monkeypatch.setenv("W4A16_DECODE_KS", str(ks))
    d = w4a16.describe(M, K, N, swiglu, path="decode")
    say("random exchange:", d)
    W = synth.weights(K, N, seed=M + K + N)
    w = w4a16.load_weight(W)
    gemm_case(M, K, N, swiglu=swiglu, path="decode", seed=M + ks, W=W, weight=w)
    if "ks=2;" in d:
        t = torch()
        A = to_dev(synth.activations(M, K, seed=M + ks))
        got = fp16_out(w4a16.gemm(A, w, swiglu=swiglu, path="decode"))
        monkeypatch.setenv("W4A16_SPLIT_FINISH", "reduce")
        ws = t.zeros(max(w4a16.workspace_bytes(M, K, N, swiglu, path="decode"), 256),
                     dtype=t.uint8, device="cuda")
        want = fp16_out(w4a16.gemm(A, w, swiglu=swiglu, path="decode", workspace=ws))
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), d


@pytest.mark.parametrize("variant", ["bf16", "zp", "int8", "zp_bf16", "int8_bf16"])
@pytest.mark.parametrize("M,K,N", [(8, 14336, 4096), (4, 28672, 8192)])
def test_split_exchange_variants_full_size(variant, M, K, N):
    """The in-launch exchange in the bf16, zero-point and INT8 instances of
    the decode kernels at the full Llama down-projection shapes whose
    automatic configuration exchanges two K splits: the library-workspace
    call equals the caller-workspace call (reduction launch) bit for bit, and
    sampled columns match the oracle."""
    from gpuhelp import bf16_dev, bf16_out
    from test_gpu_int8 import gemm8_case
    from test_gpu_zero_points import zp_case, zp_inputs
    t = torch()
    bf16 = variant.endswith("bf16")
    zp, int8 = variant.startswith("zp"), variant.startswith("int8")
    d = w4a16.describe(M, K, N, bf16=bf16, zp=zp, int8=int8)
    say("exchange variant:", variant, d)
    assert "ks=2" in d and "finished in the launch (exchange)" in d, d
    if zp:
        w = zp_inputs(K, N, 128, seed=M)[0]
    elif int8:
        w = w4a16.load_weight_int8(synth.weights(K, N, seed=M))
    else:
        w = w4a16.load_weight(synth.weights(K, N, seed=M))
    if bf16:
        A = bf16_dev(synth.activations_bf16(M, K, seed=M))
    else:
        A = to_dev(synth.activations(M, K, seed=M))
    ws = t.zeros(w4a16.workspace_bytes(M, K, N, bf16=bf16, zp=zp, int8=int8), dtype=t.uint8,
                 device="cuda")
    conv = bf16_out if bf16 else fp16_out
    ref = conv(w4a16.gemm(A, w, workspace=ws))
    got = conv(w4a16.gemm(A, w))
    assert np.array_equal(np.asarray(got).view(np.uint16), np.asarray(ref).view(np.uint16)), d
    cols = sample_indices(N, 48, seed=M, edge=8)
    if zp:
        zp_case(M, K, N, bf16=bf16, seed=M, cols=cols)
    elif int8:
        gemm8_case(M, K, N, bf16=bf16, seed=M, cols=cols)
    else:
        gemm_case(M, K, N, seed=M, bf16=True, cols=cols)
