"""The C-ABI library on the CPU: it loads, exports every function its header
declares, validates arguments without touching the GPU, and its host
quantize+pack is bit-exact with the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
from weight_only_int4_03_amd import synth, w4a16


def test_library_exports_every_header_function():
    L = w4a16.lib()
    names = w4a16.header_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), name
        assert name in w4a16._SIGNATURES, name


def test_version_and_no_error():
    assert w4a16.lib().w4a16_version().startswith(b"w4a16")


@pytest.mark.parametrize("K,N", [(128, 8), (512, 72), (4096, 4096), (11008, 264), (384, 4160)])
def test_pack_host_matches_oracle(K, N):
    W = synth.weights(K, N, seed=K + N)
    p, s = w4a16.pack_host(W)
    po, so = oracle.load().quantize_pack(W)
    assert np.array_equal(p, po)
    assert np.array_equal(s, so)


def test_pack_host_ties_and_zero_groups():
    W = synth.grid_weights(256, 16, p=1, seed=1)
    W[:, 3] = 0.0
    col = np.zeros(128, np.float32)
    col[0] = 7.0
    col[1:6] = [2.5, -2.5, 0.5, 3.5, -0.5]
    W[:128, 5] = col
    p, s = w4a16.pack_host(W)
    po, so = oracle.load().quantize_pack(W)
    assert np.array_equal(p, po) and np.array_equal(s, so)


def test_pack_host_rejects_nonfinite():
    W = np.zeros((128, 8), np.float32)
    W[5, 5] = np.inf
    with pytest.raises(w4a16.W4A16Error) as e:
        w4a16.pack_host(W)
    assert e.value.code == w4a16.ERR_NONFINITE


def _gemm_ex(**kw):
    args = dict(A=0, M=1, K=4096, rw=0, rs=0, N=4096, G=128, out=0, flags=0, ws=0, wsb=0, stream=0)
    args.update(kw)
    return w4a16.lib().w4a16_gemm_ex(args["A"], args["M"], args["K"], args["rw"], args["rs"],
                                     args["N"], args["G"], args["out"], args["flags"], args["ws"],
                                     args["wsb"], args["stream"])


def test_gemm_argument_errors_without_gpu():
    assert _gemm_ex(G=384, K=12288) == w4a16.ERR_UNSUPPORTED   # not a power of two, not K
    assert _gemm_ex(G=16) == w4a16.ERR_UNSUPPORTED              # below a lane vector
    assert _gemm_ex(G=64) == w4a16.ERR_INVALID                  # supported G: null pointers
    assert _gemm_ex(G=4096) == w4a16.ERR_INVALID                # channelwise: null pointers
    assert _gemm_ex(K=4160, G=64) == w4a16.ERR_INVALID          # K % 128
    assert _gemm_ex(K=4000) == w4a16.ERR_INVALID
    assert _gemm_ex(N=4100) == w4a16.ERR_INVALID
    assert _gemm_ex(M=-1) == w4a16.ERR_INVALID
    assert _gemm_ex() == w4a16.ERR_INVALID                       # null pointers
    assert "null" in w4a16.last_error()
    assert _gemm_ex(flags=w4a16.FLAG_SWIGLU, N=4128) == w4a16.ERR_INVALID  # N % 64
    assert _gemm_ex(flags=0x100) == w4a16.ERR_INVALID             # unknown flag
    assert _gemm_ex(flags=w4a16.FLAG_BF16) == w4a16.ERR_INVALID    # bf16 flag known: null pointers
    assert "null" in w4a16.last_error()
    assert _gemm_ex(M=0) == w4a16.OK                              # empty product: no-op
    assert _gemm_ex(A=8, rw=16, rs=16, out=16) == w4a16.ERR_INVALID  # misaligned A
    assert "aligned" in w4a16.last_error()


def test_zero_point_argument_errors_without_gpu():
    L = w4a16.lib()
    ok = dict(A=16, M=1, K=4096, rw=16, rs=16, rz=16, N=4096, G=128, rowscale=0, out=16,
              flags=0, ws=0, wsb=0, stream=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.w4a16_gemm_zp(a["A"], a["M"], a["K"], a["rw"], a["rs"], a["rz"], a["N"],
                               a["G"], a["rowscale"], a["out"], a["flags"], a["ws"], a["wsb"],
                               a["stream"])
    assert call(rz=0) == w4a16.ERR_INVALID
    assert "zero rows" in w4a16.last_error()
    assert call(rz=8) == w4a16.ERR_INVALID                       # misaligned
    assert "aligned" in w4a16.last_error()
    assert call(flags=0x100) == w4a16.ERR_INVALID
    assert call(G=384, K=12288) == w4a16.ERR_UNSUPPORTED
    assert call(M=0, rz=0) == w4a16.OK                             # empty product: no-op
    # A flag that only the zero-point entry point takes.
    assert _gemm_ex(flags=w4a16.FLAG_ZP) == w4a16.ERR_INVALID
    assert "flags" in w4a16.last_error()
    assert L.w4a16_zero_rows(0, 16, 4096, 4096, 128, 16, 0) == w4a16.ERR_INVALID
    assert L.w4a16_zero_rows(16, 16, 4096, 4096, 128, 8, 0) == w4a16.ERR_INVALID
    assert L.w4a16_zero_rows(16, 16, 4096, 4096, 100, 16, 0) == w4a16.ERR_INVALID  # K % G
    assert L.w4a16_dequant_zp(16, 16, 0, 4096, 4096, 128, 0, 16, 0) == w4a16.ERR_INVALID
    assert L.w4a16_dequant_zp(16, 16, 16, 4096, 4096, 128, 0x10, 16, 0) == w4a16.ERR_INVALID
    # Workspace sizes follow the zero-point dispatch (no cooperative decode).
    assert w4a16.workspace_bytes(16, 14336, 4096, zp=True) >= 0


def test_int8_argument_errors_without_gpu():
    L = w4a16.lib()
    assert L.w4a16_pack_int8(16, 4096, 4096, 6, 16, 16, 0) == w4a16.ERR_INVALID     # K % G
    assert L.w4a16_pack_int8(16, 4104, 4096, 1026, 16, 16, 0) == w4a16.ERR_UNSUPPORTED  # G % 4
    assert L.w4a16_pack_int8(0, 4096, 4096, 128, 16, 16, 0) == w4a16.ERR_INVALID
    assert L.w4a16_repack_int8(16, 16, 12288, 4096, 384, 16, 16, 0) == w4a16.ERR_UNSUPPORTED
    assert L.w4a16_repack_int8(16, 16, 4096, 4096, 128, 8, 16, 0) == w4a16.ERR_INVALID  # align
    assert L.w4a16_dequant_int8(16, 16, 4096, 4096, 128, 0x10, 16, 0) == w4a16.ERR_INVALID
    assert L.w4a16_gemm_int8(16, 1, 4096, 16, 16, 4096, 128, 0, 16, 0x100, 0, 0, 0) == w4a16.ERR_INVALID
    assert L.w4a16_gemm_int8(0, 1, 4096, 16, 16, 4096, 128, 0, 16, 0, 0, 0, 0) == w4a16.ERR_INVALID
    assert L.w4a16_gemm_int8(0, 0, 4096, 0, 0, 4096, 128, 0, 0, 0, 0, 0, 0) == w4a16.OK
    assert _gemm_ex(flags=w4a16.FLAG_INT8) == w4a16.ERR_INVALID    # only w4a16_gemm_int8 takes it
    assert w4a16.lib().w4a16_repacked_weight_bytes_int8(4096, 4104, 128) == 4096 * 4128
    assert w4a16.workspace_bytes(100, 4096, 4096, path="dense", int8=True) >= 4096 * 4096 * 2
    buf = ctypes.create_string_buffer(64)
    assert L.w4a16_describe(1, 4096, 4096, 128, w4a16.FLAG_INT8 | w4a16.FLAG_ZP,
                            ctypes.addressof(buf), 64) == w4a16.ERR_UNSUPPORTED


def test_other_argument_errors():
    L = w4a16.lib()
    assert L.w4a16_repack(0, 0, 4096, 4096, 128, 0, 0, 0) == w4a16.ERR_INVALID
    assert L.w4a16_repack(16, 16, 12288, 4096, 384, 16, 16, 0) == w4a16.ERR_UNSUPPORTED
    assert L.w4a16_dequant(16, 16, 100, 4096, 128, 16, 0) == w4a16.ERR_INVALID
    assert L.w4a16_pack(0, 4096, 4096, 128, 0, 0, 0) == w4a16.ERR_INVALID
    assert L.w4a16_pack(16, 4080, 4096, 30, 16, 16, 0) == w4a16.ERR_UNSUPPORTED   # G % 8
    assert L.w4a16_repacked_weight_bytes(100, 8, 128) == w4a16.ERR_INVALID
    assert L.w4a16_select_path(1, 4096, 4096, 128, 0) == w4a16.PATH_DECODE


def test_probe_argument_errors_without_gpu():
    L = w4a16.lib()
    assert L.w4a16_probe_stream_read(0, 1024, 16, 0) == w4a16.ERR_INVALID      # null buffer
    assert L.w4a16_probe_stream_read(16, 1000, 16, 0) == w4a16.ERR_INVALID     # not 16-byte words
    assert L.w4a16_probe_stream_read(16, 0, 16, 0) == w4a16.ERR_INVALID
    assert L.w4a16_probe_stream_read(8, 1024, 16, 0) == w4a16.ERR_INVALID      # misaligned
    assert "aligned" in w4a16.last_error()
    assert L.w4a16_probe_mfma(0, 1, 16, 0, 0) == w4a16.ERR_INVALID
    assert L.w4a16_probe_mfma(1, 0, 16, 0, 0) == w4a16.ERR_INVALID
    assert L.w4a16_probe_mfma(1 << 25, 1, 16, 0, 0) == w4a16.ERR_INVALID
    assert L.w4a16_probe_mfma(10, 1, 0, 0, 0) == w4a16.ERR_INVALID             # null sink


def test_repacked_sizes():
    wb, sb = w4a16.repacked_bytes(4096, 4096)
    assert wb == 4096 * 4096 // 2                      # same bytes as the packed words
    assert sb == 4096 // 128 * 4096 * 2                # scale groups already a multiple of 8
    wb, sb = w4a16.repacked_bytes(11008, 4104)         # N padded to 32, groups to 8
    assert wb == 11008 * 4128 // 2
    assert sb == 88 * 4128 * 2


def test_dispatch_table():
    assert w4a16.select_path(1, 4096, 4096) == "decode"
    assert w4a16.select_path(32, 4096, 4096) == "decode"
    assert w4a16.select_path(4096, 4096, 28672) == "prefill"
    assert w4a16.workspace_bytes(4096, 4096, 4096, path="dense") >= 4096 * 4096 * 2


def test_decode_stagger_rule(monkeypatch):
    """The rotated K order of the decode kernels is on where a strip's byte
    stride is a multiple of 128 KiB (INT4 at K = 8192, INT8 at K = 4096) and
    off elsewhere; the environment overrides it either way."""
    monkeypatch.delenv("W4A16_DECODE_STAGGER", raising=False)
    assert " stagger" in w4a16.describe(1, 8192, 10240)
    assert " stagger" in w4a16.describe(16, 8192, 57344, swiglu=True)
    assert " stagger" in w4a16.describe(1, 4096, 4096, int8=True)
    assert " stagger" not in w4a16.describe(1, 4096, 4096)
    assert " stagger" not in w4a16.describe(32, 14336, 4096)
    assert " stagger" not in w4a16.describe(16, 28672, 8192)
    d = w4a16.describe(16, 14336, 4096)
    assert d.index(" stagger") if " stagger" in d else True
    monkeypatch.setenv("W4A16_DECODE_STAGGER", "0")
    assert " stagger" not in w4a16.describe(1, 8192, 10240)
    monkeypatch.setenv("W4A16_DECODE_STAGGER", "1")
    d = w4a16.describe(16, 14336, 4096)
    assert " stagger" in d and d.index(" stagger") < d.index(";"), d
    assert " stagger" not in w4a16.describe(4096, 4096, 28672, swiglu=True)  # prefill


def test_describe_names_the_launches():
    """The launch description names kernel instances as profilers print them
    (template arguments after the tile shape: SwiGLU epilogue, bf16
    activations, then for decode_kernel the scaling before the MFMA, and for
    decode_kernel and prefill2_kernel the zero rows, and for decode_kernel the
    half-strip workgroups)."""
    d = w4a16.describe(1, 4096, 28672, swiglu=True)
    assert d.startswith("decode_coop_kernel<16, 2, ") and d.split(">")[0].endswith(
        "true, false, false, 4"), d
    d = w4a16.describe(1, 4096, 28672, swiglu=True, bf16=True)
    assert d.startswith("decode_coop_kernel<16, 2, ") and d.split(">")[0].endswith(
        "true, true, false, 4"), d
    d = w4a16.describe(1, 4096, 4096)
    assert d.startswith("decode_kernel<16, 1, ") and d.split(">")[0].endswith(
        "false, false, false, false, true, 4"), d     # 128 strips: half strips; INT4
    assert " workgroups=256 " in d and d.endswith("ks=1"), d
    # 32-row tiles: the cooperative kernel, K split to fill the CUs (its
    # 8-bit instance for INT8 weights).
    d = w4a16.describe(24, 4096, 4096)
    assert d.startswith("decode_coop_kernel<32, 1, 2, 4, 16, false, false, false, 4> workgroups=256 "), d
    assert d.endswith("ks=4; decode_reduce_kernel<1, false, false>"), d
    d = w4a16.describe(24, 4096, 4096, int8=True)
    assert d.startswith("decode_coop_kernel<32, 1, 2, 4, 16, false, false, false, 8>"), d
    # Two K splits of a small output (M * output columns <= 16 * 8192) are
    # finished inside the launch by exchanging the partials; more splits or a
    # larger output keep the reduction launch.
    d = w4a16.describe(8, 14336, 4096)
    assert d.endswith("ks=2; K splits finished in the launch (exchange)"), d
    d = w4a16.describe(16, 28672, 8192)
    assert d.endswith("ks=2; K splits finished in the launch (exchange)"), d
    d = w4a16.describe(32, 8192, 8192)
    assert "ks=2" in d and d.endswith("decode_reduce_kernel<1, false, false>"), d
    # Mid-width plain projections: one column group with eight waves along
    # K, no K split; the widest fused ones: four column groups, two groups of
    # 128 k per round.
    assert w4a16.describe(32, 4096, 6144).startswith(
        "decode_coop_kernel<32, 1, 1, 8, 16, false, false, false, 4> workgroups=192 threads=512 ks=1")
    # The same at M = 16 (and QKV above M = 8); O at M = 8-12 stays on the
    # per-wave kernel.
    assert w4a16.describe(16, 4096, 6144).startswith(
        "decode_coop_kernel<16, 1, 1, 8, 4, false, false, false, 4> workgroups=192 threads=512 ks=1")
    assert w4a16.describe(16, 4096, 4096).startswith("decode_coop_kernel<16, 1, 1, 8, 4, ")
    assert w4a16.describe(12, 4096, 4096).startswith("decode_kernel<16, 1, 8, 2, 4, ")
    assert w4a16.describe(32, 8192, 57344, swiglu=True).startswith(
        "decode_coop_kernel<32, 2, 4, 2, 16, true, false, false, 4> workgroups=224 threads=512 ks=1")
    assert w4a16.describe(32, 28672, 8192).startswith(
        "decode_coop_kernel<32, 1, 4, 2, 16, false, false, false, 4> workgroups=256 threads=512 ks=4")
    assert w4a16.describe(32, 4096, 28672, swiglu=True).startswith(
        "decode_coop_kernel<32, 2, 2, 4, 16, true, false, false, 4> workgroups=224 threads=512 ks=1")
    # Large batches: 128 x 512 tiles, the eight waves side by side.
    assert w4a16.describe(4096, 4096, 28672, swiglu=True).startswith(
        "prefill2_kernel<4, 1, 8, 2, false, true, false, false, 4> workgroups=1792 threads=512 ks=1")
    assert "prefill2_kernel<4, 1, 8, 2, false, true, true, false, 4>" in w4a16.describe(
        4096, 4096, 28672, swiglu=True, bf16=True)
    # Transition batches: the skinny-tile kernel (64-row tiles with four waves
    # along K up to M = 64, 128-row tiles with two above), K split only where
    # the tiles leave CUs idle; above M = 256 the prefill tiles.
    assert w4a16.describe(64, 4096, 28672, swiglu=True).startswith(
        "transition_kernel<2, 2, 4, true, false, false, 4> workgroups=224 threads=512 ks=1")
    assert w4a16.describe(256, 4096, 28672, swiglu=True).startswith(
        "transition_kernel<4, 4, 2, true, false, false, 4> workgroups=224 threads=512 ks=1")
    assert w4a16.describe(64, 14336, 4096).startswith(
        "transition_kernel<2, 2, 4, false, false, false, 4> workgroups=256 threads=512 ks=8; "
        "prefill_reduce_kernel<false, false>")
    # Where the 64-row grid exceeds one workgroup per CU but fits two: four-
    # wave workgroups, two per CU, no K split.
    assert w4a16.describe(100, 4096, 28672, swiglu=True).startswith(
        "transition_kernel<2, 2, 2, true, false, false, 4> workgroups=448 threads=256 ks=1")
    assert w4a16.describe(64, 8192, 57344).startswith(
        "transition_kernel<2, 2, 2, false, false, false, 4> workgroups=448 threads=256 ks=1")
    assert w4a16.describe(100, 4096, 28672, swiglu=True, zp=True).startswith(
        "transition_kernel<2, 2, 2, true, false, true, 4> workgroups=448 threads=256 ks=1")
    assert w4a16.describe(128, 4096, 28672, swiglu=True, int8=True).startswith(
        "transition_kernel<2, 2, 2, true, false, false, 8> workgroups=448 threads=256 ks=1")
    # INT8 and zero rows leave to the prefill tile a 64-row grid beyond two workgroups per CU.
    assert w4a16.describe(192, 4096, 28672, swiglu=True, int8=True).startswith("prefill2_kernel<")
    assert w4a16.describe(300, 4096, 28672, swiglu=True).startswith("prefill2_kernel<4, 1, 8, 2")
    assert w4a16.describe(33, 4096, 4096).startswith("transition_kernel<2, ")
    assert w4a16.describe(257, 4096, 4096).startswith("prefill2_kernel<")
    # Zero rows: both decode kernels scale before the MFMA (ZP instances),
    # prefill takes the ZP instance, the dense tier folds them into its dequant.
    d = w4a16.describe(1, 4096, 28672, swiglu=True, zp=True)
    assert d.startswith("decode_coop_kernel<16, 2, ") and d.split(">")[0].endswith(
        "true, false, true, 4"), d
    d = w4a16.describe(4, 4096, 4096, bf16=True, zp=True)
    assert d.startswith("decode_kernel<16, 1, ") and d.split(">")[0].endswith(
        "false, true, true, true, true, 4"), d
    # INT8 weights: the decode kernels' and the prefill kernel's 8-bit instances.
    d = w4a16.describe(1, 4096, 28672, swiglu=True, int8=True)
    assert d.startswith("decode_coop_kernel<16, 2, 1, 4, 1, true, false, false, 8>"), d
    d = w4a16.describe(3, 4096, 4096, bf16=True, int8=True)
    assert d.split(">")[0].endswith("false, true, true, false, true, 8"), d
    assert w4a16.describe(100, 4096, 4096, int8=True).startswith("transition_kernel<2, ")
    assert w4a16.describe(100, 4096, 4096, int8=True).split(">")[0].endswith(", 8")
    assert w4a16.describe(400, 4096, 4096, int8=True).startswith("prefill2_kernel<")
    assert w4a16.describe(100, 4096, 4096, path="dense", int8=True).startswith(
        "dequant8_kernel<false, false>; ")
    assert w4a16.select_path(100, 4096, 4096, int8=True) == "prefill"
    assert "prefill2_kernel<4, 1, 8, 2, false, false, false, true, 4>" in w4a16.describe(
        4096, 4096, 4096, zp=True)
    assert w4a16.describe(4096, 4096, 4096, path="dense", zp=True).startswith(
        "dequant_kernel<false, false>; prefill")
    assert w4a16.describe(64, 14336, 4096).endswith("ks=8; prefill_reduce_kernel<false, false>")
    assert w4a16.describe(4096, 4096, 4096, path="dense").startswith(
        "dequant_kernel<false, false>; ")
    assert w4a16.describe(4096, 4096, 4096, path="dense", bf16=True).startswith(
        "dequant_kernel<false, true>; ")
    assert "row slices" in w4a16.describe(100, 4096, 4096, path="decode")
    L = w4a16.lib()
    import ctypes
    buf = ctypes.create_string_buffer(8)
    assert L.w4a16_describe(1, 4096, 4096, 128, 0, ctypes.addressof(buf), 8) == 7   # truncated
    assert L.w4a16_describe(0, 4096, 4096, 128, 0, ctypes.addressof(buf), 8) == w4a16.ERR_INVALID
    assert L.w4a16_describe(1, 4096, 4096, 128, 0, 0, 8) == w4a16.ERR_INVALID


def test_forced_decode_slices_size_the_workspace_for_the_tail():
    """M > 32 on the forced decode path runs 32-row slices; the trailing
    M % 32 rows may take a split-K configuration that the full slices do
    not, and the workspace size covers it (M = 33: a one-row slice)."""
    need = w4a16.workspace_bytes(33, 8192, 6144, path="decode")
    tail = w4a16.workspace_bytes(1, 8192, 6144, path="decode")
    full = w4a16.workspace_bytes(32, 8192, 6144, path="decode")
    assert need == max(tail, full) and need > 0
    d = w4a16.describe(33, 8192, 6144, path="decode")
    assert "(x1 row slices of 32); last 1 rows: " in d, d


def test_decode_offsets_fall_back_to_prefill():
    """Shapes whose activation rows or strips exceed the decode kernels'
    32-bit offsets: the automatic path runs the prefill kernel instead and
    says so; a forced decode path is refused."""
    K = 1 << 27                     # 32 * K * 2 bytes of activations = 8 GiB
    assert w4a16.select_path(32, 4096, 4096) == "decode"
    assert w4a16.select_path(32, K, 64) == "prefill"
    d = w4a16.describe(32, K, 64)
    assert "(fallback decode-offsets:" in d, d
    L = w4a16.lib()
    import ctypes
    buf = ctypes.create_string_buffer(64)
    assert L.w4a16_describe(32, K, 64, 128, w4a16.PATH_DECODE, ctypes.addressof(buf),
                            64) == w4a16.ERR_UNSUPPORTED
    # M * K * 2 below 4 GiB at M = 1, and K * 16 below 4 GiB: still decode.
    assert w4a16.select_path(1, 1 << 27, 64) == "decode"
    assert w4a16.select_path(1, 1 << 28, 64) == "prefill"


def test_split_layout_on_the_library_workspace_and_its_size(monkeypatch):
    """Llama-8B O and down at M = 9-16 take two K splits (one strip per
    workgroup, eight waves along K) only where the launch finishes them
    itself; the workspace query covers both that launch and the one a
    caller's workspace gets (Llama-8B down at M = 16: two column groups, four
    splits, 1 MiB of partials)."""
    d = w4a16.describe(16, 4096, 4096)
    assert d.startswith("decode_coop_kernel<16, 1, 1, 8, 4, false, false, false, 4> "
                        "workgroups=256 threads=512 ks=2; K splits finished in the launch"), d
    d = w4a16.describe(9, 14336, 4096)
    assert d.startswith("decode_coop_kernel<16, 1, 1, 8, 4, false, false, false, 4> "
                        "workgroups=256 threads=512 ks=2; K splits finished in the launch"), d
    assert w4a16.workspace_bytes(16, 14336, 4096) == 128 * 4 * 16 * 32 * 4
    assert w4a16.workspace_bytes(16, 4096, 4096) == 128 * 2 * 16 * 32 * 4
    # With the reduction launch forced, the library workspace keeps the old layout.
    monkeypatch.setenv("W4A16_SPLIT_FINISH", "reduce")
    assert w4a16.describe(16, 4096, 4096).startswith(
        "decode_coop_kernel<16, 1, 1, 8, 4, false, false, false, 4> workgroups=128 "), d
    assert w4a16.describe(16, 14336, 4096).startswith(
        "decode_coop_kernel<16, 1, 2, 4, 4, false, false, false, 4> workgroups=256 "), d


def test_workspace_calls_without_gpu():
    """The workspace management calls report the HIP failure on a machine
    without a GPU instead of crashing."""
    import torch as T
    if T.cuda.is_available():
        pytest.skip("host-only check")
    assert w4a16.lib().w4a16_reserve_workspace(-1) == w4a16.ERR_INVALID
    assert w4a16.lib().w4a16_reserve_workspace(1024) == w4a16.ERR_HIP
    assert w4a16.last_fallback() == ""


def test_transition_stream_k_launch_and_workspace(monkeypatch):
    """W4A16_TRANSITION_SK=1: one workgroup per CU, each with an equal run of
    (tile, round) units; a tile's share of several workgroups goes to partial
    slices, so the workspace holds as many slices as the most workgroups that
    share a tile (transition_sk_reduce_kernel finishes them)."""
    monkeypatch.setenv("W4A16_TRANSITION_SK", "1")
    # 64 rows, 4096 x 28672: 224 tiles of 8 rounds = 1792 units, 7 per workgroup.
    d = w4a16.describe(64, 4096, 28672)
    assert d.startswith("transition_sk_kernel<2, 2, 4, false, false, false, 4> workgroups=256 "), d
    assert "stream-k units=1792 per_workgroup=7; transition_sk_reduce_kernel<false, false>" in d, d
    assert w4a16.workspace_bytes(64, 4096, 28672) == 2 * 64 * 28672 * 4
    # 260 tiles of 3 rounds, 4 units per workgroup: tiles shared by at most two.
    monkeypatch.setenv("W4A16_TRANSITION_MI", "2")
    d = w4a16.describe(256, 1152, 8320)
    assert "workgroups=195 " in d and "units=780 per_workgroup=4" in d, d
    assert w4a16.workspace_bytes(256, 1152, 8320) == 2 * 256 * 8320 * 4
    # Zero rows and INT8 weights keep the tiled form.
    assert w4a16.describe(64, 4096, 4096, zp=True).startswith("transition_kernel<")
    assert w4a16.describe(64, 4096, 4096, int8=True).startswith("transition_kernel<")
