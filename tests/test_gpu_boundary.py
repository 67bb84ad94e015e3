"""The boundary's promises on the GPU: the GEMM calls never allocate under
stream capture (they refuse with W4A16_ERR_WORKSPACE until the workspace is
reserved, and a captured call then replays correctly), a fallback is reported
once per process, and a caller workspace sized by w4a16_gemm_workspace_bytes
suffices for every row slice of the forced decode path."""
import os
import subprocess
import sys

import numpy as np
import pytest

import parity
from gpuhelp import fp16_out, orc, sample_indices, say, to_dev, torch
from weight_only_int4_03_amd import synth, w4a16

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _raw_gemm(A, w, out, stream):
    """w4a16_gemm through the C ABI, returning its status code."""
    return w4a16.lib().w4a16_gemm(A.data_ptr(), A.shape[0], A.shape[1], w.rw.data_ptr(),
                                  w.rs.data_ptr(), w.N, w.G, out.data_ptr(), stream.cuda_stream)


def test_capture_refuses_to_allocate_then_replays_after_reserve():
    T = torch()
    M, K, N = 12, 14336, 1024           # the decode path splits K: it needs a workspace
    need = w4a16.workspace_bytes(M, K, N)
    assert need > 0
    say("capture M=%d K=%d N=%d workspace=%d" % (M, K, N, need))
    w4a16.release_workspace()
    assert w4a16.workspace_reserved() == 0
    W = synth.weights(K, N, seed=21)
    A = to_dev(synth.activations(M, K, seed=21))
    w = w4a16.load_weight(W)
    out = T.empty((M, N), dtype=T.float16, device="cuda")
    s = T.cuda.Stream()
    T.cuda.synchronize()
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g, stream=s):
        rc = _raw_gemm(A, w, out, s)
    assert rc == w4a16.ERR_WORKSPACE, rc
    assert "w4a16_reserve_workspace" in w4a16.last_error()
    assert w4a16.workspace_reserved() == 0      # nothing was allocated
    del g

    w4a16.reserve_workspace(need)
    assert w4a16.workspace_reserved() >= need
    eager = w4a16.gemm_plain(A, w)
    T.cuda.synchronize()
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g, stream=s):
        rc = _raw_gemm(A, w, out, s)
    assert rc == w4a16.OK, w4a16.last_error()
    ref = eager.cpu().numpy()
    other = to_dev(synth.activations(M, K, seed=22))
    for r in range(4):
        out.fill_(7.0)
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), ref.view(np.uint16)), r
        w4a16.gemm_plain(other, w)              # eager work between replays
        T.cuda.synchronize()
    # The replays match the oracle too.
    packed_o, s16_o = orc().quantize_pack(W)
    C = orc().gemm_f64(synth.activations(M, K, seed=21), packed_o, s16_o)
    parity.assert_close(out.cpu().numpy(), C, "captured decode M=%d" % M)


def test_captured_split_exchange_replays():
    """A decode GEMM whose two K splits exchange their partials inside the
    launch, captured in a HIP graph: every replay (with eager GEMMs of the
    same kind between them) equals the eager result bit for bit, so each
    call leaves the exchange slots clear for the next."""
    T = torch()
    M, K, N = 8, 14336, 4096
    desc = w4a16.describe(M, K, N)
    say("captured exchange:", desc)
    assert "finished in the launch (exchange)" in desc, desc
    w4a16.reserve_workspace(w4a16.workspace_bytes(M, K, N))
    W = synth.weights(K, N, seed=31)
    A = to_dev(synth.activations(M, K, seed=31))
    w = w4a16.load_weight(W)
    out = T.empty((M, N), dtype=T.float16, device="cuda")
    eager = w4a16.gemm_plain(A, w).cpu().numpy()
    s = T.cuda.Stream()
    T.cuda.synchronize()
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g, stream=s):
        rc = _raw_gemm(A, w, out, s)
    assert rc == w4a16.OK, w4a16.last_error()
    other = to_dev(synth.activations(M, K, seed=32))
    for r in range(4):
        out.fill_(7.0)
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager.view(np.uint16)), r
        w4a16.gemm_plain(other, w)
        T.cuda.synchronize()


def test_growth_outside_capture_keeps_earlier_results():
    """A larger call outside capture grows the workspace without
    synchronising or freeing: work queued on the old buffer stays valid."""
    T = torch()
    w4a16.release_workspace()
    K, N = 14336, 1024
    W = synth.weights(K, N, seed=23)
    w = w4a16.load_weight(W)
    packed_o, s16_o = orc().quantize_pack(W)
    outs = []
    for M in (8, 16, 64):                       # growing split-K partials
        A = synth.activations(M, K, seed=M)
        outs.append((M, A, w4a16.gemm(to_dev(A), w)))
    T.cuda.synchronize()
    for M, A, out in outs:
        C = orc().gemm_f64(A, packed_o, s16_o)
        parity.assert_close(fp16_out(out), C, "growth M=%d" % M)
    w4a16.release_workspace()


def test_fallback_is_reported_once():
    """Three prefill calls that take the one-wave fallback kernel (forced by
    W4A16_PREFILL_V2=0) write one stderr line, and the last fallback names
    it."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import torch\n"
        "from weight_only_int4_03_amd import synth, w4a16\n"
        "w = w4a16.load_weight(synth.weights(1024, 640, seed=1))\n"
        "A = torch.from_numpy(synth.activations(70, 1024, seed=1)).cuda()\n"
        "print('BEFORE', repr(w4a16.last_fallback()), flush=True)\n"
        "for _ in range(3):\n"
        "    w4a16.gemm(A, w, path='prefill')\n"
        "torch.cuda.synchronize()\n"
        "print('AFTER', w4a16.last_fallback(), flush=True)\n" % ROOT)
    env = dict(os.environ, W4A16_PREFILL_V2="0")
    say("fallback subprocess")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stderr.splitlines() if x.startswith("w4a16: fallback")]
    assert len(lines) == 1, r.stderr
    assert "prefill-one-wave" in lines[0] and "fused prefill" in lines[0], lines[0]
    assert "BEFORE ''" in r.stdout
    assert "AFTER fused prefill: prefill-one-wave" in r.stdout, r.stdout


@pytest.mark.parametrize("M", [33, 45, 70])
def test_forced_decode_row_slices_with_caller_workspace(M):
    """M > 32 on the forced decode path with a caller workspace of exactly
    w4a16_gemm_workspace_bytes: the trailing slice's configuration (M = 33:
    one row, split K) fits in it."""
    T = torch()
    K, N = 8192, 6144
    need = w4a16.workspace_bytes(M, K, N, path="decode")
    say("forced decode M=%d K=%d N=%d workspace=%d: %s" % (M, K, N, need,
                                                           w4a16.describe(M, K, N, path="decode")))
    W = synth.weights(K, N, seed=M)
    A = synth.activations(M, K, seed=M)
    w = w4a16.load_weight(W)
    ws = T.empty(max(need, 1), dtype=T.uint8, device="cuda")
    out = fp16_out(w4a16.gemm(to_dev(A), w, path="decode", workspace=ws))
    T.cuda.synchronize()
    cols = sample_indices(N, 384, seed=M, edge=32)
    packed_o, s16_o = orc().quantize_pack(np.ascontiguousarray(W[:, cols]))
    C = orc().gemm_f64(A, packed_o, s16_o)
    parity.assert_close(out[:, cols], C, "forced decode M=%d" % M)
