"""w4a16_gemm_noalloc (the split-K partials in the library's fixed per-GPU
scratch, no allocation) against w4a16_gemm_ex, through the C ABI.  On the
library's workspace (workspace NULL) the two run the same kernels in the same
order, so the outputs agree bit for bit; with a caller's workspace too, except
where the library's layout takes two K splits that only it finishes inside
the launch (narrow plain projections at M = 9-16), where the caller's layout
sums in another FP32 order.  Two calls in a row, the second with a smaller
input (the scratch keeps the first call's contents), and a problem too large
for the scratch."""
import numpy as np
import pytest

from gpuhelp import say, to_dev, torch
from weight_only_int4_03_amd import synth, w4a16

pytestmark = pytest.mark.gpu


def _ex(A, w, swiglu):
    T = torch()
    need = w4a16.workspace_bytes(A.shape[0], w.K, w.N, swiglu)
    ws = T.empty(max(need, 256), dtype=T.uint8, device="cuda")
    return w4a16.gemm(A, w, swiglu=swiglu, workspace=ws)


def _bits(t):
    T = torch()
    return t.view(T.int16).cpu().numpy()


@pytest.mark.parametrize("K,N,swiglu,ms", [(14336, 4096, False, (64, 8)),
                                           (4096, 28672, True, (70, 5)),
                                           (8192, 8192, False, (32, 1)),
                                           (14336, 4096, False, (16, 9))])
def test_noalloc_matches_gemm_ex(K, N, swiglu, ms):
    T = torch()
    say("noalloc K=%d N=%d swiglu=%s Ms=%s" % (K, N, swiglu, ms))
    assert w4a16.lib().w4a16_noalloc_scratch_bytes() == 64 << 20
    w = w4a16.load_weight(synth.weights(K, N, seed=K + N))
    for M in ms:                                  # the second call is smaller
        need = w4a16.workspace_bytes(M, K, N, swiglu)
        desc = w4a16.describe(M, K, N, swiglu)
        say("  M=%d workspace=%d %s" % (M, need, desc))
        assert need <= 64 << 20
        A = to_dev(synth.activations(M, K, seed=M))
        got = w4a16.gemm_noalloc(A, w, swiglu=swiglu)
        own = w4a16.gemm(A, w, swiglu=swiglu)
        caller = _ex(A, w, swiglu)
        T.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(own)), M
        if desc.startswith("decode_coop_kernel<16, 1, 1, 8, 4, ") and "ks=2; K splits finished" in desc:
            g = got.float().cpu().numpy()
            c = caller.float().cpu().numpy()
            assert np.allclose(g, c, rtol=2.0 ** -9, atol=1e-3), M
        else:
            assert np.array_equal(_bits(got), _bits(caller)), M


def test_noalloc_bf16_and_forced_paths():
    T = torch()
    K, N = 14336, 1024
    w = w4a16.load_weight(synth.weights(K, N, seed=3))
    for M, path in ((130, "prefill"), (12, "decode"), (40, "decode")):
        say("noalloc bf16 M=%d path=%s" % (M, path))
        A = to_dev(synth.activations_bf16(M, K, seed=M).view(np.int16)).view(T.bfloat16)
        got = w4a16.gemm_noalloc(A, w, path=path)
        need = w4a16.workspace_bytes(M, K, N, path=path, bf16=True)
        ws = T.empty(max(need, 256), dtype=T.uint8, device="cuda")
        want = w4a16.gemm(A, w, path=path, workspace=ws)
        own = w4a16.gemm(A, w, path=path)
        T.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(want)), (M, path)
        assert np.array_equal(_bits(got), _bits(own)), (M, path)


def test_noalloc_refuses_beyond_its_scratch():
    T = torch()
    K, N, M = 8192, 8192, 64                      # dense tier: 128 MiB of fp16 weights
    need = w4a16.workspace_bytes(M, K, N, path="dense")
    assert need > 64 << 20
    w = w4a16.load_weight(synth.weights(K, N, seed=9))
    A = to_dev(synth.activations(M, K, seed=9))
    out = T.full((M, N), 3.0, dtype=T.float16, device="cuda")
    rc = w4a16.lib().w4a16_gemm_noalloc(A.data_ptr(), M, K, w.rw.data_ptr(), w.rs.data_ptr(), N,
                                        128, out.data_ptr(), w4a16.PATH_DENSE,
                                        T.cuda.current_stream().cuda_stream)
    assert rc == w4a16.ERR_WORKSPACE
    assert "scratch" in w4a16.last_error()
    T.cuda.synchronize()
    assert bool((out == 3.0).all())               # nothing was launched
