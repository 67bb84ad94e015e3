"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic path), on sampled outputs the oracle computes one
by one: 256 sampled output columns (with the first and last 16), every row up
to M = 256, and for the prefill sizes rows 0-63, the last 64 rows and 128
seeded rows."""
import numpy as np
import pytest

from gpuhelp import gemm_case, sample_indices, say
from weight_only_int4_03_amd import synth, w4a16

pytestmark = pytest.mark.gpu

_cache = {}


def _weight(K, N):
    """Seeded W and its device weight, kept for the consecutive cases of one shape."""
    key = (K, N)
    if key not in _cache:
        _cache.clear()
        say("generating weight K=%d N=%d" % (K, N))
        W = synth.weights(K, N, seed=0)
        _cache[key] = (W, w4a16.load_weight(W))
    return _cache[key]


def _rows(M):
    if M <= 256:
        return None
    rng = np.random.default_rng(M)
    mid = rng.choice(np.arange(64, M - 64), 128, replace=False)
    return np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), mid]))


CASES = []
for name in ("gemv", "decode_8b", "decode_70b", "transition", "prefill", "fallback"):
    for label, M, K, N, sw, outl in sorted(synth.CONFIGS[name], key=lambda c: (c[2], c[3], c[1])):
        paths = ["auto"] if name != "fallback" else ["dense", "prefill"]
        for path in paths:
            CASES.append(pytest.param(M, K, N, sw, outl, path, id="%s-%s" % (label, path)))


@pytest.mark.parametrize("M,K,N,swiglu,outliers,path", CASES)
def test_config(M, K, N, swiglu, outliers, path):
    W, w = _weight(K, N)
    ncols = N // 2 if swiglu else N
    cols = sample_indices(ncols, 256, seed=K + N, edge=16)
    gemm_case(M, K, N, swiglu=swiglu, path=path, seed=0, outliers=outliers, cols=cols,
              rows=_rows(M), W=W, weight=w)


@pytest.mark.parametrize("M,K,N,density", [(1, 8192, 10240, 0.25), (4, 8192, 10240, 0.25),
                                           (16, 8192, 10240, 0.25), (32, 8192, 10240, 0.25),
                                           (32, 4096, 6144, 1.0), (32, 4096, 4096, 1.0),
                                           (32, 14336, 4096, 0.1), (1, 14336, 4096, 0.1)])
def test_config_integer_exact(M, K, N, density):
    """Integer-exact inputs (power-of-two scales, activations in {-1, 0, 1})
    at full projection sizes on the automatic path: the rotated K order of
    the Llama-70B QKV projection (strips 128 KiB apart), the eight-wave
    32-row layouts of the Llama-8B projections and the one-row LDS staging
    of the down projection.  Every partial sum is exact, so the sampled
    outputs must equal the oracle's bit for bit."""
    from gpuhelp import fp16_out, orc, to_dev
    d = w4a16.describe(M, K, N)
    say("integer-exact M=%d K=%d N=%d: %s" % (M, K, N, d))
    if K == 8192:
        assert " stagger" in d, d
    W = synth.grid_weights(K, N, p=4, seed=M + K)
    A = synth.ternary_activations(M, K, density=density, seed=M)
    out = fp16_out(w4a16.gemm(to_dev(A), w4a16.load_weight(W)))
    cols = sample_indices(N, 256, seed=K + N + M, edge=16)
    packed_o, s16_o = orc().quantize_pack(np.ascontiguousarray(W[:, cols]))
    C = orc().gemm_f64(A, packed_o, s16_o)
    assert np.abs(C).max() < 128, "inputs not fp16-exact"
    assert np.array_equal(out[:, cols].astype(np.float64), C), d
