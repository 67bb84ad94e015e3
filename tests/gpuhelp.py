"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding and the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import parity
from weight_only_int4_03_amd import synth, w4a16

_oracle = None


def orc():
    global _oracle
    if _oracle is None:
        _oracle = oracle.load()
    return _oracle


def torch():
    import torch as t
    if not t.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return t


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(x)).cuda()


def fp16_out(t) -> np.ndarray:
    return t.cpu().numpy().astype(np.float16)


def sample_indices(n: int, k: int, seed: int, edge: int = 0) -> np.ndarray:
    """Sorted sample of k indices of range(n), always with the first and last
    ``edge`` indices."""
    if n <= k + 2 * edge:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    base = set(range(min(edge, n))) | set(range(max(n - edge, 0), n))
    rest = np.setdiff1d(np.arange(n), np.array(sorted(base), dtype=np.int64))
    pick = rng.choice(rest, size=k, replace=False)
    return np.array(sorted(base | set(pick.tolist())), dtype=np.int64)


def gemm_case(M, K, N, swiglu=False, path="auto", seed=0, outliers=False, cols=None, rows=None,
              W=None, A=None, weight=None, bf16=False, G=128):
    """Run the GPU GEMM on seeded inputs and compare (sampled) outputs with
    the oracle's fp64 result.  Returns the comparison statistics.  With bf16,
    A (and the output) are bf16: A is given as uint16 bit patterns."""
    if bf16:
        return gemm_case_bf16(M, K, N, swiglu, path, seed, outliers, cols, rows, W, A, weight, G)
    say("case M=%d K=%d N=%d G=%d swiglu=%s path=%s seed=%d outliers=%s" %
        (M, K, N, G, swiglu, path, seed, outliers))
    t = torch()
    if W is None:
        W = synth.weights(K, N, seed)
    if A is None:
        A = synth.activations(M, K, seed, outliers)
    w = weight if weight is not None else w4a16.load_weight(W, G=G)
    out = fp16_out(w4a16.gemm(to_dev(A), w, swiglu=swiglu, path=path, G=G))
    t.cuda.synchronize()
    ncols = N // 2 if swiglu else N
    ocols = np.arange(ncols) if cols is None else np.asarray(cols)
    orows = np.arange(M) if rows is None else np.asarray(rows)
    wcols = np.concatenate([ocols, ocols + N // 2]) if swiglu else ocols
    o = orc()
    packed_o, s16_o = o.quantize_pack(np.ascontiguousarray(W[:, wcols]), G)
    C = o.gemm_f64(np.ascontiguousarray(A[orows]), packed_o, s16_o, G)
    ref = o.swiglu_f64(C) if swiglu else C
    stats = parity.assert_close(out[np.ix_(orows, ocols)], ref,
                                "M=%d K=%d N=%d swiglu=%s path=%s" % (M, K, N, swiglu, path))
    say("  ", {k: (round(v, 6) if isinstance(v, float) else v) for k, v in stats.items()})
    return stats


def bf16_dev(bits: np.ndarray):
    """uint16 bf16 bit patterns -> a bf16 device tensor."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(t.bfloat16)


def bf16_out(x) -> np.ndarray:
    t = torch()
    return x.view(t.int16).cpu().numpy().view(np.uint16)


def gemm_case_bf16(M, K, N, swiglu=False, path="auto", seed=0, outliers=False, cols=None,
                   rows=None, W=None, A=None, weight=None, G=128):
    say("case bf16 M=%d K=%d N=%d G=%d swiglu=%s path=%s seed=%d outliers=%s" %
        (M, K, N, G, swiglu, path, seed, outliers))
    t = torch()
    if W is None:
        W = synth.weights(K, N, seed)
    if A is None:
        A = synth.activations_bf16(M, K, seed, outliers)
    w = weight if weight is not None else w4a16.load_weight(W, G=G)
    out = bf16_out(w4a16.gemm(bf16_dev(A), w, swiglu=swiglu, path=path, G=G))
    t.cuda.synchronize()
    ncols = N // 2 if swiglu else N
    ocols = np.arange(ncols) if cols is None else np.asarray(cols)
    orows = np.arange(M) if rows is None else np.asarray(rows)
    wcols = np.concatenate([ocols, ocols + N // 2]) if swiglu else ocols
    o = orc()
    packed_o, s16_o = o.quantize_pack(np.ascontiguousarray(W[:, wcols]), G)
    C = o.gemm_bf16_f64(np.ascontiguousarray(A[orows]), packed_o, s16_o, G)
    ref = o.swiglu_f64(C) if swiglu else C
    stats = parity.assert_close_bf16(out[np.ix_(orows, ocols)], ref,
                                     "bf16 M=%d K=%d N=%d swiglu=%s path=%s" % (M, K, N, swiglu,
                                                                                path))
    say("  ", {k: (round(v, 6) if isinstance(v, float) else v) for k, v in stats.items()})
    return stats
