#!/usr/bin/env python3
"""W4A16 GEMM benchmark on one MI355X.

The default run covers both halves of the metric in one JSON line:
  * the decode step (the line's ``value``): the Llama-8B-shaped decode
    projections QKV, O, fused gate/up with SwiGLU, and down at M = 1, 8, 16
    and 32 (16 GEMMs), HBM-bound, reported in GB/s of algorithmic bytes;
  * the prefill GEMMs (``prefill``): gate/up + SwiGLU and down at
    M = 4096 and 8191, MFMA-bound, reported in TFLOP/s.
Every GEMM runs the library's automatic path through the C ABI, with its
inputs resident in HBM before timing starts.  Other workloads (``--workload``):
gemv, llama70b_decode, transition, prefill, and fallback (the fused prefill
kernel and the dequantize-then-dense tier side by side at M = 16384).

Cold weights: each "layer slot" of a step uses its own copy of the
projection weights, rotating over enough copies that the data touched
between two uses of one copy exceeds 800 MB (three times the 256 MB
memory-side cache plus the L2s), so every weight byte comes from HBM.

Timing (HIP events on the stream the kernels run on):
  * the step: each step of the rotation is captured in a HIP graph (for
    workloads of fewer than 16 GEMMs, runs of consecutive steps share one
    graph so that graph launches do not dominate); W warm-up steps, then
    exactly K timed steps between two synchronisations;
  * per GEMM: a HIP graph of one launch per weight copy, replayed between two
    events (median of three trials); the kernel behind the largest share of
    the step time gives the roofline entry (algorithmic bytes = K*N/2 +
    2*(K/G)*N + 2*M*K + 2*M*N_out, FLOPs = 2*M*N*K);
  * per GEMM floor, measured in the same run: for HBM-bound GEMMs the
    library's streaming-read probe reading that GEMM's algorithmic byte count
    under the same cold rotation (what launch, first-load latency and drain
    leave of the bandwidth at that size); for MFMA-bound GEMMs the GEMM's
    FLOPs at the measured MFMA-loop rate.

Ceilings: the library's probe kernels measure the GPU's own streaming-read
rate and fp16 MFMA rate; each roofline entry gives the fraction of both the
data-sheet peak and the measured ceiling; clock levels and board power are
read from sysfs after the timing.

The CPU baseline times the oracle (test infrastructure) on the host: its
quantize+pack and dequantization (single-threaded loops) on one projection,
and its fp64 GEMM on a column sample of the decode step's GEMMs and a 256-row
slice of the prefill GEMMs (extrapolated to all rows), single-threaded and on
all cores.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from weight_only_int4_03_amd import synth, w4a16  # noqa: E402

METRIC = ("W4A16 GEMM µs + achieved HBM GB/s (M≤32) / TFLOP/s (M≥4096) "
          "vs roofline")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
ROTATE_BYTES = 800e6
G = 128
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(M, K, N, swiglu, zp=False, int8=False):
    """Bytes a GEMM must move at least once: packed weights (half a byte per
    INT4 weight, one per INT8 weight), scales (and zero rows), activations,
    output."""
    n_out = N // 2 if swiglu else N
    wbytes = K * N if int8 else K * N // 2
    return wbytes + 2 * (K // G) * N * (2 if zp else 1) + 2 * M * K + 2 * M * n_out


def flops(M, K, N):
    return 2 * M * N * K


# Workloads: name -> (description, units).  A unit is (label, M, K, N, swiglu,
# outliers, slot, path); units sharing a slot use the same copy of their
# weights.
def workloads():
    def decode(model, shapes, ms):
        units = []
        for mi, m in enumerate(ms):
            for p, (k, n, sw) in shapes.items():
                units.append(("%s_%s_m%d" % (model, p, m), m, k, n, sw, False, mi, "auto"))
        return units

    def listed(name, path="auto"):
        return [(l, m, k, n, sw, o, i, path) for i, (l, m, k, n, sw, o)
                in enumerate(synth.CONFIGS[name])]

    fallback = []
    for i, (l, m, k, n, sw, o) in enumerate(synth.CONFIGS["fallback"]):
        fallback.append((l + "_fused", m, k, n, sw, o, i, "prefill"))
        fallback.append((l + "_dense", m, k, n, sw, o, i, "dense"))
    return {
        "llama8b_decode": ("Llama-8B-shaped decode projections (QKV 4096x6144, O 4096x4096, "
                           "gate/up 4096x28672 + SwiGLU, down 14336x4096) at M = 1, 8, 16, 32",
                           decode("8b", synth.LLAMA_8B, (1, 8, 16, 32))),
        "gemv": ("single GEMV M=1 K=4096 N=4096",
                 [("gemv", 1, 4096, 4096, False, False, 0, "auto")]),
        "llama70b_decode": ("Llama-70B-shaped decode projections at M = 1, 4, 16, 32",
                            decode("70b", synth.LLAMA_70B, (1, 4, 16, 32))),
        "transition": ("transition batches M = 64, 128, 256 with 1% outlier channels",
                       listed("transition")),
        "prefill": ("prefill M = 4096, 8191: gate/up 4096x28672 + SwiGLU, down 14336x4096",
                    listed("prefill")),
        "fallback": ("M = 16384, gate/up 4096x28672 + SwiGLU and down 14336x4096: the fused "
                     "prefill kernel and the dense tier (dequantize, then dense fp16 GEMM)",
                     fallback),
    }


# The default run: the decode step (the line's value) and the prefill GEMMs.
DEFAULT_PARTS = ("llama8b_decode", "prefill")


def kernel_key(M, K, N, swiglu, bf16=False, zp=False, int8=False, path="auto"):
    """The kernel instance a GEMM launches, as the profiler names it, marked
    when a second (split-K reduction) launch follows it."""
    desc = w4a16.describe(M, K, N, swiglu, path=path, bf16=bf16, zp=zp, int8=int8)
    first = desc.split(";")[0]
    name = first.split(" workgroups=")[0].strip()
    if first.startswith("dequant"):
        name = desc.split(";")[1].split(" workgroups=")[0].strip()
        return name + " (dense tier)"
    return name + (" + reduce" if "reduce_kernel" in desc else "")


# HIP sources that define each kernel family (the digest of stored counters
# covers these; a kernel of no listed family is covered by every source).
KERNEL_SOURCES = {
    "decode": ("common.h", "decode.hip", "decode_args.h", "decode_coop.hip"),
    "prefill": ("common.h", "prefill.hip"),
    "transition": ("common.h", "transition.hip"),
}


def source_digest(kernel=None):
    """Digest of the HIP sources that define ``kernel``, to tell whether
    stored counters still apply."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_int4_03_amd", "csrc")
    fam = next((f for f in KERNEL_SOURCES if kernel and kernel.startswith(f)), None)
    for f in (KERNEL_SOURCES[fam] if fam else sorted(os.listdir(csrc))):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources, for this workload and kernel."""
    path = os.path.join(PROFILES, "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_]+)\s*=\s*(.+?)\s*$", line)
        if m:
            vals[m.group(1)] = m.group(2)
    if (vals.get("source_digest") != source_digest(kernel) or vals.get("workload") != workload
            or vals.get("kernel") != kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# CPU baseline (the oracle).

def host_info():
    info = {"nproc": os.cpu_count()}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return info


def _gemm_sample(o, units, host_w, frac, nthreads, bf16, host_zp, int8, rows=None):
    """Oracle fp64 GEMM (+ SwiGLU) on the first `frac` of each unit's output
    columns (all rows, or the first `rows` rows): (seconds, bytes, flops,
    columns per unit)."""
    done_bytes = done_flops = 0
    elapsed, cols = 0.0, []
    for label, M, K, N, sw, outl, *_ in units:
        ncols = N // 2 if sw else N
        ns = min(ncols, max(32, int(round(ncols * frac / 32)) * 32))
        W = host_w[(K, N)] if (K, N) in host_w else synth.weights(K, N, seed=0)
        Ws = np.concatenate([W[:, :ns], W[:, N // 2:N // 2 + ns]], axis=1) if sw else W[:, :ns]
        packed, s16 = (o.quantize_pack8 if int8 else o.quantize_pack)(np.ascontiguousarray(Ws))
        m = M if rows is None else min(M, rows)
        A = (synth.activations_bf16 if bf16 else synth.activations)(M, K, seed=0, outliers=outl)
        A = np.ascontiguousarray(A[:m])
        if host_zp is not None:
            Z = host_zp[(K, N)]
            Zs = np.concatenate([Z[:, :ns], Z[:, N // 2:N // 2 + ns]], axis=1) if sw else Z[:, :ns]
            z16 = o.zero_rows(s16, np.ascontiguousarray(Zs))
        t0 = time.perf_counter()
        if host_zp is not None:
            Wz = o.dequant_zp(packed, s16, z16, bf16=bf16)
            C = (o.gemm_wb_f64 if bf16 else o.gemm_w16_f64)(A, Wz, nthreads=nthreads)
        elif int8:
            C = o.gemm8_f64(A, packed, s16, bf16=bf16, nthreads=nthreads)
        else:
            C = (o.gemm_bf16_f64 if bf16 else o.gemm_f64)(A, packed, s16, nthreads=nthreads)
        if sw:
            o.swiglu_f64(C)
        elapsed += time.perf_counter() - t0
        done_bytes += alg_bytes(m, K, Ws.shape[1], sw, host_zp is not None, int8)
        done_flops += flops(m, K, Ws.shape[1])
        cols.append(ns)
    return elapsed, done_bytes, done_flops, cols


def cpu_baseline(decode_units, host_w, prefill_units=None, target_s=5.0, bf16=False,
                 host_zp=None, int8=False):
    """Time the oracle on the host (host_w: the same seeded fp32 weights the
    GPU was given, keyed by (K, N)).  ``value`` is the all-core fp64 GEMM
    rate on the decode GEMMs' column sample, in GB/s of algorithmic bytes."""
    import oracle
    o = oracle.load()
    threads = o.max_threads()
    out = {"unit": "GB/s", "cores": threads, "kind": "oracle", "host": host_info()}

    # Quantize + pack and dequantize (the oracle's single-threaded loops) on
    # one 4096 x 4096 projection.
    K, N = 4096, 4096
    W = host_w.get((K, N))
    if W is None:
        W = synth.weights(K, N, seed=0)
    t0 = time.perf_counter()
    packed, s16 = (o.quantize_pack8 if int8 else o.quantize_pack)(W)
    t_pack = time.perf_counter() - t0
    t0 = time.perf_counter()
    (o.dequant8 if int8 else o.dequant)(packed, s16)
    t_deq = time.perf_counter() - t0
    wbytes = K * N if int8 else K * N // 2
    detail = {
        "pack": {"shape": "%dx%d" % (K, N), "threads": 1, "us": round(t_pack * 1e6, 1),
                 "GB/s": round((4 * K * N + wbytes + 2 * (K // G) * N) / t_pack / 1e9, 4),
                 "bytes": "fp32 W read, packed words and fp16 scales written"},
        "dequant": {"shape": "%dx%d" % (K, N), "threads": 1, "us": round(t_deq * 1e6, 1),
                    "GB/s": round((wbytes + 2 * (K // G) * N + 2 * K * N) / t_deq / 1e9, 4),
                    "bytes": "packed words and scales read, fp16 weights written"},
    }

    # The fp64 GEMM on a column sample of the decode GEMMs: calibrate the
    # single-thread rate, then size each sample to about target_s seconds.
    total_mac = sum(u[1] * u[2] * u[3] for u in decode_units)
    Wc = synth.weights(4096, 1024, seed=5)
    pc, sc = o.quantize_pack(Wc)
    Ac = synth.activations(8, 4096, seed=5)
    t0 = time.perf_counter()
    o.gemm_f64(Ac, pc, sc, nthreads=1)
    rate1 = 8 * 4096 * 1024 / max(time.perf_counter() - t0, 1e-6)
    fracs = {}
    for nthr, key in ((1, "gemm_1thread"), (threads, "gemm_all")):
        frac = min(1.0, max(target_s * rate1 * (1 if nthr == 1 else 0.7 * nthr) / total_mac,
                            1.0 / 256))
        fracs[key] = frac
        t, by, fl, cols = _gemm_sample(o, decode_units, host_w, frac, nthr, bf16, host_zp, int8)
        detail[key] = {"threads": nthr, "s": round(t, 2), "GB/s": round(by / t / 1e9, 4),
                       "GFLOP/s": round(fl / t / 1e9, 3),
                       "sample": "first %.2f%% of output columns of each of the %d GEMMs "
                                 "(all rows, full K)" % (100 * frac, len(decode_units))}
    out["value"] = detail["gemm_all"]["GB/s"]
    out["sample"] = ("fp64 oracle GEMM (+SwiGLU) on the first %.2f%% of output columns of each "
                     "of the %d GEMMs (all rows, full K), %.1f s on %d threads; pack, dequant "
                     "and the single-thread GEMM in 'detail'"
                     % (100 * fracs["gemm_all"], len(decode_units), detail["gemm_all"]["s"],
                        threads))

    if prefill_units:
        # A 256-row slice of each prefill GEMM on a column sample,
        # extrapolated to all rows and columns.
        pmac = sum(256 * u[2] * u[3] for u in prefill_units)
        for nthr, key in ((1, "prefill_gemm_1thread"), (threads, "prefill_gemm_all")):
            frac = min(1.0, max(target_s * rate1 * (1 if nthr == 1 else 0.7 * nthr) / pmac,
                                1.0 / 512))
            t, by, fl, cols = _gemm_sample(o, prefill_units, host_w, frac, nthr, bf16, host_zp,
                                           int8, rows=256)
            detail[key] = {"threads": nthr, "s": round(t, 2),
                           "TFLOP/s": round(fl / t / 1e12, 6),
                           "extrapolated": True,
                           "sample": "rows 0-255 and the first %.2f%% of output columns of each "
                                     "of the %d prefill GEMMs; the rate applies to all M rows "
                                     "(row-independent work)" % (100 * frac, len(prefill_units))}
    out["detail"] = detail
    return out


# ---------------------------------------------------------------------------
# GPU measurements.

def measure_ceilings(stream, torch, dev):
    """The GPU's own ceilings, from the library's probe kernels: a streaming
    read of two alternating 1 GiB buffers (each read exceeds the memory-side
    cache) and a register-only fp16 MFMA loop with two waves per SIMD."""
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    bufs = [torch.ones(1 << 28, dtype=torch.int32, device=dev) for _ in range(2)]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    reps = 10
    with torch.cuda.stream(stream):
        for b in bufs:
            w4a16.probe_stream_read(b, sink, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            w4a16.probe_stream_read(bufs[i % 2], sink, stream)
        b.record(stream)
    torch.cuda.synchronize()
    read_gbs = reps * (1 << 30) / (a.elapsed_time(b) * 1e-3) / 1e9
    del bufs
    iters = 8192
    with torch.cuda.stream(stream):
        w4a16.probe_mfma(64, 2 * cus, sink, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fl = 0
        for _ in range(3):
            fl += w4a16.probe_mfma(iters, 2 * cus, sink, stream)
        b.record(stream)
    torch.cuda.synchronize()
    mfma_tf = fl / (a.elapsed_time(b) * 1e-3) / 1e12
    return {"stream_read_GBs": round(read_gbs, 1), "mfma_f16_TFLOPs": round(mfma_tf, 1),
            "how": "w4a16_probe_stream_read over 2 x 1 GiB alternating (10 reads); "
                   "w4a16_probe_mfma %d workgroups x 4 waves, %d rounds of 4 MFMA 32x32x16 f16"
                   % (2 * cus, iters)}


def time_graph(torch, stream, build, reps):
    """Median of three trials of `reps` replays of the graph `build` records
    (after three warm-up replays), in ms per replay."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        build()
    trials = []
    with torch.cuda.stream(stream):
        for _ in range(3):
            g.replay()
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            trials.append((a, b))
    torch.cuda.synchronize()
    del g
    return sorted(a.elapsed_time(b) for a, b in trials)[1] / reps


def read_floors(torch, stream, dev, sizes, reps):
    """Streaming-read floor per byte count: the probe reading `bytes` bytes,
    one launch per slice of a rotating pool (at least 800 MB between reuses of
    a slice, as for the GEMMs' weight copies), in microseconds per launch."""
    pool_bytes = 1 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev)
    pool.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    out = {}
    for nbytes in sorted(set(sizes)):
        B = (nbytes + 255) // 256 * 256
        n = max(2, math.ceil(ROTATE_BYTES / B))
        slots = max(1, (pool_bytes - B) // B + 1)
        views = [pool[(i % slots) * B:(i % slots) * B + B] for i in range(n)]

        def build():
            for v in views:
                w4a16.probe_stream_read(v, sink, stream)
        out[nbytes] = time_graph(torch, stream, build, reps) * 1e3 / n
    del pool
    return out


def run_workload(name, args, torch, dev, stream, zp, int8, bf16):
    """Weights, step timing and per-GEMM timing of one workload."""
    desc, units = workloads()[name]
    nslots = max(u[6] for u in units) + 1

    # Weights: one seeded W per distinct projection, quantized, packed and
    # repacked on the device, then cloned into rotation copies.
    shapes = sorted({(u[2], u[3]) for u in units})
    base, host_w, host_zp = {}, {}, ({} if zp else None)
    for (k, n) in shapes:
        log("weights K=%d N=%d" % (k, n))
        host_w[(k, n)] = synth.weights(k, n, seed=0)
        base[(k, n)] = (w4a16.load_weight_int8 if int8 else w4a16.load_weight)(host_w[(k, n)])
        if zp:
            host_zp[(k, n)] = synth.zero_points(k // G, n, seed=0)
            _, scales = w4a16.unrepack(base[(k, n)])
            base[(k, n)] = w4a16.zero_rows(base[(k, n)], scales,
                                           torch.from_numpy(host_zp[(k, n)]).to(dev))
    torch.cuda.synchronize()
    slot_bytes = [sum(base[(u[2], u[3])].nbytes for u in units if u[6] == slot)
                  for slot in range(nslots)]
    per_slot = max(slot_bytes)
    ncopies = max(2, math.ceil(ROTATE_BYTES / per_slot)) if per_slot < ROTATE_BYTES else 2
    copies = {key: [w] + [w.clone() for _ in range(ncopies - 1)] for key, w in base.items()}
    log("rotation: %d copies of %.1f MB per slot" % (ncopies, per_slot / 1e6))

    act_dtype = torch.bfloat16 if bf16 else torch.float16
    acts = {}
    for u in units:
        m, k, outl = u[1], u[2], u[5]
        if (m, k, outl) not in acts:
            if bf16:
                bits = synth.activations_bf16(m, k, seed=0, outliers=outl)
                acts[(m, k, outl)] = torch.from_numpy(bits.view(np.int16)).to(dev).view(
                    torch.bfloat16)
            else:
                acts[(m, k, outl)] = torch.from_numpy(
                    synth.activations(m, k, seed=0, outliers=outl)).to(dev)
    outs = {u[0]: torch.empty((u[1], u[3] // 2 if u[4] else u[3]), dtype=act_dtype, device=dev)
            for u in units}

    def run_unit(u, copy):
        label, m, k, n, sw, outl, _, path = u
        w = copies[(k, n)][copy]
        A = acts[(m, k, outl)]
        if zp or int8 or bf16 or path != "auto":
            w4a16.gemm(A, w, swiglu=sw, out=outs[label], path=path)
        elif sw:
            w4a16.gemm_swiglu(A, w, out=outs[label])
        else:
            w4a16.gemm_plain(A, w, out=outs[label])

    # Rotation: step s, slot t uses copy (s * nslots + t) % ncopies; the
    # pattern repeats every `period` steps, one graph per step of the period.
    period = ncopies // math.gcd(ncopies, nslots)

    def step_copy(s, slot):
        return (s * nslots + slot) % ncopies

    # The library workspace is sized before any capture (a GEMM under stream
    # capture does not allocate).
    need = max(w4a16.workspace_bytes(u[1], u[2], u[3], u[4], path=u[7], bf16=bf16, zp=zp,
                                     int8=int8) for u in units)
    w4a16.reserve_workspace(need)
    with torch.cuda.stream(stream):
        for s in range(period):
            for u in units:
                run_unit(u, step_copy(s, u[6]))
    torch.cuda.synchronize()

    # Graphs: one per step of the rotation period, and, for workloads of few
    # GEMMs, graphs of `spg` consecutive steps (at least 16 launches each) so
    # that graph-launch overhead does not dominate the step.
    spg = max(1, math.ceil(16 / len(units)))

    def capture(first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s in range(first, first + count):
                for u in units:
                    run_unit(u, step_copy(s % period, u[6]))
        return g

    graphs = [capture(s, 1) for s in range(period)]
    multi = {}
    if spg > 1:
        for s in range(0, period * spg, spg):
            multi.setdefault(s % period, capture(s % period, spg))
    torch.cuda.synchronize()

    def replay_steps(first, count):
        s = first
        while s < first + count:
            if spg > 1 and first + count - s >= spg and (s % period) in multi:
                multi[s % period].replay()
                s += spg
            else:
                graphs[s % period].replay()
                s += 1

    steps = args.steps if args.steps is not None else (200 if name != "fallback" else 20)
    warmup = args.warmup if args.warmup is not None else (20 if name != "fallback" else 3)
    with torch.cuda.stream(stream):
        replay_steps(0, warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        replay_steps(warmup, steps)
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / steps
    step_bytes = sum(alg_bytes(u[1], u[2], u[3], u[4], zp, int8) for u in units)
    step_flops = sum(flops(u[1], u[2], u[3]) for u in units)
    log("%s step: %.2f us (wall %.2f us), %.1f MB, %.2f GFLOP"
        % (name, ms_step * 1e3, wall / steps * 1e6, step_bytes / 1e6, step_flops / 1e9))
    del graphs, multi

    # Per-GEMM timing: a graph of one launch per weight copy (all cold).
    detail = []
    for u in units:
        label, m, k, n, sw, outl, slot, path = u
        reps = args.reps if m < 4096 else max(2, args.reps // 4)
        us = time_graph(torch, stream, lambda: [run_unit(u, c) for c in range(ncopies)],
                        reps) * 1e3 / ncopies
        by, fl = alg_bytes(m, k, n, sw, zp, int8), flops(m, k, n)
        detail.append({"gemm": label, "M": m, "K": k, "N": n, "swiglu": sw, "path": path,
                       "kernel": kernel_key(m, k, n, sw, bf16, zp, int8, path),
                       "launch": w4a16.describe(m, k, n, sw, path=path, bf16=bf16, zp=zp,
                                                int8=int8),
                       "us": round(us, 3),
                       "GB/s": round(by / us / 1e3, 1), "TFLOP/s": round(fl / us / 1e6, 2),
                       "hbm_frac": round(by / us / 1e3 / HBM_PEAK_GBS, 4),
                       "mfma_frac": round(fl / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)})
        log("  %-26s %-52s %9.2f us %8.1f GB/s %8.2f TFLOP/s" %
            (label, detail[-1]["kernel"][:52], us, detail[-1]["GB/s"], detail[-1]["TFLOP/s"]))
        if args.comparator and m >= 64 and not (zp or int8 or bf16):
            # External comparator: the vendor's dense fp16 GEMM (torch.matmul,
            # hipBLASLt) on the dequantized weights of the same shape, without
            # the epilogue, with its own cold rotation of fp16 weight copies.
            W16 = w4a16.dequant(copies[(k, n)][0])
            nd = max(2, math.ceil(ROTATE_BYTES / W16.nbytes))
            dense = [W16] + [W16.clone() for _ in range(nd - 1)]
            A = acts[(m, k, outl)]
            C = torch.empty((m, n), dtype=torch.float16, device=dev)
            torch.matmul(A, dense[0], out=C)
            torch.cuda.synchronize()
            # Timed eagerly (launches queue ahead of the GPU), median of three.
            trials = []
            with torch.cuda.stream(stream):
                for d in dense:
                    torch.matmul(A, d, out=C)
                for _ in range(3):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(reps):
                        for d in dense:
                            torch.matmul(A, d, out=C)
                    b.record(stream)
                    trials.append((a, b))
            torch.cuda.synchronize()
            cus = sorted(a.elapsed_time(b) for a, b in trials)[1] * 1e3 / (reps * nd)
            detail[-1]["comparator"] = {"what": "torch.matmul fp16 dense (hipBLASLt), same shape, "
                                                "no epilogue, %d cold weight copies, eager "
                                                "launches" % nd,
                                        "us": round(cus, 3),
                                        "TFLOP/s": round(fl / cus / 1e6, 2)}
            log("  %-26s %-52s %9.2f us %8.2f TFLOP/s" % ("", "comparator: torch.matmul fp16",
                                                         cus, fl / cus / 1e6))
            del dense, W16, C
    result = {"name": name, "desc": desc, "units": units, "host_w": host_w, "host_zp": host_zp,
              "ms_step": ms_step, "steps": steps, "warmup": warmup, "spg": spg,
              "step_bytes": step_bytes, "step_flops": step_flops, "ncopies": ncopies,
              "detail": detail}
    del copies, base, acts, outs
    torch.cuda.synchronize()
    return result


def roofline_entry(res, ceilings, zp, int8, suffix):
    """The dominant kernel's entry: the kernel instance with the largest share
    of the per-GEMM times; HBM-bound (GB/s) if all its GEMMs have M <= 256,
    else MFMA-bound (TFLOP/s)."""
    by_kernel = {}
    for d in res["detail"]:
        e = by_kernel.setdefault(d["kernel"], {"us": 0.0, "bytes": 0, "flops": 0, "launches": 0})
        e["us"] += d["us"]
        e["bytes"] += alg_bytes(d["M"], d["K"], d["N"], d["swiglu"], zp, int8)
        e["flops"] += flops(d["M"], d["K"], d["N"])
        e["launches"] += 1
    dom = max(by_kernel, key=lambda k: by_kernel[k]["us"])
    e = by_kernel[dom]
    hbm_bound = all(d["M"] <= 64 for d in res["detail"] if d["kernel"] == dom)
    if hbm_bound:
        achieved = e["bytes"] / e["us"] / 1e3
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        ceiling = ceilings["stream_read_GBs"]
    else:
        achieved = e["flops"] / e["us"] / 1e6
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4)}
        ceiling = ceilings["mfma_f16_TFLOPs"]
    roof["frac_of_measured_ceiling"] = round(achieved / ceiling, 4) if ceiling else None
    kname = dom.split(" (")[0].replace(" + reduce", "")
    roof["traffic"] = stored_traffic(res["name"] + suffix, kname)
    roof["kernel"] = dom
    roof["launch_workgroups"] = sorted({int(re.search(r"workgroups=(\d+)", d["launch"]).group(1))
                                        for d in res["detail"] if d["kernel"] == dom})
    roof["launches_per_step"] = e["launches"]
    roof["avg_launch_us"] = round(e["us"] / e["launches"], 3)
    roof["alg_bytes_per_launch"] = round(e["bytes"] / e["launches"])
    roof["alg_flops_per_launch"] = round(e["flops"] / e["launches"])
    return roof


# Dispatch sweeps (--sweep NAME): GEMM shapes timed under launch-configuration
# variants (the environment overrides the library reads at every call), each
# variant's output compared with the first's.  Two passes (forward, then
# reverse order) and the better of the two kept, so the first variant timed
# after a weight change is not favoured or penalised.
SWEEPS = {
    "transition": {
        "what": "the transition kernel against the 1 x 8 prefill tile it replaced, its "
                "four-wave tiles and its Stream-K form (1% outlier activations; Llama-8B gate/up "
                "and down, Llama-70B gate/up)",
        "shapes": [(m, 4096, 28672, False) for m in (48, 64, 96, 128, 192, 256, 384)]
                  + [(m, 14336, 4096, False) for m in (48, 64, 96, 128, 192, 256, 384)]
                  + [(m, 8192, 57344, False) for m in (48, 64, 128)],
        "outliers": True,
        "variants": [("prefill tile", {"W4A16_TRANSITION": "0"}),
                     ("transition (automatic)", {"W4A16_TRANSITION": "1"}),
                     ("tiles", {"W4A16_TRANSITION": "1", "W4A16_TRANSITION_SK": "0"}),
                     ("tiles MI=2", {"W4A16_TRANSITION": "1", "W4A16_TRANSITION_SK": "0",
                                     "W4A16_TRANSITION_MI": "2"}),
                     ("tiles MI=4", {"W4A16_TRANSITION": "1", "W4A16_TRANSITION_SK": "0",
                                     "W4A16_TRANSITION_MI": "4"}),
                     ("four-wave tiles", {"W4A16_TRANSITION": "1", "W4A16_TRANSITION_SK": "0",
                                          "W4A16_TRANSITION_WAVES": "4"}),
                     ("stream-K", {"W4A16_TRANSITION": "1", "W4A16_TRANSITION_SK": "1"}),
                     ("stream-K MI=4", {"W4A16_TRANSITION": "1", "W4A16_TRANSITION_SK": "1",
                                        "W4A16_TRANSITION_MI": "4"})],
    },
    "dot": {
        "what": "one-row GEMMs: the per-wave kernel with MFMA (activation row padded to 16 rows) "
                "against its v_dot2_f32_f16 instances (lane sums by ds_swizzle and "
                "v_permlane32_swap)",
        "shapes": [(1, 4096, 4096, False), (1, 4096, 6144, False), (1, 14336, 4096, False),
                   (1, 8192, 8192, False), (1, 8192, 10240, False), (1, 28672, 8192, False)],
        "outliers": False,
        "variants": [("MFMA", {"W4A16_DECODE_COOP": "0"}),
                     ("v_dot2", {"W4A16_DECODE_COOP": "0", "W4A16_DECODE_DOT": "1"})],
    },
    "smallm": {
        "what": "the decode kernels against the transition kernel forced down to M = 16-32 (the "
                "prefill path with W4A16_TRANSITION=1), Llama-8B projections",
        "shapes": [(m, k, n, sw) for m in (16, 24, 32)
                   for k, n, sw in ((4096, 6144, False), (4096, 4096, False), (4096, 28672, True),
                                    (14336, 4096, False))],
        "outliers": False,
        "variants": [("decode", {}),
                     ("transition", {"_path": "prefill", "W4A16_TRANSITION": "1"})],
    },
    "decode70b": {
        "what": "Llama-70B one-row and small-M projections under both decode kernels",
        "shapes": [(m, 28672, 8192, False) for m in (1, 4, 16)]
                  + [(m, 8192, 10240, False) for m in (1, 4, 16)],
        "outliers": False,
        "variants": [("auto", {}),
                     ("per-wave", {"W4A16_DECODE_COOP": "0"}),
                     ("per-wave half", {"W4A16_DECODE_COOP": "0", "W4A16_DECODE_HALF": "1"}),
                     ("cooperative", {"W4A16_DECODE_COOP": "1"})],
    },
    "splitk": {
        "what": "decode GEMMs that split K: the reduction launch against finishing the splits "
                "inside the GEMM launch (W4A16_SPLIT_FINISH: pairwise atomic exchanges of the "
                "partial values, or the last workgroup of a tile summing partial tiles written "
                "through to the point of coherence), with the automatic configuration and with one "
                "strip per workgroup, eight waves along K and two K splits",
        "shapes": [(8, 14336, 4096, False), (16, 14336, 4096, False), (16, 4096, 4096, False),
                   (32, 4096, 4096, False), (32, 14336, 4096, False), (4, 28672, 8192, False),
                   (16, 28672, 8192, False), (32, 8192, 8192, False), (32, 28672, 8192, False),
                   (8, 4096, 28672, True), (16, 4096, 28672, True)],
        "outliers": False,
        "variants": [("automatic", {}),
                     ("reduction launch", {"W4A16_SPLIT_FINISH": "reduce"}),
                     ("exchange", {"W4A16_SPLIT_FINISH": "exchange"}),
                     ("last workgroup", {"W4A16_SPLIT_FINISH": "last"}),
                     ("1x8 KS=2, reduction launch",
                      {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "8",
                       "W4A16_COOP_KS": "2", "W4A16_SPLIT_FINISH": "reduce"}),
                     ("1x8 KS=2, exchange",
                      {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "8",
                       "W4A16_COOP_KS": "2", "W4A16_SPLIT_FINISH": "exchange"}),
                     ("2x4 KS=2, exchange",
                      {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "2", "W4A16_COOP_WK": "4",
                       "W4A16_COOP_KS": "2", "W4A16_SPLIT_FINISH": "exchange"})],
    },
    "narrow": {
        "what": "narrow, short-K decode GEMMs (Llama-8B QKV and O, and down at M = 16 and 32): "
                "the automatic launch against the per-wave kernel with two K splits (whole and "
                "half strips) and the cooperative kernel with one strip per workgroup and two or "
                "four K splits (in-launch exchange or reduction launch)",
        "shapes": [(m, 4096, n, False) for m in (1, 8, 16, 32) for n in (6144, 4096)]
                  + [(16, 14336, 4096, False), (32, 14336, 4096, False)],
        "outliers": False,
        "variants": [("automatic", {}),
                     ("per-wave KS=2",
                      {"W4A16_DECODE_COOP": "0", "W4A16_DECODE_HALF": "0", "W4A16_DECODE_KS": "2"}),
                     ("per-wave half strips KS=2",
                      {"W4A16_DECODE_COOP": "0", "W4A16_DECODE_HALF": "1", "W4A16_DECODE_KS": "2"}),
                     ("1x8 KS=1",
                      {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "8",
                       "W4A16_COOP_KS": "1"}),
                     ("1x8 KS=2, exchange",
                      {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "8",
                       "W4A16_COOP_KS": "2", "W4A16_SPLIT_FINISH": "exchange"}),
                     ("1x8 KS=2, reduction launch",
                      {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "8",
                       "W4A16_COOP_KS": "2", "W4A16_SPLIT_FINISH": "reduce"}),
                     ("1x8 KS=4, exchange",
                      {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "8",
                       "W4A16_COOP_KS": "4", "W4A16_SPLIT_FINISH": "exchange"}),
                     ("1x4 KS=2, exchange",
                      {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "4",
                       "W4A16_COOP_KS": "2", "W4A16_SPLIT_FINISH": "exchange"})],
    },
}
SWEEPS["coop4"] = {
    "what": "cooperative decode workgroups of four waves (two per CU) against the automatic "
            "eight-wave layout on the fused and 32-row projections",
    "shapes": [(m, 4096, 28672, True) for m in (8, 16, 32)] + [(m, 8192, 57344, True) for m in (16, 32)]
              + [(32, 4096, 6144, False), (32, 14336, 4096, False), (32, 8192, 10240, False)],
    "outliers": False,
    "variants": [("automatic", {}),
                 ("1x4", {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "4",
                          "W4A16_COOP_KS": "1"}),
                 ("2x2", {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "2", "W4A16_COOP_WK": "2",
                          "W4A16_COOP_KS": "1"}),
                 ("1x4 KS=2", {"W4A16_DECODE_COOP": "1", "W4A16_COOP_WC": "1", "W4A16_COOP_WK": "4",
                               "W4A16_COOP_KS": "2"})],
}
for _kind, _what in (("int8", "INT8 weights"), ("zp", "INT4 weights with zero points")):
    SWEEPS["transition_" + _kind] = {
        "what": "%s in the transition window: the automatic launch against the prefill tile "
                "and the transition kernel with eight- and four-wave workgroups (1%% outlier activations; Llama-8B "
                "gate/up and down)" % _what,
        "weights": _kind,
        "shapes": [(m, 4096, 28672, True) for m in (64, 96, 128, 192)]
                  + [(m, 14336, 4096, False) for m in (96, 128)],
        "outliers": True,
        "variants": [("automatic", {}),
                     ("prefill tile", {"W4A16_TRANSITION": "0"}),
                     ("tiles", {"W4A16_TRANSITION": "1", "W4A16_TRANSITION_WAVES": "8"}),
                     ("four-wave tiles", {"W4A16_TRANSITION": "1", "W4A16_TRANSITION_WAVES": "4"})],
    }
SWEEP_ENV = ("W4A16_TRANSITION", "W4A16_TRANSITION_MI", "W4A16_TRANSITION_KS", "W4A16_TRANSITION_SK",
             "W4A16_TRANSITION_WAVES",
             "W4A16_DECODE_COOP", "W4A16_DECODE_DOT", "W4A16_DECODE_HALF", "W4A16_DECODE_KS",
             "W4A16_DECODE_WAVES",
             "W4A16_COOP_WC", "W4A16_COOP_WK", "W4A16_COOP_KS", "W4A16_SPLIT_FINISH")


def run_sweep(name, reps, torch, dev):
    sw = SWEEPS[name]
    stream = torch.cuda.Stream()
    print("# Sweep %s: %s" % (name, sw["what"]), flush=True)
    print("", flush=True)
    print("Command (repository root, one MI355X): `python bench.py --sweep %s`" % name, flush=True)
    print("", flush=True)
    print("Cold weights (one launch per weight copy, at least 800 MB between reuses of a copy) in a "
          "HIP graph, median of three trials of %d replays; two passes over the variants (forward, "
          "then reverse order), the better kept; rel = relative L2 distance of the output from the "
          "first variant's." % reps, flush=True)
    print("", flush=True)
    print("| M | K | N | variant | launch | us (pass 1, pass 2) | best us | rel |", flush=True)
    print("|---|---|---|---|---|---|---|---|", flush=True)
    cache = {}
    for M, K, N, swg in sw["shapes"]:
        kind = sw.get("weights", "int4")
        if (K, N) not in cache:
            cache.clear()
            W = synth.weights(K, N, seed=0)
            w = (w4a16.load_weight_int8 if kind == "int8" else w4a16.load_weight)(W)
            if kind == "zp":
                _, scales = w4a16.unrepack(w)
                w = w4a16.zero_rows(w, scales, torch.from_numpy(
                    synth.zero_points(K // G, N, seed=0)).to(dev))
            ncp = max(2, math.ceil(ROTATE_BYTES / w.nbytes))
            cache[(K, N)] = [w] + [w.clone() for _ in range(ncp - 1)]
        copies = cache[(K, N)]
        A = torch.from_numpy(synth.activations(M, K, seed=0, outliers=sw["outliers"])).to(dev)
        out = torch.empty((M, N // 2 if swg else N), dtype=torch.float16, device=dev)
        times, descs, rels, ref = {}, {}, {}, None
        order = sw["variants"] + sw["variants"][::-1]
        for vname, env in order:
            for k in SWEEP_ENV:
                os.environ.pop(k, None)
            path = env.get("_path", "auto")  # a path for the call, not an environment variable
            os.environ.update({k: v for k, v in env.items() if not k.startswith("_")})
            flags = {"int8": kind == "int8", "zp": kind == "zp"}
            descs[vname] = w4a16.describe(M, K, N, swg, path=path, **flags)
            w4a16.reserve_workspace(w4a16.workspace_bytes(M, K, N, swg, path=path, **flags))
            with torch.cuda.stream(stream):
                w4a16.gemm(A, copies[0], swiglu=swg, out=out, path=path)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy()
            if ref is None:
                ref = got
            rels[vname] = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
            us = time_graph(torch, stream, lambda: [w4a16.gemm(A, c, swiglu=swg, out=out, path=path)
                                                    for c in copies], reps) * 1e3 / len(copies)
            times.setdefault(vname, []).append(us)
        best = min(times, key=lambda v: min(times[v]))
        for vname, _ in sw["variants"]:
            t = times[vname]
            print("| %d | %d | %d | %s%s | `%s` | %.2f, %.2f | %.2f | %.1e |" % (
                M, K, N, vname, " (best)" if vname == best else "", descs[vname], t[0], t[1],
                min(t), rels[vname]), flush=True)
    for k in SWEEP_ENV:
        os.environ.pop(k, None)


def clocks_snapshot():
    """Current shader and memory clock levels and board power, read from the
    amdgpu sysfs files (best effort; no child process)."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        card = dev.split("/")[-2]
        for f in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                for line in open(os.path.join(dev, f)):
                    if "*" in line:
                        out["%s %s" % (card, f)] = line.split(":", 1)[1].replace("*", "").strip()
            except OSError:
                pass
        for f in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_*")):
            if f.endswith(("_average", "_input")):
                try:
                    out["%s %s W" % (card, os.path.basename(f))] = int(open(f).read()) / 1e6
                except (OSError, ValueError):
                    pass
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps per workload (default 200; fallback 20)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="warm-up steps per workload (default 20; fallback 3)")
    ap.add_argument("--workload", default="default", choices=["default"] + sorted(workloads()))
    ap.add_argument("--reps", type=int, default=20, help="graph replays per GEMM timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-floors", action="store_true", help="skip the per-GEMM floor probes")
    ap.add_argument("--comparator", action="store_true",
                    help="also time torch.matmul (hipBLASLt) fp16 dense GEMMs of the M >= 64 shapes")
    ap.add_argument("--dtype", default="fp16", choices=["fp16", "bf16"],
                    help="activation and output type (the weights are the same)")
    ap.add_argument("--zero-points", action="store_true",
                    help="asymmetric weights: seeded zero points as prescaled zero rows")
    ap.add_argument("--int8", action="store_true",
                    help="INT8 weights (W8A16) instead of INT4")
    ap.add_argument("--sweep", choices=sorted(SWEEPS),
                    help="only time the dispatch sweep NAME (a markdown table on stdout)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for hardware-counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this library runs on a single MI355X and has no "
              "multi-GPU path (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # A plain copy of known size: reads and writes exactly 2^30 bytes each.
        src = torch.ones(1 << 29, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 5}))
        return
    w4a16.lib()
    if args.sweep:
        run_sweep(args.sweep, 10, torch, dev)
        return

    zp, int8, bf16 = args.zero_points, args.int8, args.dtype == "bf16"
    if zp and int8:
        raise SystemExit("--zero-points and --int8 do not combine (INT8 weights have no zero points)")
    suffix = ("_bf16" if bf16 else "") + ("_zp" if zp else "") + ("_int8" if int8 else "")
    parts = DEFAULT_PARTS if args.workload == "default" else (args.workload,)
    stream = torch.cuda.Stream()
    results = [run_workload(p, args, torch, dev, stream, zp, int8, bf16) for p in parts]

    log("ceilings ...")
    ceilings = measure_ceilings(stream, torch, dev)
    ceilings["clocks_after_timing"] = clocks_snapshot()
    log("  ", ceilings)

    # Floors: the streaming read of each HBM-bound GEMM's byte count, and the
    # MFMA-loop time of each MFMA-bound GEMM's FLOPs.
    hbm_sizes = [alg_bytes(d["M"], d["K"], d["N"], d["swiglu"], zp, int8)
                 for r in results for d in r["detail"] if d["M"] <= 256]
    floors = {} if args.no_floors else read_floors(torch, stream, dev, hbm_sizes, args.reps)
    for r in results:
        for d in r["detail"]:
            d["hbm_frac_of_measured"] = round(d["GB/s"] / ceilings["stream_read_GBs"], 4)
            d["mfma_frac_of_measured"] = round(d["TFLOP/s"] / ceilings["mfma_f16_TFLOPs"], 4)
            by = alg_bytes(d["M"], d["K"], d["N"], d["swiglu"], zp, int8)
            t_mfma = flops(d["M"], d["K"], d["N"]) / ceilings["mfma_f16_TFLOPs"] / 1e6
            if d["M"] <= 256 and by in floors:
                read = floors[by]
                d["floor_us"] = round(max(read, t_mfma), 3)
                d["floor"] = ("stream read of the GEMM's algorithmic bytes, cold rotation"
                              if read >= t_mfma else "the GEMM's FLOPs at the measured MFMA-loop "
                              "rate (above the stream read of its bytes)")
                d["read_floor_us"] = round(read, 3)
            elif d["M"] > 256:
                d["floor_us"] = round(t_mfma, 3)
                d["floor"] = "the GEMM's FLOPs at the measured MFMA-loop rate"
            if "floor_us" in d:
                d["frac_of_floor"] = round(d["floor_us"] / d["us"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        first = results[0]
        host_w = {}
        for r in results:
            host_w.update(r["host_w"])
        pre = next((r for r in results if r["name"] in ("prefill", "fallback")), None)
        dec_units = first["units"] if first["name"] not in ("prefill", "fallback") else None
        if dec_units is None:
            # Prefill-only runs: the 256-row slice is the sample and the value.
            cpu = cpu_baseline(workloads()["gemv"][1], {**host_w}, pre["units"], bf16=bf16,
                               host_zp=first["host_zp"], int8=int8)
            cpu["value"] = cpu["detail"]["prefill_gemm_all"]["TFLOP/s"]
            cpu["unit"] = "TFLOP/s"
            cpu["sample"] = cpu["detail"]["prefill_gemm_all"]["sample"] + " (extrapolated)"
        else:
            cpu = cpu_baseline(dec_units, host_w, pre["units"] if pre else None, bf16=bf16,
                               host_zp=first["host_zp"], int8=int8)
        log("  ", cpu)

    main_res = results[0]
    is_mfma = main_res["name"] in ("prefill", "fallback")
    if is_mfma:
        value, unit = main_res["step_flops"] / (main_res["ms_step"] * 1e-3) / 1e12, "TFLOP/s"
    else:
        value, unit = main_res["step_bytes"] / (main_res["ms_step"] * 1e-3) / 1e9, "GB/s"
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": main_res["steps"],
        "warmup": main_res["warmup"],
        "ms_per_step": round(main_res["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "fp16",
        "data": "synthetic (seeded N(0,1) " + args.dtype + " activations, N(0,0.02) weights "
                "quantized to " + ("int8" if int8 else "int4") + " G=128"
                + (", seeded zero points near 8 as prescaled zero rows" if zp else "") + ")",
        "config": {"workload": main_res["name"] + suffix, "description": main_res["desc"],
                   "activations": args.dtype, "G": G, "zero_points": zp,
                   "weights": "int8" if int8 else "int4",
                   "gemms_per_step": len(main_res["units"]),
                   "alg_bytes_per_step": main_res["step_bytes"],
                   "flops_per_step": main_res["step_flops"], "weight_copies": main_res["ncopies"],
                   "path": "auto" if main_res["name"] != "fallback" else "prefill and dense",
                   "timing": "HIP graphs of %d step(s), HIP events" % main_res["spg"]},
        "roofline": roofline_entry(main_res, ceilings, zp, int8, suffix),
        "ceilings": ceilings,
        "cpu_baseline": cpu,
        "per_gemm": main_res["detail"],
    }
    for r in results[1:]:
        mf = r["step_flops"] / (r["ms_step"] * 1e-3) / 1e12
        line[r["name"]] = {
            "value": round(mf, 2), "unit": "TFLOP/s", "ms_per_step": round(r["ms_step"], 5),
            "steps": r["steps"], "warmup": r["warmup"], "description": r["desc"],
            "gemms_per_step": len(r["units"]), "flops_per_step": r["step_flops"],
            "alg_bytes_per_step": r["step_bytes"], "weight_copies": r["ncopies"],
            "per_gemm": r["detail"]}
        line["roofline_" + r["name"]] = roofline_entry(r, ceilings, zp, int8, suffix)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
