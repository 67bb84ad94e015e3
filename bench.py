#!/usr/bin/env python3
"""W4A16 GEMM benchmark on one MI355X.

A step is one pass over a workload's GEMMs (default: the Llama-8B-shaped
decode projections QKV, O, fused gate/up with SwiGLU, and down, at
M = 1, 8, 16 and 32), each call running the library's automatic path
through the C ABI.  Inputs are resident in HBM before timing starts.

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
    the step time gives the
    roofline entry (algorithmic bytes = K*N/2 + 2*(K/G)*N + 2*M*K + 2*M*N_out,
    FLOPs = 2*M*N*K).

Ceilings: the library's probe kernels measure the GPU's own streaming-read
rate and fp16 MFMA rate; the roofline entry gives the fraction of both the
data-sheet peak and the measured ceiling; clock levels and board power are
read from sysfs after the timing.

The CPU baseline times the oracle (test infrastructure) on a column sample of
the same GEMMs.

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
# outliers, slot); units sharing a slot use the same copy of their weights.
def workloads():
    def decode(model, shapes, ms):
        units = []
        for mi, m in enumerate(ms):
            for p, (k, n, sw) in shapes.items():
                units.append(("%s_%s_m%d" % (model, p, m), m, k, n, sw, False, mi))
        return units

    w = {
        "llama8b_decode": ("Llama-8B-shaped decode projections (QKV 4096x6144, O 4096x4096, "
                           "gate/up 4096x28672 + SwiGLU, down 14336x4096) at M = 1, 8, 16, 32",
                           decode("8b", synth.LLAMA_8B, (1, 8, 16, 32))),
        "gemv": ("single GEMV M=1 K=4096 N=4096",
                 [("gemv", 1, 4096, 4096, False, False, 0)]),
        "llama70b_decode": ("Llama-70B-shaped decode projections at M = 1, 4, 16, 32",
                            decode("70b", synth.LLAMA_70B, (1, 4, 16, 32))),
        "transition": ("transition batches M = 64, 128, 256 with 1% outlier channels",
                       [(l, m, k, n, sw, o, i) for i, (l, m, k, n, sw, o)
                        in enumerate(synth.CONFIGS["transition"])]),
        "prefill": ("prefill M = 4096, 8191: gate/up 4096x28672 + SwiGLU, down 14336x4096",
                    [(l, m, k, n, sw, o, i) for i, (l, m, k, n, sw, o)
                     in enumerate(synth.CONFIGS["prefill"])]),
    }
    return w


def kernel_key(M, K, N, swiglu, bf16=False, zp=False, int8=False):
    """The kernel instance a GEMM launches under the automatic path, as the
    profiler names it, marked when a second (split-K reduction) launch
    follows it."""
    desc = w4a16.describe(M, K, N, swiglu, bf16=bf16, zp=zp, int8=int8)
    first = desc.split(";")[0]
    name = first.split(" workgroups=")[0].strip()
    return name + (" + reduce" if ";" in desc else "")


# HIP sources that define each kernel family (the digest of stored counters
# covers these; a kernel of no listed family is covered by every source).
KERNEL_SOURCES = {
    "decode": ("common.h", "decode.hip", "decode_args.h", "decode_coop.hip"),
    "prefill": ("common.h", "prefill.hip"),
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


def cpu_baseline(units, host_w, target_s=12.0, bf16=False, host_zp=None, int8=False):
    """Time the oracle's fp64 GEMM (+ SwiGLU) on a column sample of every unit
    (host_w: the same seeded fp32 weights the GPU was given, keyed by (K, N))."""
    import oracle
    o = oracle.load()
    threads = o.max_threads()
    total_mac = sum(m * k * n for _, m, k, n, *_ in units)
    # Calibrate the oracle's rate on a small product, then size the sample.
    Wc = synth.weights(4096, 1024, seed=5)
    pc, sc = o.quantize_pack(Wc)
    Ac = synth.activations(8, 4096, seed=5)
    t0 = time.perf_counter()
    o.gemm_f64(Ac, pc, sc)
    rate = 8 * 4096 * 1024 / max(time.perf_counter() - t0, 1e-6)
    frac = min(1.0, target_s * rate / total_mac)
    frac = max(frac, 1.0 / 64)
    done_bytes, elapsed, cols_desc = 0, 0.0, []
    for label, M, K, N, sw, outl, _ in units:
        ncols = N // 2 if sw else N
        ns = max(32, int(round(ncols * frac / 32)) * 32)
        ns = min(ns, ncols)
        W = host_w[(K, N)]
        Ws = np.concatenate([W[:, :ns], W[:, N // 2:N // 2 + ns]], axis=1) if sw else W[:, :ns]
        packed, s16 = (o.quantize_pack8 if int8 else o.quantize_pack)(np.ascontiguousarray(Ws))
        A = (synth.activations_bf16 if bf16 else synth.activations)(M, K, seed=0, outliers=outl)
        if host_zp is not None:
            Z = host_zp[(K, N)]
            Zs = np.concatenate([Z[:, :ns], Z[:, N // 2:N // 2 + ns]], axis=1) if sw else Z[:, :ns]
            z16 = o.zero_rows(s16, np.ascontiguousarray(Zs))
        t0 = time.perf_counter()
        if host_zp is not None:
            Wz = o.dequant_zp(packed, s16, z16, bf16=bf16)
            C = (o.gemm_wb_f64 if bf16 else o.gemm_w16_f64)(A, Wz)
        elif int8:
            C = o.gemm8_f64(A, packed, s16, bf16=bf16)
        else:
            C = (o.gemm_bf16_f64 if bf16 else o.gemm_f64)(A, packed, s16)
        if sw:
            o.swiglu_f64(C)
        elapsed += time.perf_counter() - t0
        done_bytes += alg_bytes(M, K, Ws.shape[1], sw, host_zp is not None, int8)
        cols_desc.append(ns)
    return {
        "value": round(done_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("fp64 oracle GEMM (+SwiGLU) on the first %.1f%% of output columns of each of "
                   "the %d GEMMs (all rows, full K), %.1f s on %d threads; quantize/pack untimed"
                   % (100 * frac, len(units), elapsed, threads)),
    }


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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_decode", choices=sorted(workloads()))
    ap.add_argument("--reps", type=int, default=20, help="graph replays per GEMM timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dtype", default="fp16", choices=["fp16", "bf16"],
                    help="activation and output type (the weights are the same)")
    ap.add_argument("--zero-points", action="store_true",
                    help="asymmetric weights: seeded zero points as prescaled zero rows")
    ap.add_argument("--int8", action="store_true",
                    help="INT8 weights (W8A16) instead of INT4")
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

    desc, units = workloads()[args.workload]
    nslots = max(u[6] for u in units) + 1

    # Weights: one seeded W per distinct projection, quantized, packed and
    # repacked on the device, then cloned into rotation copies.
    shapes = sorted({(k, n) for _, _, k, n, *_ in units})
    zp = args.zero_points
    int8 = args.int8
    if zp and int8:
        raise SystemExit("--zero-points and --int8 do not combine (INT8 weights have no zero points)")
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
    slot_bytes = [sum(base[(k, n)].nbytes for _, _, k, n, _, _, s in units if s == slot)
                  for slot in range(nslots)]
    per_slot = max(slot_bytes)
    ncopies = max(2, math.ceil(ROTATE_BYTES / per_slot)) if per_slot < ROTATE_BYTES else 2
    copies = {key: [w] + [w.clone() for _ in range(ncopies - 1)] for key, w in base.items()}
    log("rotation: %d copies of %.1f MB per slot" % (ncopies, per_slot / 1e6))

    bf16 = args.dtype == "bf16"
    act_dtype = torch.bfloat16 if bf16 else torch.float16
    acts = {}
    for _, m, k, n, sw, outl, _ in units:
        if (m, k, outl) not in acts:
            if bf16:
                bits = synth.activations_bf16(m, k, seed=0, outliers=outl)
                acts[(m, k, outl)] = torch.from_numpy(bits.view(np.int16)).to(dev).view(
                    torch.bfloat16)
            else:
                acts[(m, k, outl)] = torch.from_numpy(
                    synth.activations(m, k, seed=0, outliers=outl)).to(dev)
    outs = {}
    for label, m, k, n, sw, *_ in units:
        outs[label] = torch.empty((m, n // 2 if sw else n), dtype=act_dtype, device=dev)

    stream = torch.cuda.Stream()

    def run_unit(u, copy):
        label, m, k, n, sw, outl, _ = u
        w = copies[(k, n)][copy]
        if zp or int8:
            w4a16.gemm(acts[(m, k, outl)], w, swiglu=sw, out=outs[label])
        elif sw:
            if bf16:
                w4a16.gemm(acts[(m, k, outl)], w, swiglu=True, out=outs[label])
            else:
                w4a16.gemm_swiglu(acts[(m, k, outl)], w, out=outs[label])
        elif bf16:
            w4a16.gemm(acts[(m, k, outl)], w, out=outs[label])
        else:
            w4a16.gemm_plain(acts[(m, k, outl)], w, out=outs[label])

    # Rotation: step s, slot t uses copy (s * nslots + t) % ncopies; the
    # pattern repeats every `period` steps, one graph per step of the period.
    period = ncopies // math.gcd(ncopies, nslots)

    def step_copy(s, slot):
        return (s * nslots + slot) % ncopies

    with torch.cuda.stream(stream):
        for s in range(period):      # eager warm-up: allocates the library workspace
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
        """Replay steps first .. first+count-1 (rotation order kept)."""
        s = first
        while s < first + count:
            if spg > 1 and first + count - s >= spg and (s % period) in multi:
                multi[s % period].replay()
                s += spg
            else:
                graphs[s % period].replay()
                s += 1

    # Warm-up, then exactly K timed steps.
    with torch.cuda.stream(stream):
        replay_steps(0, args.warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        replay_steps(args.warmup, args.steps)
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    step_bytes = sum(alg_bytes(m, k, n, sw, zp, int8) for _, m, k, n, sw, *_ in units)
    step_flops = sum(flops(m, k, n) for _, m, k, n, *_ in units)
    log("step: %.2f us (wall %.2f us), %.1f MB, %.2f GFLOP"
        % (ms_step * 1e3, wall / args.steps * 1e6, step_bytes / 1e6, step_flops / 1e9))

    # Per-GEMM timing: a graph of one launch per weight copy (all cold).
    detail = []
    for u in units:
        label, m, k, n, sw, outl, slot = u
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in range(ncopies):
                run_unit(u, c)
        # Three replays of warm-up, then the median of three trials of
        # `reps` replays each (the first GEMM timed after the step graphs
        # otherwise reads high on some runs).
        trials = []
        with torch.cuda.stream(stream):
            for _ in range(3):
                g.replay()
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(args.reps):
                    g.replay()
                b.record(stream)
                trials.append((a, b))
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) for a, b in trials)[1] * 1e3 / (args.reps * ncopies)
        by, fl = alg_bytes(m, k, n, sw, zp, int8), flops(m, k, n)
        detail.append({"gemm": label, "M": m, "K": k, "N": n, "swiglu": sw,
                       "kernel": kernel_key(m, k, n, sw, bf16, zp, int8),
                       "launch": w4a16.describe(m, k, n, sw, bf16=bf16, zp=zp, int8=int8),
                       "us": round(us, 3),
                       "GB/s": round(by / us / 1e3, 1), "TFLOP/s": round(fl / us / 1e6, 2),
                       "hbm_frac": round(by / us / 1e3 / HBM_PEAK_GBS, 4),
                       "mfma_frac": round(fl / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)})
        log("  %-22s %-44s %9.2f us %8.1f GB/s %8.2f TFLOP/s" %
            (label, detail[-1]["kernel"], us, detail[-1]["GB/s"], detail[-1]["TFLOP/s"]))
        del g

    log("ceilings ...")
    ceilings = measure_ceilings(stream, torch, dev)
    ceilings["clocks_after_timing"] = clocks_snapshot()
    log("  ", ceilings)
    for d in detail:
        d["hbm_frac_of_measured"] = round(d["GB/s"] / ceilings["stream_read_GBs"], 4)
        d["mfma_frac_of_measured"] = round(d["TFLOP/s"] / ceilings["mfma_f16_TFLOPs"], 4)

    # Dominant kernel: the largest share of the per-GEMM times.
    by_kernel = {}
    for d in detail:
        e = by_kernel.setdefault(d["kernel"], {"us": 0.0, "bytes": 0, "flops": 0, "launches": 0})
        e["us"] += d["us"]
        e["bytes"] += alg_bytes(d["M"], d["K"], d["N"], d["swiglu"], zp, int8)
        e["flops"] += flops(d["M"], d["K"], d["N"])
        e["launches"] += 1
    dom = max(by_kernel, key=lambda k: by_kernel[k]["us"])
    e = by_kernel[dom]
    avg_us = e["us"] / e["launches"]
    hbm_bound = all(d["M"] <= 64 for d in detail if d["kernel"] == dom)
    if hbm_bound:
        achieved = e["bytes"] / e["us"] / 1e3
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = e["flops"] / e["us"] / 1e6
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4)}
    ceiling = ceilings["stream_read_GBs"] if hbm_bound else ceilings["mfma_f16_TFLOPs"]
    roof["frac_of_measured_ceiling"] = round(achieved / ceiling, 4) if ceiling else None
    suffix = ("_bf16" if bf16 else "") + ("_zp" if zp else "") + ("_int8" if int8 else "")
    roof["traffic"] = stored_traffic(args.workload + suffix, dom)
    roof["kernel"] = dom
    roof["launch_workgroups"] = sorted({int(re.search(r"workgroups=(\d+)", d["launch"]).group(1))
                                        for d in detail if d["kernel"] == dom})
    roof["launches_per_step"] = e["launches"]
    roof["avg_launch_us"] = round(avg_us, 3)
    roof["alg_bytes_per_launch"] = round(e["bytes"] / e["launches"])
    roof["alg_flops_per_launch"] = round(e["flops"] / e["launches"])

    any_prefill = any(m >= 4096 for _, m, *_ in units)
    if any_prefill:
        value, unit = step_flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
    else:
        value, unit = step_bytes / (ms_step * 1e-3) / 1e9, "GB/s"

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(units, host_w, bf16=bf16, host_zp=host_zp, int8=int8)
        if unit == "TFLOP/s":
            cpu["value"] = round(cpu["value"] * step_flops / step_bytes / 1e3, 6)
            cpu["unit"] = "TFLOP/s"
        log("  ", cpu)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "fp16",
        "data": "synthetic (seeded N(0,1) " + args.dtype + " activations, N(0,0.02) weights quantized to "
                + ("int8" if int8 else "int4") + " G=128"
                + (", seeded zero points near 8 as prescaled zero rows" if zp else "") + ")",
        "config": {"workload": args.workload + suffix, "description": desc,
                   "activations": args.dtype, "G": G, "zero_points": zp,
                   "weights": "int8" if int8 else "int4",
                   "gemms_per_step": len(units), "alg_bytes_per_step": step_bytes,
                   "flops_per_step": step_flops, "weight_copies": ncopies,
                   "path": "auto",
                   "timing": "HIP graphs of %d step(s), HIP events" % spg},
        "roofline": roof,
        "ceilings": ceilings,
        "cpu_baseline": cpu,
        "per_gemm": detail,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
