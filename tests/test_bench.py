"""bench.py's host-side arithmetic and refusals (CPU only): the algorithmic
bytes and FLOPs of a GEMM, the choice of the dominant kernel and its roofline
entry, the stored-counter lookup, and the single-GPU refusal."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_gpus_above_one_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("M,K,N,swiglu,zp,int8", [
    (1, 4096, 6144, False, False, False),
    (16, 4096, 28672, True, False, False),
    (8191, 14336, 4096, False, True, False),
    (32, 8192, 57344, True, False, True),
])
def test_algorithmic_bytes(M, K, N, swiglu, zp, int8):
    # The INT4 kernels page's byte count, written out per operand: the
    # weights once (4 bits each, 8 for INT8), one fp16 scale per column and
    # 128 rows of K (and a zero row as large), the fp16 activations once and
    # the fp16 output once (half the columns after SwiGLU).
    weights = K * N * (8 if int8 else 4) / 8
    scales = (K / 128) * N * 2 * (2 if zp else 1)
    acts = M * K * 2
    out = M * (N / 2 if swiglu else N) * 2
    assert bench.alg_bytes(M, K, N, swiglu, zp, int8) == weights + scales + acts + out
    assert bench.flops(M, K, N) == 2 * M * N * K


def _detail(gemm, M, K, N, kernel, us, wg, swiglu=False):
    return {"gemm": gemm, "M": M, "K": K, "N": N, "swiglu": swiglu, "kernel": kernel, "us": us,
            "launch": "%s workgroups=%d threads=512 ks=1" % (kernel, wg)}


def test_roofline_entry_takes_the_kernel_with_the_largest_time_share():
    a, b = "decode_kernel<16, 1, 8, 2, 4, x>", "decode_coop_kernel<16, 2, 2, 4, 4, y>"
    res = {"name": "unit", "detail": [
        _detail("q", 8, 4096, 6144, a, 7.0, 192),
        _detail("o", 8, 4096, 4096, a, 6.0, 256),
        _detail("gu8", 8, 4096, 28672, b, 14.0, 224, swiglu=True),
        _detail("gu16", 16, 4096, 28672, b, 15.0, 224, swiglu=True),
    ]}
    ceil = {"stream_read_GBs": 6000.0, "mfma_f16_TFLOPs": 1900.0}
    r = bench.roofline_entry(res, ceil, False, False, "")
    assert r["kernel"] == b and r["bound"] == "hbm" and r["unit"] == "GB/s"
    byts = bench.alg_bytes(8, 4096, 28672, True) + bench.alg_bytes(16, 4096, 28672, True)
    assert r["achieved"] == pytest.approx(byts / 29.0 / 1e3, abs=0.05)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.HBM_PEAK_GBS, abs=1e-4)
    assert r["frac_of_measured_ceiling"] == pytest.approx(r["achieved"] / 6000.0, abs=1e-4)
    assert r["launches_per_step"] == 2 and r["launch_workgroups"] == [224]
    assert r["avg_launch_us"] == pytest.approx(14.5)
    assert r["alg_bytes_per_launch"] == round(byts / 2)
    assert r["traffic"] is None     # no counter summary for this workload


def test_roofline_entry_is_compute_bound_above_64_rows():
    k = "prefill2_kernel<4, 1, 8, 2, z>"
    res = {"name": "unit", "detail": [_detail("p", 4096, 4096, 28672, k, 800.0, 1792, swiglu=True)]}
    r = bench.roofline_entry(res, {"stream_read_GBs": 6000.0, "mfma_f16_TFLOPs": 1900.0},
                             False, False, "")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(2 * 4096 * 4096 * 28672 / 800.0 / 1e6, abs=0.05)
    assert r["peak"] == bench.MFMA_F16_PEAK_TFLOPS


def test_stored_traffic_applies_only_to_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    kernel = "decode_coop_kernel<16, 2, 2, 4, 4, true, false, false, 4>"
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))

    def write(digest, workload="unit", kern=kernel):
        (tmp_path / "traffic_unit.txt").write_text(
            "# summary\n\nsource_digest = %s\nworkload = %s\nkernel = %s\n"
            "hbm_bytes_per_launch = 61905361\n" % (digest, workload, kern))

    assert bench.stored_traffic("unit", kernel) is None          # no file
    write(bench.source_digest(kernel))
    assert bench.stored_traffic("unit", kernel) == 61905361.0
    write("0123456789abcdef")                                     # other sources
    assert bench.stored_traffic("unit", kernel) is None
    write(bench.source_digest(kernel), kern="decode_kernel<16, 1, 8, 2, 4>")
    assert bench.stored_traffic("unit", kernel) is None          # other kernel


def test_source_digest_follows_the_kernel_family():
    d = bench.source_digest("decode_coop_kernel<16, 2, 2, 4, 4, true, false, false, 4>")
    assert d == bench.source_digest("decode_kernel<16, 1, 8, 2, 4>")      # same family
    assert d != bench.source_digest("prefill2_kernel<4, 1, 8, 2, false>")
    assert len(d) == 16
