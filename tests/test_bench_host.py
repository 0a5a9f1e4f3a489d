"""Host-side checks of bench.py's measurement helpers (no GPU)."""
import json
import os

import bench

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_roofline_formula_matches_the_pages_example():
    ex = GOLDEN["roofline_example"]
    peak = ex["peak_gflops"]
    ridge = ex["ridge_intensity_flop_per_byte"]
    bw = peak / ridge                       # the ridge is where both roofs meet
    assert bench.roofline(peak, bw, ridge) == peak
    assert bench.roofline(peak, bw, ex["bandwidth_limited_point_intensity"]) < peak
    assert bench.roofline(peak, bw, ex["compute_limited_point_intensity"]) == peak
    assert bench.roofline(peak, bw, 0.5) == bw * 0.5


def test_stage_work_counts_useful_flops():
    T, d, E, f, k = 16384, 4096, 128, 1536, 4
    R = T * k
    gemm = [s for s in bench.STAGES if s.startswith("gemm")]
    flops = sum(bench.stage_work(s, T, d, E, f, k, R)[0] for s in gemm)
    assert flops == 18 * R * d * f            # fwd 6·R·d·f + bwd 12·R·d·f
    # permute moves each token row once in and k times out
    assert bench.stage_work("permute", T, d, E, f, k, R)[1] == T * d * 2 + R * d * 2 + T * k * 4
    # weights are read once per GEMM that uses them
    _, by = bench.stage_work("gemm_gate_up", T, d, E, f, k, R)
    assert by >= E * 2 * f * d * 2


def test_traffic_record_is_ignored_after_a_source_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"hbm_bytes_per_launch": 123, "source_sha256_16": bench.source_hash("gemm_wgrad")}
    (tmp_path / "traffic_gemm_wgrad_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("gemm_wgrad", "w") == 123
    rec["source_sha256_16"] = "0" * 16
    (tmp_path / "traffic_gemm_wgrad_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("gemm_wgrad", "w") is None


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_stage_work_mx_counts_codes_and_scales():
    T, d, E, f, k = 32768, 4096, 16, 1536, 1
    R = T * k
    gemm = [s for s in bench.STAGES if s.startswith("gemm")]
    assert sum(bench.stage_work(s, T, d, E, f, k, R, mx=True)[0] for s in gemm) == 18 * R * d * f
    # MXFP8 payload: one code byte plus one scale byte per 32 elements
    assert bench.stage_work("permute", T, d, E, f, k, R, mx=True)[1] == \
        T * d * 2 + R * d * 33 / 32 + T * k * 4
    bf, mx = (bench.stage_work("gemm_gate_up", T, d, E, f, k, R, mx=m)[1] for m in (False, True))
    assert bf - mx == (R * d + E * 2 * f * d) * (2 - 33 / 32)
    # the bf16 and MXFP8 GEMMs are different kernels: their traffic records differ
    assert bench.source_hash("gemm_wgrad") != bench.source_hash("gemm_wgrad", mx=True)
