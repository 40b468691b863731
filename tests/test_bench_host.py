"""Host-side logic of bench.py (no GPU): the algorithmic work model behind the roofline,
the derived peaks, the committed traffic record and the one-GPU guard."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_work_model_per_entry_counts(bench):
    """Per score entry: one exp per pass, 2D flops per contraction over D, one code byte
    per pair per pass (shared by all heads), node tensors once."""
    N, H, D, s = 32768, 8, 8, 2
    E = H * N * N
    node, f32node = N * H * D * s, N * H * D * 4
    fl, ex, by = bench.work_model("fwd", N, H, D, s)
    assert ex == E and fl == E * (2 * 2 * D + 4)
    assert by == N * N + 3 * node + f32node + N * H * 4
    fl, ex, by = bench.work_model("bwd_kv", N, H, D, s)
    assert ex == E and fl == E * (4 * 2 * D + 5)
    fl, ex, by = bench.work_model("bwd_q", N, H, D, s)
    assert ex == E and fl == E * (3 * 2 * D + 4)
    # the one-pass backward: one exp per entry for both the key-side and the query-side gradients
    fl, ex, by = bench.work_model("bwd_fused", N, H, D, s)
    assert ex == E and fl == E * (5 * 2 * D + 5)
    assert by == N * N + 4 * node + 2 * N * H * 4 + 3 * f32node
    # the contraction counts behind the MFMA bound agree with the flop model
    for name, n in bench.CONTRACTIONS.items():
        fl, ex, _ = bench.work_model(name, N, H, D, s)
        assert fl - n * 2 * D * E in (4 * E, 5 * E)


def test_derived_peaks(bench):
    # 256 CUs x 4 SIMDs x 8 lanes per clock (half-rate v_exp_f32) x 2.4 GHz
    assert bench.EXP_PEAK_TOPS == pytest.approx(19.6608)
    # the fp32 vector peak with the same unit counts is the published 157.3 TFLOP/s
    assert 256 * 4 * 16 * 2 * 2 * 2.4e9 / 1e12 == pytest.approx(157.3, rel=1e-3)
    assert bench.MFMA_PEAK_TFLOPS == 2500.0
    assert bench.HBM_PEAK_GBS == 8000.0


def test_binding_unit_by_head_dimension(bench):
    """The MFMA bound applies at D = 32 (sbm65536) and the exp bound at D = 8."""
    def mfma_bound(N, D):
        E = 8 * N * N
        return bench.CONTRACTIONS["bwd_kv"] * 2 * D * E / (bench.MFMA_PEAK_TFLOPS * 1e12) > E / (bench.EXP_PEAK_TOPS * 1e12)
    assert not mfma_bound(32768, 8)
    assert mfma_bound(65536, 32)


def test_traffic_record_is_tied_to_the_kernel_sources(bench, tmp_path, monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_ba32768-bf16.json")
    with open(path) as f:
        rec = json.load(f)
    # the kernels of the default step: the forward and the one-pass backward
    for k in ("fwd", "bwd_fused"):
        assert rec["kernels"][k]["hbm_bytes_per_launch"] > 0
    if rec["source_hash"] == bench.kernel_source_hash():
        assert (bench.recorded_traffic("bwd_fused", "ba32768-bf16")
                == rec["kernels"]["bwd_fused"]["hbm_bytes_per_launch"])
    assert bench.recorded_traffic("bwd_fused", "no-such-workload") is None
    # the head-dimension-32 record is checked against that path's sources
    with open(os.path.join(ROOT, "profiles", "traffic_sbm65536-d32-bf16.json")) as f:
        rec32 = json.load(f)
    assert bench.kernel_source_hash(32) != bench.kernel_source_hash(8)
    if rec32["source_hash"] == bench.kernel_source_hash(32):
        assert (bench.recorded_traffic("bwd_kv", "sbm65536-d32-bf16", 32)
                == rec32["kernels"]["bwd_kv"]["hbm_bytes_per_launch"])
    assert bench.recorded_traffic("bwd_kv", "sbm65536-d32-bf16", 8) is None
    # a record taken from other sources is not used
    (tmp_path / "profiles").mkdir()
    rec["source_hash"] = "0" * 16
    (tmp_path / "profiles" / "traffic_ba32768-bf16.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda D=8: "f" * 16)
    assert bench.recorded_traffic("bwd_fused", "ba32768-bf16") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
