"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the roofline
arithmetic and the algorithmic work per step, and that a traffic summary
taken on other kernel sources is not used."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_02_amd.synth import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_attention_work_per_selected_pair():
    # decode: 64 tokens, each with k = 2048 selected rows, 128 heads over
    # 576 + 512 columns; every selected row is read once (disjoint caches)
    wl = WORKLOADS["decode_128k"]
    w = bench.work(wl)["attention"]
    pairs = 64 * 2048
    assert w["flops"] == pairs * 2 * 128 * (576 + 512)
    assert w["bytes"] == pairs * 576 * 2 + 64 * (128 * (576 + 512) * 2 + 2048 * 4)
    assert w["flop_unit"] == "bf16"


def test_indexer_work_counts_causal_candidates_only():
    wl = WORKLOADS["prefill_8k"]
    w = bench.work(wl)["indexer"]
    pairs = 8192 * 8193 // 2  # query t sees keys 0..t
    assert w["flops"] == pairs * 2 * 8 * 128
    assert w["bytes"] == 8192 * (128 + 4) + 8192 * 8 * (128 + 8)
    topk = bench.work(wl)["topk"]
    assert topk["bytes"] == pairs * 4 + 8192 * 2048 * 4


def test_roofline_picks_the_binding_roof():
    wl = WORKLOADS["chunk_128k"]
    w = bench.work(wl)["attention"]
    r = bench.roofline("attention", w, 2.0e-3)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(w["flops"] / 2.0e-3 / 1e12, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    wd = bench.work(WORKLOADS["decode_128k"])["indexer"]
    rd = bench.roofline("indexer", wd, 2.0e-4)
    assert rd["bound"] == "hbm" and rd["unit"] == "GB/s" and rd["peak"] == 8000.0
    assert rd["achieved"] == pytest.approx(wd["bytes"] / 2.0e-4 / 1e9, rel=1e-3)
    assert bench.phase_floor(wd) == pytest.approx(wd["bytes"] / 8000e9)


def test_traffic_summary_is_ignored_after_a_source_change(monkeypatch, tmp_path):
    wl = WORKLOADS["decode_128k"]
    kernel = "sparse_mla_attn_bf16<true>"
    assert bench.profile_name(kernel) == "sparse_mla_attn_bf16_true"
    real = bench.source_hash(kernel)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "sparse_mla_attn_bf16_true_decode_128k_traffic.txt").write_text(
        f"# test summary\nhbm_bytes_per_launch = 123456\nkernel_source_sha256 = {real}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda k: real)
    assert bench.measured_traffic(kernel, wl) == 123456
    monkeypatch.setattr(bench, "source_hash", lambda k: "0" * 64)
    assert bench.measured_traffic(kernel, wl) is None


def test_kernel_work_attribution():
    w = bench.work(WORKLOADS["decode_128k"])
    assert bench.kernel_work("indexer_fp8_stream<false, 1, true>", w) is w["indexer"]
    assert bench.kernel_work("sparse_mla_attn_bf16<true>", w) is w["attention"]
    assert bench.kernel_work("indexer_fp8_tiled<false>", w) is w["indexer"]
    assert bench.kernel_work("topk_rows", w) is w["topk"]
    assert bench.kernel_work("attn_combine", w) is None
    assert bench.kernel_work("indexer_sample_threshold", w) is None


def test_roofline_against_measured_peaks():
    w = bench.work(WORKLOADS["decode_128k"])["attention"]
    r = bench.roofline("a", w, 5e-5, {"hbm_read_gbs": 6000.0})
    assert r["bound"] == "hbm"
    assert r["frac_of_measured"] == pytest.approx(r["achieved"] / 6000.0, rel=1e-3)
    wc = bench.work(WORKLOADS["chunk_128k"])["indexer"]
    rc = bench.roofline("i", wc, 5e-4, {"fp8_mfma_tflops": 3000.0})
    assert rc["bound"] == "mfma" and rc["peak"] == 5000.0
    assert rc["frac_of_measured"] == pytest.approx(rc["achieved"] / 3000.0, rel=1e-3)


def test_cpu_info_reports_affinity_cores():
    model, cores, threads = bench.cpu_info()
    assert cores == len(os.sched_getaffinity(0))
    assert isinstance(model, str) and model
    assert threads >= 1


def test_row_parity_rule():
    wl = WORKLOADS["decode_128k"].with_(k=4)
    scores = np.array([5.0, 1.0, 4.0, 3.0, 2.0, 4.0005, 0.5])
    ref_sel = np.array([0, 2, 3, 5])
    out = np.zeros((2, 3))
    assert bench._check_row(np.array([0, 2, 3, 5]), out, scores, ref_sel, out, wl, 7, "x") is None
    # token 2 (4.0) and 5 (4.0005) are not at the k-th score (3.0): a swap
    # with token 4 (2.0) is outside the band
    assert "band" in bench._check_row(np.array([0, 2, 4, 5]), out, scores, ref_sel, out, wl, 7, "x")
    assert "malformed" in bench._check_row(np.array([0, 3, 2, 5]), out, scores, ref_sel, out, wl, 7, "x")
    assert "attention" in bench._check_row(np.array([0, 2, 3, 5]), out + 0.05, scores, ref_sel, out, wl,
                                           7, "x")
