"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the roofline
arithmetic and the algorithmic work per step, and that a traffic summary
taken on other kernel sources is not used."""
import os
import subprocess
import sys

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


def test_traffic_summary_is_ignored_after_a_source_change(monkeypatch):
    wl = WORKLOADS["decode_128k"]
    path = os.path.join(ROOT, "profiles", "attention_decode_128k_traffic.txt")
    if not os.path.exists(path):
        pytest.skip("no attention traffic summary committed")
    real = bench.source_hash("attention")
    with open(path) as f:
        recorded = [ln.split("=", 1)[1].strip() for ln in f if ln.startswith("kernel_source_sha256")]
    if recorded != [real]:
        assert bench.measured_traffic("attention", wl) is None
    else:
        assert bench.measured_traffic("attention", wl) > 0
    monkeypatch.setattr(bench, "source_hash", lambda phase: "0" * 64)
    assert bench.measured_traffic("attention", wl) is None
