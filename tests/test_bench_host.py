"""Host-side logic of bench.py (no GPU): the algorithmic work it divides by
the measured time, the counter table's source check, and the one-GPU rule.
The expected values are written out from the layer shapes, not taken from
bench.py's own formulas."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_config  # noqa: E402


def test_mixtral_launch_work_closed_form():
    """Mixtral-shaped prefill, every token kept (16384 rows over 8 experts):
    fc1 = two projections of 14336 x 4096, fc2 one of 4096 x 14336."""
    cfg = get_config("c4")
    kept, used = 8192 * 2, 8
    w = bench.launch_work(cfg, kept, used, 8192)
    assert w["fc1"]["flops"] == 2 * 16384 * 4096 * 14336 * 2
    assert w["fc2"]["flops"] == 2 * 16384 * 14336 * 4096
    # weights once (W1 and W3 of all 8 experts) plus x read once; H is not counted
    assert w["fc1"]["bytes"] == 8 * 2 * 14336 * 4096 * 2 + 8192 * 4096 * 2
    assert w["fc2"]["bytes"] == 8 * 4096 * 14336 * 2


def test_decode_layer_work_closed_form():
    """Decode layer: the router's logits and the expert projections over the
    768 kept rows; bytes are the router matrix, the 64 experts' three
    matrices once, x in and out."""
    cfg = get_config("c5")
    flops, nbytes = bench.layer_work(cfg, 128 * 6, 64)
    assert flops == 2 * 128 * 2048 * 64 + 2 * 768 * 2048 * 1408 * 3
    assert nbytes == 64 * 2048 * 2 + 64 * 3 * 2048 * 1408 * 2 + 2 * 128 * 2048 * 2


def test_biased_layer_counts_its_biases():
    """The tiny fp32 layer has biases: 4-byte elements, b1 with fc1, b2 with
    fc2, only for the experts that received rows."""
    cfg = get_config("c1")
    w = bench.launch_work(cfg, 100, 3, 50)
    assert w["fc1"]["bytes"] == 3 * (1024 * 256 + 1024) * 4 + 50 * 256 * 4
    assert w["fc2"]["bytes"] == 3 * (256 * 1024 + 256) * 4


def test_code_hash_ignores_comments_and_layout_only():
    a = "int f(int x) {\n  // old note\n  return x + 1;  /* tail */\n}\n"
    b = "int f(int x) {\n\n  // a different note\n      return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_counter_figures_need_matching_sources(monkeypatch):
    rec = {"sources": "not-the-current-hash",
           "fc1": {"fetch_kib": 1.0, "write_kib": 1.0, "grbm": 8e6, "mfma_busy": 1e6, "simds": 1024,
                   "dur_ns": 2e6}}
    monkeypatch.setitem(bench.PMC_TRAFFIC, "c4", rec)
    assert bench.measured_traffic("c4", "fc1") is None
    assert bench.counter_clock("c4", "fc1") is None
    rec = dict(rec, sources=bench.sources_sha(bench.pmc_sources("c4")))
    monkeypatch.setitem(bench.PMC_TRAFFIC, "c4", rec)
    assert bench.measured_traffic("c4", "fc1") == pytest.approx(
        1024 * bench.PMC_COPY_FACTOR["fetch"] + 1024 * bench.PMC_COPY_FACTOR["write"])
    clk = bench.counter_clock("c4", "fc1")
    assert clk["ghz"] == pytest.approx(8e6 / 8 / 2e6)  # cycles per XCD over ns
    assert clk["mfma_busy"] == pytest.approx(1e6 / 1024 / (8e6 / 8))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
