"""Host-side logic of bench.py (no GPU): the one-GPU guard and the choice of
the binding roofline for the grouped GEMM."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_ffn_roofline_picks_the_binding_resource():
    import bench
    # headline gate/up: ~1.54e16 flops over ~20 GB -> above the machine balance
    r = bench.ffn_roofline("g", 1.54e16, 2.0e10, 0.012)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1.54e16 / 0.012 / 1e12, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.BF16_PEAK_TFLOPS, rel=1e-3)
    # small-batch inference: weights dominate, 32 flop per byte -> HBM-bound
    r = bench.ffn_roofline("g", 4.8e11, 1.5e10, 0.003)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(5000.0, rel=1e-3)
    assert r["per_launch"] == {"flops": 4.8e11, "bytes": 1.5e10, "avg_s": 0.003}


def test_algorithmic_bytes_scale_with_the_row_width():
    import bench
    import moonep_synth as synth
    w = synth.WORKLOADS["fwd_r8_s4096_k8_e256"]
    p, d, c = bench.alg_bytes(w)
    ntok = w.R * w.S
    # the bf16 rows dominate: one read and K writes (dispatch), K reads and one write (combine)
    assert d == pytest.approx(ntok * 2 * w.H * (1 + w.K), rel=0.01)
    assert c == pytest.approx(ntok * 2 * w.H * (1 + w.K), rel=0.01)
    assert p == 8 * ntok * w.K + 4 * w.R * (w.E + w.B)
