"""Host-side logic of bench.py (no GPU): the one-GPU guard and the choice of
the binding roofline for the grouped GEMM, and the counter-measured traffic."""
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


def test_measured_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """Counter figures are reported only while the kernel sources they were
    taken with are unchanged (one hash for the GEMMs, one for data movement)."""
    import hashlib
    import bench
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    for f, text in (("gemm_core.h", "a"), ("gemm.hip", "b"), ("move.hip", "c")):
        (csrc / f).write_text(text)
    gemm = hashlib.sha256(b"ab").hexdigest()
    move = hashlib.sha256(b"c").hexdigest()
    summary = tmp_path / "traffic.txt"
    summary.write_text(f"header: text\nsource_sha256: {gemm}\nhbm_bytes_per_launch: 123\n"
                       f"down_hbm_bytes_per_launch: 45\nmove_source_sha256: {move}\n"
                       f"dispatch_hbm_bytes_per_launch: 6\ncombine_hbm_bytes_per_launch: 7\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    monkeypatch.setattr(bench, "_CSRC", str(csrc))
    got = {k: bench.measured_traffic(k) for k in ("ffn_gateup", "ffn_down", "dispatch", "combine")}
    assert got == {"ffn_gateup": 123, "ffn_down": 45, "dispatch": 6, "combine": 7}
    (csrc / "move.hip").write_text("changed")
    assert bench.measured_traffic("dispatch") is None and bench.measured_traffic("combine") is None
    assert bench.measured_traffic("ffn_gateup") == 123
    (csrc / "gemm.hip").write_text("changed")
    assert bench.measured_traffic("ffn_gateup") is None and bench.measured_traffic("ffn_down") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("ffn_gateup") is None
