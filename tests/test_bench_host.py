"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte counts of the
workloads, the peaks derived from the chip's unit counts, and the source-hash gate on the
committed traffic figures (a summary taken on other kernel sources is not reported)."""
import json
import os
import subprocess
import sys

import bench
from selective_scan_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_workloads():
    """Each tensor read once, each output written once: x + four routes' delta + B/C + z + out."""
    assert bench.algorithmic_bytes(synth.STAGE1) == 1_181_745_152      # 154.1 + 616.6 + 102.8 + 154.1 + 154.1 MB
    assert bench.algorithmic_bytes(synth.STAGE3) == 276_168_704        # 38.5 + 154.1 + 6.4 + 38.5 + 38.5 MB
    assert bench.algorithmic_bytes(synth.LOWSTATE) == 468_844_544      # 77.1 + 308.3 + 6.4 + 0 + 77.1 MB
    assert bench.algorithmic_bytes(synth.HIGHRES) == 385_875_968       # fp32: 50.3 + 201.3 + 33.6 + 50.3 + 50.3 MB
    assert bench.algorithmic_bytes(synth.TINY) == 36_864
    # the backward adds dout, dx, ddelta, dB, dC, dz
    hb = bench.algorithmic_bytes(synth.HIGHRES, bwd=True) - bench.algorithmic_bytes(synth.HIGHRES)
    assert hb == 4 * (2 * 12_582_912 + 4 * 12_582_912 + 2 * 4 * 4 * 16 * 16384 + 12_582_912)


def test_peaks_from_unit_counts():
    # 1024 SIMDs x 16 fp32 lanes x 2 flops x 2.4 GHz; the mix: 4 full-rate ops (4 cycles each) and
    # one transcendental (8 cycles) per 64 (element, state) units, 7 flops each
    assert abs(bench.VALU_PEAK_TFLOPS - 78.6432) < 1e-9
    assert abs(bench.MIX_PEAK_TFLOPS - 1024 * 2.4e9 * 64 / 24 * 7 / 1e12) < 1e-9
    assert bench.PUBLISHED_FP32_VECTOR_TFLOPS == 157.3


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    rec = {"w": {"hbm_bytes_per_launch": 123.0, "kernel_source_sha": "abc"}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "scan_fwd_traffic.txt").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("w", "abc") == 123.0
    assert bench.load_traffic("w", "abd") is None
    assert bench.load_traffic("other", "abc") is None

