"""Host-side checks of the benchmark's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_traffic_record_matches_the_kernel_sources():
    # the HBM byte counts in bench.py were measured on the current Direct-P sources; after a
    # change to them the counters must be taken again (bench.py would report traffic null)
    import bench

    assert bench.measured_traffic() is not None, (bench.MEASURED_TRAFFIC, bench.sources_sha())


def test_mixed_peaks():
    import bench

    assert abs(bench.PEAK_FWD_FP4_FP8_TFLOPS - 6715.5) < 1.0
    assert abs(bench.PEAK_BWD_TFLOPS - 5591.3) < 1.0
