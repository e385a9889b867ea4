"""fp4attn_clock_probe on the GPU: the shader clock from s_memtime over s_memrealtime agrees with
the clock implied by the probe's own wall time (its loop is a fixed number of instructions per
wave, so a slower clock must show as a longer loop), and lies within the MI355X's range."""
import pytest

from tests.gpuhelpers import require_gpu

pytestmark = pytest.mark.gpu


def test_clock_probe_range_and_consistency():
    import precision_attention_amd as pa

    require_gpu()
    for _ in range(3):  # warm the clocks
        pa.clock_probe(iters=8000)
    a = pa.clock_probe(iters=8000)
    b = pa.clock_probe(iters=16000)
    print("clock probe: %s / %s" % (a, b), flush=True)
    for r in (a, b):
        assert 0.5 <= r["ghz_min"] <= r["ghz_median"] <= r["ghz_max"] <= 3.0
        assert r["ghz_max"] - r["ghz_min"] < 0.2 * r["ghz_median"]
        assert r["realtime_khz"] > 0
    # twice the iterations take about twice the time at about the same clock
    assert 1.7 <= b["loop_ms"] / a["loop_ms"] <= 2.3
    assert abs(a["ghz_median"] - b["ghz_median"]) < 0.15 * b["ghz_median"]
