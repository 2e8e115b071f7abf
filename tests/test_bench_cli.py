"""bench.py on the host: the one-GPU contract and the stored counter summary."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_matches_the_current_gemv_sources():
    """The HBM byte counts in the gate/up counter summary were taken on the
    GEMV sources as they stand (bench.py reports them only then)."""
    sys.path.insert(0, ROOT)
    import bench
    t = bench.stored_traffic()
    assert t is not None, "re-take the gate/up FETCH_SIZE / WRITE_SIZE counters"
    assert 631_301_120 <= t <= 1.05 * 631_301_120
