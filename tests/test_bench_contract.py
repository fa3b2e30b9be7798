"""bench.py's command-line contract on the host (no GPU): the path runs on one GPU, so any
other --gpus value exits with status 2 and says why, before touching the device; the
attention traffic figure is either the calibrated counter bytes of the current kernel
source or null."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_attention_traffic_is_counter_bytes_or_null():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.attention_traffic_bytes()
    c = bench.ATTN_COUNTERS
    if t is not None:
        assert t == (c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024.0
        # at least the algorithmic Q, K, V read and O written once (480p, f16)
        assert t >= 4 * 33272 * 3072 * 2
