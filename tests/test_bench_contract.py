"""Host-side checks of bench.py's command-line contract (no GPU needed):
more than one GPU is refused with a JSON message before any device work, and
the byte and flop counts it reports against come from the per-token formulas
stated with the roofline."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_per_token_counts():
    sys.path.insert(0, ROOT)
    import bench
    # q, k, v, o at 2 bytes, g at 4 bytes per channel, beta at 4: 1540 B for d = 128 bf16
    assert bench.bytes_per_token_head(128, 128, 2) == 1540
    assert bench.bytes_per_token_head(64, 64, 4) == 4 * 64 * 4 + 4 * 64 + 4
    # chunked form at C = 64, d = 128, triangles exploited: 141,013 flop
    assert round(bench.chunk_flops_per_token_head(64, 128, 128)) == 141013
