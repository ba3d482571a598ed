"""Host-side checks of bench.py's bookkeeping (no GPU): the committed counter summary belongs
to the indexer source in the tree, so the bench reports measured HBM traffic, and the
single-GPU contract refuses more GPUs."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_summary_matches_indexer_source():
    t = bench.measured_traffic()
    assert t is not None, ("profiles/indexer_c2_traffic.txt was taken for another indexer.hip: "
                           "take the FETCH_SIZE / WRITE_SIZE passes again")
    # the calibrated traffic is within a few percent of the algorithmic bytes (no re-reads)
    alg = 16 * (32768 * 128 + 64 * 128 + 2 * 64)
    assert 0.95 * alg <= t <= 1.2 * alg


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
