"""The benchmark's host-side contract, on the CPU: the one-GPU refusal and the
tile and K-pass counts it reports for the scheduling comparison."""
import json
import os
import subprocess
import sys

import numpy as np

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_tile_counts_worked_example():
    """MLX PR 4567 (Proposed changes): loads 13 / 8 / 2 / 10 at BM 16 are 4
    expert-aware tiles, one K pass each, against 3 naive tiles that make 6
    K passes (one per expert a tile touches)."""
    counts = np.array([13, 8, 2, 10])
    assert bench.tile_counts(counts, 16, "scheduled", 512) == (4, 4)
    assert bench.tile_counts(counts, 16, "naive", 512) == (3, 6)


def test_two_size_count_matches_the_oracle_tables():
    """The report's host count of the two-size schedule equals the number of
    entries in the oracle's tables, on both sides of the small-tile switch."""
    g = np.random.default_rng(11)
    for trial in range(200):
        E = int(g.integers(1, 300))
        scale = g.choice([1, 4, 40, 400])
        counts = (g.zipf(1.3, E) * scale // 4).astype(np.int64) * (g.random(E) < 0.7)
        counts = np.minimum(counts, 5000)
        inter = int(g.choice([512, 1024, 2048]))
        offsets = np.concatenate([[0], np.cumsum(counts)])
        big, small = oracle.hybrid_tiles(offsets, 0, col_blocks=inter // 128)
        assert bench.hybrid_tile_count(counts, inter) == len(big) + len(small), (trial, inter)
