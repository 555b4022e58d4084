"""CPU tests of the benchmark's host arithmetic and its command line."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("nq,nk", [(1, 1), (5, 5), (7, 3), (3, 7), (1, 9), (9, 1), (64, 100), (100, 64)])
def test_visible_pairs_brute_force(nq, nk):
    mask = np.arange(nk)[None, :] <= (np.arange(nq) + nk - nq)[:, None]
    assert bench.visible_pairs(nq, nk, True) == int(mask.sum())
    assert bench.visible_pairs(nq, nk, False) == nq * nk


def test_workload_figures():
    fl = bench.attention_flops(2, 16, 4096, 4096, 128, True)
    assert fl["fwd"] == 137_472_507_904                      # 4 d B H N(N+1)/2
    assert fl["dkdv"] + fl["dq"] == 343_681_269_760          # 2.5 x forward
    assert bench.attention_flops(1, 16, 16384, 16384, 128, True)["fwd"] == 1_099_578_736_640
    assert bench.attention_flops(4, 8, 1024, 1024, 64, False)["fwd"] == 8_589_934_592
    assert bench.decode_bytes(8, 32, 8, 32768, 128, 2) == 1_073_939_488


def test_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
