"""Host-side checks of the large-array scan inputs and of the algorithmic byte count
the scan bench reports (no GPU).

The planted-context generator is pinned by brute force: an index of every
kappa-gram's end positions (a different algorithm from the oracle's backward
walk) must contain every planted end, and the oracle must return exactly the W
newest positions of that index.
"""
import os
import sys
from collections import defaultdict

import numpy as np
import pytest

import oracle
from workloads import scan_ids_planted

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _ends_by_index(x, kappa):
    idx = defaultdict(list)
    for p in range(kappa - 1, len(x)):
        idx[tuple(x[p - kappa + 1:p + 1])].append(p)
    return idx


@pytest.mark.parametrize("kappa", [1, 3, 5, 9])
def test_planted_occurrences_are_found(kappa):
    lens = [9000, 8193, 40, 6, 17000]
    ids, cu = scan_ids_planted(lens, kappa=kappa, seed=4400 + kappa)
    assert ids.dtype == np.int32 and cu.tolist() == [0] + np.cumsum(lens).tolist()
    W, D = 64, 20
    r = oracle.kgram_retrieve(ids, cu, kappa, W, D)
    for b, n in enumerate(lens):
        x = [int(v) for v in ids[cu[b]:cu[b + 1]]]
        if n < kappa + 1:
            assert r["n_match"][b] == 0
            continue
        ends = [p for p in _ends_by_index(x, kappa)[tuple(x[n - kappa:])] if p <= n - 2]
        expect = sorted(ends, reverse=True)[:W]
        assert r["n_match"][b] == len(expect)
        assert r["match_end"][b, :len(expect)].tolist() == expect


def test_planted_generator_is_deterministic_and_seeded():
    a = scan_ids_planted([5000, 300], seed=7)
    b = scan_ids_planted([5000, 300], seed=7)
    c = scan_ids_planted([5000, 300], seed=8)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    assert not np.array_equal(a[0], c[0])


def test_scan_algorithmic_bytes():
    # full scans read every id; a context with W matches reads back to the W-th
    # match's first id; offsets, gathered ids and outputs are added once
    n = np.array([100, 100, 50])
    W, D, kappa = 2, 3, 5
    n_match = np.array([0, 2, 1])
    last_end = np.array([-1, 40, -1])
    cand_len = np.array([[0, 0], [3, 3], [2, 0]])
    scanned = 100 + (100 - 40 + kappa - 1) + 50
    out = 3 * (4 * W + 4 + 4 * W * D + 4 * W + 1)
    expect = 4 * scanned + 4 * 4 + 4 * 8 + out
    assert bench.scan_algorithmic(n, kappa, W, D, n_match, last_end, cand_len) == expect
