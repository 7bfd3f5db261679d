"""Pins for the oracle's kappa-gram evidence and retrieval.

SwitchSD write-up §2.5 (gate: the kappa-gram ending at the current token occurred
before), paper §3.3 "Copy-Based Speculative Generation" and write-up §2.6 (up to
W continuations of up to D tokens, ranked by recency).

The brute-force reference below uses a different algorithm from the oracle's
backward walk: it indexes every kappa-gram of the context in a dictionary and
reads off the suffix's positions.  Hand-built cases pin the readings (suffix
excluded, newest first, truncated recent candidates kept).
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def _one(x, kappa, W, D, fire=None):
    cu = np.array([0, len(x)], dtype=np.int32)
    f = None if fire is None else np.array([fire])
    r = oracle.kgram_retrieve(np.array(x, dtype=np.int32), cu, kappa, W, D, f)
    return {k: v[0] for k, v in r.items()}


def test_hand_built_two_earlier_occurrences():
    # x: 7 1 2 3 4 1 2 3 9 9 1 2 3   (n = 13, suffix [1,2,3] at 10..12)
    # earlier [1,2,3] end at p = 3 and p = 7; newest first -> [7, 3]
    # cand(p=7) = x[8..11] = 9 9 1 2 ; cand(p=3) = x[4..7] = 4 1 2 3 ; L = min(4, 12 - p) = 4
    x = [7, 1, 2, 3, 4, 1, 2, 3, 9, 9, 1, 2, 3]
    r = _one(x, 3, 2, 4)
    assert list(r["match_end"]) == [7, 3]
    assert r["n_match"] == 2 and bool(r["copy_gate"])
    assert r["cand"].tolist() == [[9, 9, 1, 2], [4, 1, 2, 3]]
    assert list(r["cand_len"]) == [4, 4]
    r3 = _one(x, 3, 3, 4)
    assert r3["n_match"] == 2 and list(r3["match_end"]) == [7, 3, -1]
    assert r3["cand"][2].tolist() == [-1, -1, -1, -1] and r3["cand_len"][2] == 0
    r1 = _one(x, 3, 1, 4)                     # W = 1 keeps only the newest
    assert list(r1["match_end"]) == [7]


def test_periodic_closed_form():
    # period 3: x = [1,2,3]*3 + [1], suffix (kappa=3) = [2,3,1]; occurrences end at
    # p = n-1-3k for k >= 1 with p >= kappa-1:  p = 6, 3
    x = [1, 2, 3] * 3 + [1]
    r = _one(x, 3, 10, 5)
    assert list(r["match_end"][:2]) == [6, 3] and r["n_match"] == 2
    assert r["cand"][0][:3].tolist() == [2, 3, 1]       # x[7..9], L = min(5, 9 - 6) = 3
    assert r["cand"][1].tolist() == [2, 3, 1, 2, 3]     # x[4..8]
    assert r["cand_len"][0] == 3 and r["cand_len"][1] == 5


def test_constant_context_lengths():
    # constant run: every p = n-2, n-3, ... matches; L_w = min(D, n-1-p) = 1, 2, ...
    n, kappa, W, D = 30, 5, 10, 20
    r = _one([5] * n, kappa, W, D)
    assert list(r["match_end"]) == list(range(n - 2, n - 2 - W, -1))
    assert list(r["cand_len"]) == list(range(1, W + 1))
    for w in range(W):
        L = r["cand_len"][w]
        assert np.all(r["cand"][w][:L] == 5) and np.all(r["cand"][w][L:] == -1)


def test_truncated_recent_candidates_are_kept():
    # suffix match ends 2 tokens before the anchor -> L = 2 < D, still kept first
    x = [9, 8, 1, 2, 3, 4, 5, 6, 1, 2, 3, 1, 2, 3]
    r = _one(x, 3, 4, 6)
    # suffix [1,2,3] (11..13); earlier ends: p = 10 (x[8..10]), p = 4 (x[2..4])
    assert list(r["match_end"][:2]) == [10, 4]
    assert list(r["cand_len"][:2]) == [3, 6]
    assert r["cand"][0][:3].tolist() == [1, 2, 3]


def test_distinct_ids_and_short_contexts_give_no_match():
    r = _one(list(range(50)), 5, 10, 20)
    assert r["n_match"] == 0 and not bool(r["copy_gate"]) and np.all(r["match_end"] == -1)
    for n in range(1, 6):                      # n <= kappa: no earlier occurrence possible
        r = _one([4] * n, 5, 10, 20)
        assert r["n_match"] == 0
    r = _one([4] * 6, 5, 10, 20)               # n = kappa + 1: only p = kappa-1 = n-2
    assert list(r["match_end"][:1]) == [4] and r["cand_len"][0] == 1


def test_probe_off_retrieves_nothing():
    x = [1, 2, 3, 1, 2, 3]
    r = _one(x, 3, 4, 4, fire=False)
    assert r["n_match"] == 0 and not bool(r["copy_gate"]) and np.all(r["cand"] == -1)
    r = _one(x, 3, 4, 4, fire=True)
    assert r["n_match"] == 1


def _brute(x, kappa, W, D):
    """kappa-gram index -> positions, then the suffix's earlier ends, newest first."""
    n = len(x)
    index = {}
    for end in range(kappa - 1, n):
        index.setdefault(tuple(x[end - kappa + 1:end + 1]), []).append(end)
    if n < kappa + 1:
        return [], []
    ends = sorted((p for p in index[tuple(x[n - kappa:])] if p <= n - 2), reverse=True)[:W]
    cands = [list(x[p + 1:p + 1 + D]) for p in ends]
    return ends, cands


@settings(max_examples=300, deadline=None)
@given(st.lists(st.lists(st.integers(0, 3), min_size=1, max_size=64), min_size=1, max_size=4),
       st.integers(1, 5), st.integers(1, 12), st.integers(1, 25))
def test_brute_force_batch(seqs, kappa, W, D):
    ids = np.array([t for s in seqs for t in s], dtype=np.int32)
    cu = np.zeros(len(seqs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum([len(s) for s in seqs])
    r = oracle.kgram_retrieve(ids, cu, kappa, W, D)
    for b, s in enumerate(seqs):
        ends, cands = _brute(s, kappa, W, D)
        M = len(ends)
        assert r["n_match"][b] == M
        assert bool(r["copy_gate"][b]) == (M > 0)
        assert list(r["match_end"][b][:M]) == ends and np.all(r["match_end"][b][M:] == -1)
        for w in range(W):
            want = cands[w] if w < M else []
            assert r["cand_len"][b][w] == len(want)
            assert r["cand"][b][w][:len(want)].tolist() == want
            assert np.all(r["cand"][b][w][len(want):] == -1)


def test_generated_full_shape_anchor_has_w_candidates():
    from workloads import generate
    wl = generate("small_bf16", with_tensors=False)
    s = wl.spec
    r = oracle.kgram_retrieve(wl.ids, wl.cu_len, s.kappa, s.W, s.D)
    assert np.all(r["n_match"] == s.W)
    for b in range(s.B):
        x = wl.ids[wl.cu_len[b]:wl.cu_len[b + 1]]
        ends, _ = _brute(list(x), s.kappa, s.W, s.D)
        assert list(r["match_end"][b]) == ends
