"""Pins of the T > 0 verification oracle (oracle/sampling.py) against things other
than itself: numpy's Philox4x64 generator and the published Philox4x32-10
known-answer vectors; the Gumbel-max law; the defining property of speculative
sampling (every emitted token is distributed as the target's conditional),
checked by Monte Carlo with chi-square tests; the T -> 0 limit, which must equal
greedy verification; hand-built tries and walks."""
import json
import math
import os

import numpy as np
import pytest
from scipy.stats import chisquare

import oracle
from oracle import sampling as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_kat.json")


# ------------------------------------------------------------------ generator
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_philox4x64_matches_numpy(seed):
    # numpy's Philox (4x64-10) advances its 256-bit counter before each block: the
    # block at counter c comes first from a generator started at c - 1
    rng = np.random.default_rng(seed)
    for _ in range(20):
        key = [int(x) for x in rng.integers(0, 2 ** 63, 2, dtype=np.int64)]
        ctr = [int(x) for x in rng.integers(1, 2 ** 63, 4, dtype=np.int64)]
        bg = np.random.Philox(key=np.array(key, np.uint64),
                              counter=np.array([ctr[0] - 1] + ctr[1:], np.uint64))
        assert [int(v) for v in bg.random_raw(4)] == S.philox(ctr, key, bits=64)


def test_philox4x32_known_answers():
    kat = json.load(open(GOLDEN))
    for case in kat["philox4x32_10"]:
        ctr = [int(h, 16) for h in case["ctr"]]
        key = [int(h, 16) for h in case["key"]]
        want = [int(h, 16) for h in case["out"]]
        assert S.philox(ctr, key, bits=32) == want
        got = S.philox4x32_np(*[np.array([c]) for c in ctr], *key)
        assert [int(w[0]) for w in got] == want


def test_philox4x32_vectorised_equals_scalar():
    rng = np.random.default_rng(4)
    c = rng.integers(0, 2 ** 32, (4, 64), dtype=np.uint64)
    k0, k1 = 0x9E3779B9, 0x12345678
    vec = S.philox4x32_np(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(64):
        assert [int(w[i]) for w in vec] == S.philox([int(x) for x in c[:, i]], [k0, k1], bits=32)


def test_uniform_mapping():
    u = S.word_to_uniform(np.array([0, 511, 512, 0xFFFFFFFF], np.uint64))
    assert u[0] == u[1] == 2.0 ** -24
    assert u[2] == 3 * 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24
    assert np.all(u.astype(np.float32).astype(np.float64) == u)   # exact in binary32


def test_streams_are_distinct_and_keyed():
    a = S.gumbel_row(7, 3, 16)
    assert not np.array_equal(a, S.gumbel_row(8, 3, 16))           # seed
    assert not np.array_equal(a, S.gumbel_row(7, 4, 16))           # row
    assert not np.array_equal(a, S.gumbel_row(7 + (1 << 32), 3, 16))  # high key word
    assert S.accept_uniform(7, 3, 0) != S.accept_uniform(7, 3, 1)
    # the residual stream (counter word 2 = 0) and the acceptance stream (= 1) differ
    w = S.philox([0, 3, 0, 0], [7, 0])[0]
    assert S.accept_uniform(7, 3, 0) != float(S.word_to_uniform(w))


def test_gumbel_max_samples_softmax():
    # argmax(t + G) over fresh noise follows softmax(t); a wrong sign or a missing
    # log in G shifts these frequencies far beyond chance
    t = np.array([0.0, 1.0, -0.5, 2.0, 0.3, -2.0])
    n = 20000
    counts = np.zeros(len(t))
    for g in range(n):
        counts[int(np.argmax(t + S.gumbel_row(11, g, len(t))))] += 1
    p = np.exp(t - t.max())
    p /= p.sum()
    assert chisquare(counts, n * p).pvalue > 1e-4


# ------------------------------------------------------------------ trie
def test_trie_hand_built():
    W, D = 4, 3
    cand = [[5, 6, 7], [5, 6, 8], [5, 9, -1], [4, -1, -1]]
    L = [3, 3, 2, 1]
    kids = S.candidate_trie(cand, L, True, W, D)
    row = lambda w, j: 1 + w * D + j  # noqa: E731
    assert kids[0] == [(5, 0), (4, 3)]
    assert kids[row(0, 0)] == [(6, 0), (9, 2)]
    assert kids[row(0, 1)] == [(7, 0), (8, 1)]
    for r in (row(0, 2), row(1, 2), row(2, 1), row(3, 0), row(1, 0), row(2, 0), row(1, 1)):
        assert kids[r] == [], r
    assert S.candidate_trie(cand, L, False, W, D)[0] == []


def test_trie_duplicates_and_truncation():
    # identical candidates share every node; a candidate that ends early keeps its
    # group's node but adds no child
    W, D = 3, 2
    kids = S.candidate_trie([[1, 2], [1, 2], [1, -1]], [2, 2, 1], True, W, D)
    assert kids[0] == [(1, 0)]
    assert kids[1] == [(2, 0)]
    assert kids[2] == [] and kids[1 + D] == [] and kids[1 + 2 * D] == []


# ------------------------------------------------------------------ the walk
def test_walk_hand_example_with_injected_streams():
    V, W, D, T = 5, 1, 2, 1.0
    logits = {0: np.log([0.5, 0.1, 0.2, 0.1, 0.1]), 1: np.log([0.1, 0.1, 0.1, 0.6, 0.1]),
              2: np.log([0.2] * 5)}
    seen = []

    def draw(row, g, excl):
        seen.append((row, tuple(excl)))
        return 4

    def run(us):
        it = iter(us)
        seen.clear()
        return S.sample_step(lambda r: logits[r], [[0, 3]], [2], True, W, D, T, 0, 0,
                             uniform=lambda g, k: next(it), draw=draw)

    r = run([0.49, 0.59])                 # 0.49 < p(0) = 0.5; 0.59 < p(3) = 0.6
    assert (r["best_w"], r["best_len"], r["tokens"]) == (0, 2, [0, 3])
    assert seen == [(2, ())]              # bonus draw at the leaf, nothing excluded
    r = run([0.51])                       # rejected at the root: residual without token 0
    assert (r["best_len"], r["next_token"]) == (0, 4) and seen == [(0, (0,))]
    r = run([0.1, 0.61])                  # rejected at depth 1: residual of row 1 without 3
    assert (r["best_len"], r["tokens"]) == (1, [0]) and seen == [(1, (3,))]
    assert r["decisions"] == [(0, 0, 0.1, pytest.approx(0.5)), (1, 0, 0.61, pytest.approx(0.6))]


def test_second_child_uses_the_residual_probability():
    # root children 0 then 1; p = (0.5, 0.3, 0.2): after rejecting 0, token 1 is
    # accepted with 0.3 / 0.5 = 0.6
    logits = {0: np.log([0.5, 0.3, 0.2]), 1: np.log([1 / 3] * 3), 3: np.log([1 / 3] * 3)}
    it = iter([0.9, 0.59])
    r = S.sample_step(lambda row: logits[row], [[0, 0], [1, 0]], [1, 1], True, 2, 2, 1.0, 0, 0,
                      uniform=lambda g, k: next(it), draw=lambda row, g, e: 2)
    assert r["tokens"] == [1] and r["best_w"] == 1
    assert r["decisions"][1][3] == pytest.approx(0.6)


def test_closed_gate():
    r = S.sample_step(lambda row: None, [[1]], [1], False, 1, 1, 1.0, 0, 0)
    assert (r["best_w"], r["best_len"], r["next_token"]) == (-1, 0, -1)


def _consistent_model(rng, V, scale, fixed=None):
    """A target whose next-token logits depend only on the prefix (a dict cache);
    `fixed` maps some prefixes to given probabilities."""
    table = {k: np.log(np.asarray(v, dtype=np.float64)) for k, v in (fixed or {}).items()}

    def logits(prefix):
        key = tuple(prefix)
        if key not in table:
            table[key] = rng.standard_normal(V) * scale
        return table[key]
    return logits


def _row_logits(model, cand, W, D):
    def f(row):
        if row == 0:
            return model([])
        w, j = divmod(row - 1, D)
        return model(list(cand[w][:j + 1]))
    return f


def test_emitted_tokens_follow_the_target():
    # the defining property of speculative sampling: whatever the drafts, the
    # emitted sequence (accepted tokens, then the drawn one) has the target's law.
    # Candidates share prefixes and collide with likely tokens; 3 levels deep.
    # The tried children carry real mass (0.4 and 0.3 at the root, 0.45 and 0.3
    # below token 1), so a rule that skips the residual renormalisation, or that
    # draws without removing the rejected children, misses by many sigmas.
    V, W, D, T = 4, 4, 2, 1.0
    rng = np.random.default_rng(3)
    model = _consistent_model(rng, V, 1.2, fixed={(): [0.1, 0.4, 0.2, 0.3],
                                                  (1,): [0.3, 0.1, 0.45, 0.15]})
    cand = [[1, 2], [1, 0], [3, 1], [1, 2]]
    L = [2, 2, 2, 1]
    f = _row_logits(model, cand, W, D)
    n = 30000
    obs = {}
    for s in range(n):
        r = S.sample_step(f, cand, L, True, W, D, T, s, 0)
        seq = tuple(r["tokens"]) + (r["next_token"],)
        obs[seq] = obs.get(seq, 0) + 1

    def prob(seq):
        p = 1.0
        for i, x in enumerate(seq):
            p *= S.softmax_T(model(list(seq[:i])), T)[x]
        return p
    kids = S.candidate_trie(cand, L, True, W, D)

    def emitted(prefix, row, depth):
        # every complete emitted sequence reachable from this node, with its law
        out = []
        ch = {x: w for x, w in kids[row]}
        for x in range(V):
            if x in ch:
                out += emitted(prefix + (x,), 1 + ch[x] * D + depth, depth + 1)
            else:
                out.append(prefix + (x,))
        return out
    seqs = emitted((), 0, 0)
    exp = np.array([prob(q) for q in seqs])
    assert abs(exp.sum() - 1.0) < 1e-12
    got = np.array([obs.get(q, 0) for q in seqs], dtype=float)
    assert got.sum() == n                              # nothing emitted outside the tree
    assert chisquare(got, n * exp).pvalue > 1e-4


def test_plain_rejection_without_residual_would_fail():
    # guard of the test above: accepting the second child with p(x) instead of
    # p(x) / (1 - tried) changes the law by far more than the test tolerates
    V, T = 3, 1.0
    p = S.softmax_T(np.log([0.5, 0.3, 0.2]), T)
    right = 0.5 * 0.6          # P(emit token 1 first) under the rule: rejected 0, then 0.3/0.5
    wrong = 0.5 * 0.3
    assert abs(right - p[1]) < 1e-12 and abs(wrong - p[1]) > 0.1


@pytest.mark.parametrize("seed", range(6))
def test_low_temperature_equals_greedy(seed):
    # as T -> 0 each row's law concentrates on its argmax: the walk accepts exactly
    # the candidates' agreement with the greedy choices, as accept_longest does
    rng = np.random.default_rng(100 + seed)
    V, W, D = 6, 5, 4
    model = _consistent_model(rng, V, 3.0)
    base = rng.integers(0, V, D)
    cand = []
    for w in range(W):
        c = base.copy()
        cut = int(rng.integers(0, D + 1))
        c[cut:] = rng.integers(0, V, D - cut)
        cand.append([int(x) for x in c])
    L = [int(x) for x in rng.integers(1, D + 1, W)]
    f = _row_logits(model, cand, W, D)
    R = 1 + W * D
    am = np.array([[int(np.argmax(f(r))) for r in range(R)]])
    greedy = oracle.accept_longest(np.array([cand]), np.array([L]), np.array([1]), am, W, D)
    r = S.sample_step(f, cand, L, True, W, D, 1e-4, seed, 0)
    assert r["best_len"] == greedy["best_len"][0]
    assert r["next_token"] == greedy["next_token"][0]
    assert r["best_w"] == greedy["best_w"][0]


def test_batch_form_matches_steps():
    rng = np.random.default_rng(5)
    B, W, D, V = 3, 2, 3, 7
    logits = rng.standard_normal((B, 1 + W * D, V))
    cand = rng.integers(0, 3, (B, W, D))
    L = np.array([[3, 2], [1, 3], [2, 2]])
    gate = np.array([1, 0, 1])
    out = S.sample_verify(logits, cand, L, gate, W, D, 0.7, 99)
    for b in range(B):
        r = S.sample_step(lambda row: logits[b][row], cand[b], L[b], bool(gate[b]), W, D, 0.7, 99, b)
        assert (out["best_w"][b], out["best_len"][b], out["next_token"][b]) == \
            (r["best_w"], r["best_len"], r["next_token"])
    assert out["best_w"][1] == -1
