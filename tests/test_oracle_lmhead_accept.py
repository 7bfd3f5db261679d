"""Pins for the oracle's LM head + argmax and for longest-accept.

LM head: SwitchSD paper §3.3 (one target forward pass verifies all candidates),
write-up §3.1 (T = 0): the target's choice per row is the argmax of the logits.
Accept: paper §3.3 (the candidate with the longest verified continuation is
kept); the VIA-SD page's "Draft–Verify and Lossy Acceptance" (acceptance halts at
the first rejected token).

References here: hand-computed logits, Python-loop dot products on non-square
shapes (a transposed weight fails), planted argmax columns, a hand-computed
acceptance example, a vectorised prefix-compare formulation, and a chained
check that blocktri verification + accept equals plain greedy decoding of each
candidate (paper §3.3 "Overall Framework": correctness is preserved).
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


# ---------------------------------------------------------------- LM head
def test_hand_logits_and_margin():
    O = np.array([[1.0, 2.0]], np.float32)
    Wt = np.array([[1, 0], [0, 1], [1, 1], [-1, 3]], np.float32)     # [V=4, hid=2]
    r = oracle.lmhead_argmax(O, Wt)
    assert r["logits"].tolist() == [[1.0, 2.0, 3.0, 5.0]]
    assert r["pred"][0] == 3 and r["margin"][0] == 2.0


def test_ties_go_to_lowest_index():
    pred, top1, margin = oracle.argmax_with_margin(np.array([[2.0, 5.0, 5.0, 1.0],
                                                             [7.0, 7.0, 7.0, 7.0]]))
    assert pred.tolist() == [1, 0] and margin.tolist() == [0.0, 0.0]


def test_loop_dot_products_non_square():
    rng = np.random.default_rng(3)
    O = rng.standard_normal((3, 5)).astype(np.float32)
    Wt = rng.standard_normal((7, 5)).astype(np.float32)
    got = oracle.lm_logits(O, Wt)
    assert got.shape == (3, 7)
    for r in range(3):
        for v in range(7):
            want = math.fsum(float(O[r, k]) * float(Wt[v, k]) for k in range(5))
            assert got[r, v] == pytest.approx(want, abs=1e-12)


def test_planted_column_wins_with_bf16_inputs():
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(4)
    O = rng.standard_normal((6, 64)).astype(np.float32)
    Wt = (0.02 * rng.standard_normal((500, 64))).astype(np.float32)
    targets = [0, 499, 17, 250, 250, 3]
    for r, v in enumerate(targets):
        Wt[v] += 0.0                                  # keep the weight; plant through O
    # row r gets a large component along Wt[target] so that logit[target] dominates
    for r, v in enumerate(targets):
        O[r] = 50.0 * Wt[v] / np.linalg.norm(Wt[v]) ** 2 + 0.01 * O[r]
    r = oracle.lmhead_argmax(f32_to_bf16_bits(O), f32_to_bf16_bits(Wt))
    assert r["pred"].tolist() == targets


# ---------------------------------------------------------------- accept
def _acc(cand, lens, argmax, W, D, gate=True):
    r = oracle.accept_longest(np.array([cand]), np.array([lens]), np.array([gate]),
                              np.array([argmax]), W, D)
    return {k: v[0] for k, v in r.items()}


def _argmax_rows(p0, preds, W, D):
    a = [p0] + [-1] * (W * D)
    for w, pw in enumerate(preds):
        for j, t in enumerate(pw):
            a[1 + w * D + j] = t
    return a


def test_hand_computed_example():
    # cand = [[5,6,7,8],[5,6,9,9],[4,1,1,1]]; anchor row predicts 5;
    # pred(0,.) = [6,7,1,2], pred(1,.) = [6,9,9,3], pred(2,.) = [0,0,0,0]
    # a_0: 5=5, 6=6, 7=7, 8!=1 -> 3 ; a_1: 5,6,9,9 all agree -> 4 ; a_2: 4!=5 -> 0
    # best_w = 1, best_len = 4, next = pred(1,3) = 3
    W, D = 3, 4
    am = _argmax_rows(5, [[6, 7, 1, 2], [6, 9, 9, 3], [0, 0, 0, 0]], W, D)
    r = _acc([[5, 6, 7, 8], [5, 6, 9, 9], [4, 1, 1, 1]], [4, 4, 4], am, W, D)
    assert r["accept_len"].tolist() == [3, 4, 0]
    assert (r["best_w"], r["best_len"], r["next_token"]) == (1, 4, 3)


def test_tie_goes_to_most_recent_and_partial_next_token():
    # a = [2, 2, 0] -> best_w = 0; next = pred(0, 1) = 9 (the target's correction)
    W, D = 3, 4
    am = _argmax_rows(5, [[6, 9, 0, 0], [6, 8, 0, 0], [0, 0, 0, 0]], W, D)
    r = _acc([[5, 6, 7, 8], [5, 6, 7, 7], [1, 1, 1, 1]], [4, 4, 4], am, W, D)
    assert r["accept_len"].tolist() == [2, 2, 0]
    assert (r["best_w"], r["best_len"], r["next_token"]) == (0, 2, 9)


def test_candidate_length_caps_acceptance():
    # predictions would keep agreeing, but L_0 = 2 stops the walk
    W, D = 2, 4
    am = _argmax_rows(5, [[6, 7, 8, 9], [0, 0, 0, 0]], W, D)
    r = _acc([[5, 6, 7, 8], [5, -1, -1, -1]], [2, 1], am, W, D)
    assert r["accept_len"].tolist() == [2, 1]
    assert (r["best_w"], r["best_len"], r["next_token"]) == (0, 2, 7)


def test_nothing_accepted_and_closed_gate():
    W, D = 2, 3
    am = _argmax_rows(42, [[1, 1, 1], [1, 1, 1]], W, D)
    r = _acc([[7, 7, 7], [8, 8, 8]], [3, 3], am, W, D)
    assert r["accept_len"].tolist() == [0, 0]
    assert (r["best_w"], r["best_len"], r["next_token"]) == (0, 0, 42)
    r = _acc([[42, 1, 1], [8, 8, 8]], [3, 3], am, W, D, gate=False)
    assert r["accept_len"].tolist() == [0, 0]
    assert (r["best_w"], r["best_len"], r["next_token"]) == (-1, 0, -1)


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 6), st.integers(1, 8), st.integers(0, 2 ** 31 - 1))
def test_prefix_compare_formulation(W, D, seed):
    # a_w = number of leading True in (cand[w] == [p0] + pred_w[:-1]) over j < L_w
    rng = np.random.default_rng(seed)
    cand = rng.integers(0, 3, (W, D))
    lens = rng.integers(0, D + 1, W)
    argmax = rng.integers(0, 3, 1 + W * D)
    # make long agreements likely: copy candidate tokens into the predictions
    for w in range(W):
        for j in range(D - 1):
            if rng.random() < 0.7:
                argmax[1 + w * D + j] = cand[w, j + 1]
    if rng.random() < 0.7:
        argmax[0] = cand[0, 0]
    r = _acc(cand.tolist(), lens.tolist(), argmax.tolist(), W, D)
    for w in range(W):
        prev = np.concatenate([[argmax[0]], argmax[1 + w * D:1 + w * D + D - 1]])
        ok = (cand[w] == prev) & (np.arange(D) < lens[w])
        want = int(np.argmin(ok)) if not ok.all() else D
        assert r["accept_len"][w] == want
        assert 0 <= r["accept_len"][w] <= lens[w] <= D
    best = int(np.argmax(r["accept_len"]))
    assert r["best_w"] == best and r["best_len"] == r["accept_len"][best]


def test_blocktri_plus_accept_equals_greedy_decoding(page_constants):
    """Chained: verification of all candidates in one pass accepts exactly what plain
    greedy decoding of the one-layer synthetic target would emit, candidate by candidate."""
    rng = np.random.default_rng(11)
    n, W, D, d, V = 9, 3, 4, 8, 6
    # a tiny 'target': token embeddings feed q/k/v directly, logits = O . E^T
    E = rng.standard_normal((V, d))
    x = list(rng.integers(0, V, n))
    cands = [list(rng.integers(0, V, D)) for _ in range(W)]
    Lw = [4, 3, 2]

    def emb(t):
        return E[t].astype(np.float32)

    k_pre = np.stack([emb(t) for t in x])[:, None, :]
    q = np.zeros((1, 1 + W * D, 1, d), np.float32)
    k_c = np.zeros((1, W * D, 1, d), np.float32)
    q[0, 0, 0] = emb(x[-1])
    for w in range(W):
        for j in range(D):
            q[0, 1 + w * D + j, 0] = emb(cands[w][j])
            k_c[0, w * D + j, 0] = emb(cands[w][j])
    out, _ = oracle.blocktri_attention(q, k_pre, k_pre, np.array([0, n]), k_c, k_c,
                                       np.array([Lw]), np.array([True]), 1, 1, d, W, D)
    am = np.full((1, 1 + W * D), -1)
    real = [0] + [1 + w * D + j for w in range(W) for j in range(Lw[w])]
    am[0, real] = oracle.lmhead_argmax(out[0, real], E)["pred"]
    # force some agreement so acceptance is non-trivial: rewrite candidates to follow
    # the target's own predictions where the draw allows, then re-verify
    for w in range(W):
        cands[w][0] = int(am[0, 0])
    for w in range(W):
        for j in range(D):
            q[0, 1 + w * D + j, 0] = emb(cands[w][j])
            k_c[0, w * D + j, 0] = emb(cands[w][j])
    out, _ = oracle.blocktri_attention(q, k_pre, k_pre, np.array([0, n]), k_c, k_c,
                                       np.array([Lw]), np.array([True]), 1, 1, d, W, D)
    am[0, real] = oracle.lmhead_argmax(out[0, real], E)["pred"]
    acc = oracle.accept_longest(np.array([cands]), np.array([Lw]), np.array([True]), am, W, D)

    def greedy_next(ctx):
        # one causal step of the same target on context ctx (queries the last token)
        K = np.stack([E[t] for t in ctx])
        s = K @ E[ctx[-1]] / math.sqrt(d)
        p = np.exp(s - s.max())
        o = (p / p.sum()) @ K
        return int(np.argmax(E @ o))

    for w in range(W):
        a = 0
        ctx = list(x)
        while a < Lw[w] and greedy_next(ctx) == cands[w][a]:
            ctx.append(cands[w][a])
            a += 1
        assert acc["accept_len"][0, w] == a
    assert acc["accept_len"].max() >= 1
    assert acc["accept_len"].max() <= page_constants["max_speculative_length"]["value"]
