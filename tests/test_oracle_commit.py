"""Pins for the oracle's commit of the accepted draft into the KV cache.

SwitchSD paper §3.3 "Parallel Verification": the longest validated
continuation is kept and extends the context.  The VIA-SD page's "Draft–Verify
and Lossy Acceptance" fixes the token that follows an accepted prefix under
greedy decoding.

References: a hand-built two-sequence case with every copied value spelled out,
the capacity and closed-gate cases, and a chained check on a one-layer
synthetic target.  After verify, accept and commit, the context equals what
plain greedy decoding emits, and the cache holds the keys of every context token
but the new anchor.
"""
import math

import numpy as np

import oracle


def test_hand_built_commit():
    B, W, D, Hkv, d = 2, 2, 3, 1, 2
    k_cand = np.arange(B * W * D * Hkv * d, dtype=np.float32).reshape(B, W * D, Hkv, d)
    v_cand = -k_cand
    cand = np.array([[[10, 11, 12], [20, 21, 22]], [[30, 31, 32], [40, 41, 42]]])
    k_cache = np.full((6, Hkv, d), 99.0, np.float32)
    v_cache = np.full((6, Hkv, d), 99.0, np.float32)
    tokens, n = oracle.commit_accepted(k_cand, v_cand, cand, [1, -1], [2, 0], [9, -1], W, D,
                                       k_cache, v_cache, [3, 0])
    # sequence 0: candidate 1 rows 0 and 1 are flat rows 3 and 4 of k_cand[0]
    assert k_cache[3, 0].tolist() == [6.0, 7.0] and k_cache[4, 0].tolist() == [8.0, 9.0]
    assert v_cache[3, 0].tolist() == [-6.0, -7.0] and v_cache[4, 0].tolist() == [-8.0, -9.0]
    untouched = [0, 1, 2, 5]
    assert np.all(k_cache[untouched] == 99.0) and np.all(v_cache[untouched] == 99.0)
    assert tokens.tolist() == [[20, 21, 9, -1], [-1, -1, -1, -1]]
    assert n.tolist() == [3, 0]


def test_nothing_accepted_commits_only_the_next_token():
    k_cand = np.ones((1, 4, 1, 2), np.float32)
    k_cache = np.zeros((4, 1, 2), np.float32)
    v_cache = np.zeros((4, 1, 2), np.float32)
    tokens, n = oracle.commit_accepted(k_cand, k_cand, np.zeros((1, 2, 2), int), [0], [0], [5],
                                       2, 2, k_cache, v_cache, [1])
    assert tokens.tolist() == [[5, -1, -1]] and n.tolist() == [1]
    assert np.all(k_cache == 0.0)


def test_commit_past_capacity_writes_nothing():
    k_cand = np.ones((1, 4, 1, 2), np.float32)
    k_cache = np.zeros((4, 1, 2), np.float32)
    v_cache = np.zeros((4, 1, 2), np.float32)
    tokens, n = oracle.commit_accepted(k_cand, k_cand, np.ones((1, 2, 2), int), [1], [2], [5],
                                       2, 2, k_cache, v_cache, [3])
    assert n.tolist() == [-1] and np.all(tokens == -1) and np.all(k_cache == 0.0)


def test_verify_accept_commit_equals_greedy_decoding():
    """One-layer synthetic target (token embeddings are q = k = v, logits = O . E^T):
    after verifying, accepting and committing, the context must be exactly what
    greedy decoding emits from the old context, and the cache must hold the keys
    of all context tokens but the new anchor."""
    rng = np.random.default_rng(21)
    n, W, D, d, V = 11, 3, 5, 8, 7
    E = rng.standard_normal((V, d)).astype(np.float32)

    def greedy_next(ctx):
        K = np.stack([E[t].astype(np.float64) for t in ctx])
        s = K @ E[ctx[-1]].astype(np.float64) / math.sqrt(d)
        p = np.exp(s - s.max())
        o = (p / p.sum()) @ K
        return int(np.argmax(E.astype(np.float64) @ o))

    for trial in range(6):
        x = [int(t) for t in rng.integers(0, V, n)]
        # candidates follow greedy decoding for a random stretch, then go astray
        cands = []
        for w in range(W):
            ctx, c = list(x), []
            stop = int(rng.integers(0, D + 1))
            for j in range(D):
                t = greedy_next(ctx) if j < stop else int(rng.integers(0, V))
                c.append(t)
                ctx.append(t)
            cands.append(c)
        Lw = [D] * W
        q = np.zeros((1, 1 + W * D, 1, d), np.float32)
        kc = np.zeros((1, W * D, 1, d), np.float32)
        q[0, 0, 0] = E[x[-1]]
        for w in range(W):
            for j in range(D):
                q[0, 1 + w * D + j, 0] = E[cands[w][j]]
                kc[0, w * D + j, 0] = E[cands[w][j]]
        kp = np.stack([E[t] for t in x])[:, None, :]
        out, _ = oracle.blocktri_attention(q, kp, kp, np.array([0, n]), kc, kc, np.array([Lw]),
                                           np.array([True]), 1, 1, d, W, D)
        am = oracle.lmhead_argmax(out[0], E)["pred"][None, :]
        acc = oracle.accept_longest(np.array([cands]), np.array([Lw]), np.array([True]), am, W, D)
        cap = n + D + 2
        k_cache = np.zeros((cap, 1, d), np.float32)
        v_cache = np.zeros((cap, 1, d), np.float32)
        k_cache[:n] = kp
        v_cache[:n] = kp
        tokens, nt = oracle.commit_accepted(kc, kc, np.array([cands]), acc["best_w"],
                                            acc["best_len"], acc["next_token"], W, D,
                                            k_cache, v_cache, [n])
        L = int(acc["best_len"][0])
        assert nt[0] == L + 1
        new_ctx = x + [int(t) for t in tokens[0, :L + 1]]
        ref = list(x)
        for _ in range(L + 1):
            ref.append(greedy_next(ref))
        assert new_ctx == ref, (trial, new_ctx[n:], ref[n:])
        # the cache holds the keys of every context token but the new anchor
        want = np.stack([E[t] for t in new_ctx[:-1]])
        assert np.array_equal(k_cache[:n + L, 0], want)
        assert np.all(k_cache[n + L:] == 0.0)
