"""Verification of copy candidates at temperature T > 0 (oracle; test infrastructure only).

The pages give no acceptance rule for copy candidates at T > 0 (the SwitchSD paper
reports temperature sweeps in its App. A / the write-up's Table 4 without one).
They do fix the requirement: verification is delegated to the target model and
keeps speculative decoding's correctness guarantee (SwitchSD paper §3.3 "Overall
Framework", §2 "Speculative Decoding"); in the lossless setting each drafted token
is accepted by its relative likelihood and a rejected token is replaced by a
sample from the residual distribution (VIA-SD page, "Draft-Verify and Lossy
Acceptance" with alpha = 0).

Reading.  A copy candidate is a draft whose proposal q is a point mass on its
token c, so speculative sampling accepts c with probability min(1, p(c)/q(c)) =
p(c), and on rejection samples from the residual, p with c removed and
renormalised.  The W candidates form a trie (candidates with equal prefixes share
a node).  At a node with distribution p and distinct child tokens x_1, x_2, ...
(in order of their first candidate, i.e. recency), x_k is tried with probability
p(x_k) / (1 - p(x_1) - ... - p(x_{k-1})), the residual left after the tokens
already rejected at this node; an accepted child moves the walk to its node.
When every child is rejected, or the node has no child, the next token is drawn
from p with the tried children removed.  Every emitted token is then distributed
exactly as the target's conditional (recursive rejection sampling), which the
pins check by Monte Carlo.

* p at a node = softmax(logits / T) of the node's row: the anchor row for the
  root, else row (r, j - 1) where r is the lowest-index candidate of the node's
  group (candidates whose first j tokens equal the node's prefix).
* Ties: children are ordered by their lowest candidate index; the returned
  best_w is the lowest candidate of the final group (0 when nothing is accepted,
  as at T = 0); the residual draw takes the lowest token index among equal scores.
* Random numbers come from Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011) keyed by the 64-bit
  seed (key = (low word, high word)); a 32-bit output word w becomes
  u = (floor(w / 512) + 1/2) / 2^23 = (2 floor(w / 512) + 1) / 2^24, a float in
  (0, 1) with 24 significant bits, exact in binary32.
  - residual draw at global row g (= b * R + row), token x: counter
    (floor(x / 4), g, 0, 0), word x mod 4; Gumbel noise G = -ln(-ln u); the draw
    is argmax over allowed x of logits[x] / T + G_x (Gumbel-max).
  - acceptance test of child k at global row g: counter (k, g, 1, 0), word 0.
* The acceptance ratio is r = p(x) / max(1 - tried, p(x)) (0 when p(x) = 0), which
  equals the residual probability and stays in [0, 1] under rounding.
* A closed gate verifies nothing: best_w = -1, best_len = 0, next_token = -1.
"""
import numpy as np

_PHILOX = {
    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85),
    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),
}


def philox(ctr, key, bits=32, rounds=10):
    """Philox4xW-R block function on Python integers: 4 counter words, 2 key words
    -> 4 output words of `bits` bits."""
    m0, m1, w0, w1 = _PHILOX[bits]
    mask = (1 << bits) - 1
    c0, c1, c2, c3 = (int(v) & mask for v in ctr)
    k0, k1 = (int(v) & mask for v in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0, p1 = m0 * c0, m1 * c2
        c0, c1, c2, c3 = ((p1 >> bits) ^ c1 ^ k0, p1 & mask, (p0 >> bits) ^ c3 ^ k1, p0 & mask)
    return [c0, c1, c2, c3]


def philox4x32_np(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x32-R over numpy arrays of counters (uint64 arithmetic on 32-bit words)."""
    m0, m1, w0, w1 = _PHILOX[32]
    M = np.uint64(0xFFFFFFFF)
    c = [np.asarray(v, dtype=np.uint64) & M for v in (c0, c1, c2, c3)]
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    c0, c1, c2, c3 = (x.copy() for x in (c0, c1, c2, c3))
    k0, k1 = np.uint64(k0 & 0xFFFFFFFF), np.uint64(k1 & 0xFFFFFFFF)
    for r in range(rounds):
        if r:
            k0 = (k0 + np.uint64(w0)) & M
            k1 = (k1 + np.uint64(w1)) & M
        p0 = np.uint64(m0) * c0
        p1 = np.uint64(m1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & M, (p0 >> np.uint64(32)) ^ c3 ^ k1,
                          p0 & M)
    return c0, c1, c2, c3


def _key(seed):
    seed = int(seed) & ((1 << 64) - 1)
    return seed & 0xFFFFFFFF, seed >> 32


def word_to_uniform(w):
    """32-bit word -> (floor(w / 512) + 1/2) / 2^23 in (0, 1)."""
    return ((np.asarray(w, dtype=np.uint64) >> np.uint64(9)).astype(np.float64) + 0.5) / 2.0 ** 23


def gumbel_row(seed, g, V):
    """Gumbel noise of every token x < V at global row g: -ln(-ln u)."""
    k0, k1 = _key(seed)
    x = np.arange(V, dtype=np.uint64)
    words = philox4x32_np(x >> np.uint64(2), np.uint64(g), 0, 0, k0, k1)
    w = np.choose((x & np.uint64(3)).astype(np.int64), words)
    return -np.log(-np.log(word_to_uniform(w)))


def accept_uniform(seed, g, k):
    """Uniform of the acceptance test of child k at global row g."""
    return float(word_to_uniform(philox([k, g, 1, 0], _key(seed))[0]))


def candidate_trie(cand, cand_len, gate, W, D):
    """Trie of one sequence's candidates, keyed by verification row.

    Returns dict row -> list of (token, w) children of the node whose distribution
    is that row (row 0 = anchor = root; row 1 + r*D + j-1 for the node of the
    group with lowest candidate r and prefix length j).  Every real row appears
    (nodes without children and rows that are not nodes map to []) and only
    nodes have children."""
    R = 1 + W * D
    kids = {r: [] for r in range(R)}
    if not gate:
        return kids
    L = [int(min(max(int(cand_len[w]), 0), D)) for w in range(W)]
    toks = [[int(cand[w][j]) for j in range(L[w])] for w in range(W)]
    # group representative after j tokens: lowest w with the same first j tokens
    for j in range(D):
        for w in range(W):
            if L[w] <= j:
                continue
            prefix = toks[w][:j]
            rep_parent = min(v for v in range(W) if L[v] >= j and toks[v][:j] == prefix)
            first = min(v for v in range(W) if L[v] > j and toks[v][:j + 1] == toks[w][:j + 1])
            if first != w:
                continue
            parent_row = 0 if j == 0 else 1 + rep_parent * D + (j - 1)
            kids[parent_row].append((toks[w][j], w))
    return kids


def softmax_T(logits, T):
    z = np.asarray(logits, dtype=np.float64) / T
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def accept_ratio(p, tried):
    return 0.0 if p == 0.0 else p / max(1.0 - tried, p)


def residual_draw(logits_row, T, seed, g, excluded):
    """Gumbel-max draw from softmax(logits / T) without the excluded tokens.
    Returns (token, margin): margin is the gap between the two best scores."""
    y = np.asarray(logits_row, dtype=np.float64) / T + gumbel_row(seed, g, len(logits_row))
    for x in excluded:
        if 0 <= x < len(y):
            y[x] = -np.inf
    order = np.argsort(-y, kind="stable")
    tok = int(order[0])
    margin = float(y[order[0]] - y[order[1]]) if len(y) > 1 else np.inf
    return tok, margin


def sample_step(row_logits, cand, cand_len, gate, W, D, T, seed, b, uniform=None, draw=None):
    """The T > 0 verification walk of sequence b.

    row_logits(row) -> logits [V] (float64) of verification row `row` of b.
    uniform(g, k) and draw(row, g, excluded) may replace the Philox streams (tests).
    Returns dict best_w, best_len, next_token, tokens (accepted path) and
    decisions: list of (row, k, u, ratio)."""
    R = 1 + W * D
    if not gate:
        return {"best_w": -1, "best_len": 0, "next_token": -1, "tokens": [], "decisions": []}
    kids = candidate_trie(cand, cand_len, gate, W, D)
    uniform = uniform or (lambda g, k: accept_uniform(seed, g, k))
    if draw is None:
        def draw(row, g, excluded):
            return residual_draw(row_logits(row), T, seed, g, excluded)[0]
    row, j, best_w, path, decisions = 0, 0, 0, [], []
    while True:
        ch = kids[row]
        g = b * R + row
        p = softmax_T(row_logits(row), T) if ch else None
        tried, moved = 0.0, False
        for k, (x, w) in enumerate(ch):
            px = float(p[x]) if 0 <= x < len(p) else 0.0
            u, r = uniform(g, k), accept_ratio(px, tried)
            decisions.append((row, k, u, r))
            if u < r:
                path.append(x)
                best_w, row, j, moved = w, 1 + w * D + j, j + 1, True
                break
            tried += px
        if not moved:
            nxt = draw(row, g, [x for x, _ in ch])
            return {"best_w": best_w, "best_len": j, "next_token": int(nxt), "tokens": path,
                    "decisions": decisions}


def sample_verify(logits, cand, cand_len, copy_gate, W, D, T, seed):
    """Batch form: logits [B, R, V] (float64).  Returns best_w, best_len, next_token
    [B] int32 and the per-sequence decision lists."""
    B = len(copy_gate)
    out = {"best_w": np.full(B, -1, np.int32), "best_len": np.zeros(B, np.int32),
           "next_token": np.full(B, -1, np.int32), "decisions": []}
    for b in range(B):
        r = sample_step(lambda row: logits[b][row], cand[b], cand_len[b], bool(copy_gate[b]), W, D,
                        T, seed, b)
        out["best_w"][b], out["best_len"][b], out["next_token"][b] = r["best_w"], r["best_len"], r["next_token"]
        out["decisions"].append(r["decisions"])
    return out
