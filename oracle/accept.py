"""Longest accepted continuation at T = 0 (oracle; test infrastructure only).

SwitchSD paper §3.3 "Parallel Verification": after the single verification pass
the framework keeps the candidate whose verified continuation is longest; the
write-up's §2.6 states the same rule.  Greedy verification checks a drafted token
against the target's own choice after the tokens before it and stops at the
first disagreement, the prefix-acceptance rule of the draft-verify paradigm as
the VIA-SD page states it ("Draft–Verify and Lossy Acceptance": decoding halts
at the first rejected token; "VIA-SD Inference" step 4: the accepted prefix is
the longest one).

Readings:
* pred(w, -1) is the anchor row's choice (row 0); pred(w, j) is the choice at
  row 1 + w*D + j.  Candidate token (w, j) is accepted when every token before
  it is accepted and cand[w][j] == pred(w, j-1); a_w counts accepted tokens.
* Ties between candidates go to the lowest w, the most recent one (candidates
  are ranked by recency, paper §3.3 "Copy-Based Speculative Generation").
* next_token is the target's choice right after the accepted tokens,
  pred(best_w, best_len - 1), or the anchor row's choice when nothing is
  accepted: greedy decoding emits it whatever happens to the draft.
* A sequence whose gate is closed was not verified: best_w = -1,
  best_len = 0, next_token = -1, every a_w = 0 (the caller drafts neurally).
"""
import numpy as np


def accept_longest(cand, cand_len, copy_gate, argmax, W, D):
    """cand [B, W, D]; cand_len [B, W]; copy_gate [B]; argmax [B, 1 + W*D].

    Returns dict of accept_len [B, W], best_w [B], best_len [B], next_token [B]
    (all int32).
    """
    B = len(copy_gate)
    accept_len = np.zeros((B, W), dtype=np.int32)
    best_w = np.full(B, -1, dtype=np.int32)
    best_len = np.zeros(B, dtype=np.int32)
    next_token = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        if not bool(copy_gate[b]):
            continue

        def pred(w, j):
            return int(argmax[b][0]) if j < 0 else int(argmax[b][1 + w * D + j])

        for w in range(W):
            a = 0
            while a < int(cand_len[b][w]) and int(cand[b][w][a]) == pred(w, a - 1):
                a += 1
            accept_len[b, w] = a
        bw = 0
        for w in range(1, W):
            if accept_len[b, w] > accept_len[b, bw]:
                bw = w
        best_w[b] = bw
        best_len[b] = accept_len[b, bw]
        next_token[b] = pred(bw, int(best_len[b]) - 1)
    return {"accept_len": accept_len, "best_w": best_w, "best_len": best_len,
            "next_token": next_token}
