"""kappa-gram evidence and candidate retrieval (oracle; test infrastructure only).

SwitchSD write-up §2.5 (the dual-gate "formula 4"): copy speculation is enabled
only if the probe fires AND the kappa-gram (kappa = 5) that ends at the current
token has appeared at least once earlier in the context; a probe hit without such
a match falls back to neural drafting.
Paper §3.3 "Copy-Based Speculative Generation" and write-up §2.6: when copying
is triggered, up to W candidate continuations are taken from the context, each
of (at most) D tokens, ranked by recency (W = 10, D = 20 in the write-up).

Readings where the pages leave a step open:
* The suffix is s = x[n-kappa .. n-1], the newest kappa ids; x[n-1] is the
  current (anchor) token.  An earlier occurrence is an end position p with
  kappa-1 <= p <= n-2 and x[p-kappa+1 .. p] == s.  The suffix itself (p = n-1)
  is not an earlier occurrence; occurrences may overlap the suffix.
* Recency = larger end position first.  Positions are distinct, so the order is
  total; identical continuations are not merged (the pages mention no merging).
* Candidate w continues its occurrence: cand[w][j] = x[p_w + 1 + j] for
  j < L_w = min(D, n - 1 - p_w).  The paper gives every candidate length D,
  the write-up caps it at D; a recent occurrence too close to the end to supply
  D tokens is kept with the tokens it has.
* When the probe does not fire, nothing is retrieved (the paper retrieves only
  once the copy regime is triggered), and the gate is closed.
"""
import numpy as np


def kgram_matches(x, kappa, limit=None):
    """End positions of earlier occurrences of the newest kappa-gram of x, newest first.

    Walks p from n-2 down to kappa-1 and compares all kappa ids; stops after
    `limit` hits when a limit is given.
    """
    x = [int(t) for t in x]
    n = len(x)
    if n < kappa + 1:
        return []
    suffix = x[n - kappa:]
    hits = []
    for p in range(n - 2, kappa - 2, -1):
        if x[p - kappa + 1:p + 1] == suffix:
            hits.append(p)
            if limit is not None and len(hits) == limit:
                break
    return hits


def kgram_retrieve(ids, cu_len, kappa, W, D, fire=None):
    """Gate evidence + recency-ordered candidates for each sequence of a batch.

    ids: concatenated int32 context ids; cu_len: [B+1] offsets; fire: [B] probe
    decisions or None (= every probe fired).
    Returns dict of
      match_end [B, W] int32 (end positions p_w, -1 padded),
      n_match   [B]    int32 (M = min(W, number of earlier occurrences)),
      cand      [B, W, D] int32 (continuation ids, -1 padded),
      cand_len  [B, W] int32 (L_w, 0 for w >= M),
      copy_gate [B]    bool  (fire and M > 0).
    """
    ids = np.asarray(ids)
    cu = np.asarray(cu_len)
    B = len(cu) - 1
    match_end = np.full((B, W), -1, dtype=np.int32)
    n_match = np.zeros(B, dtype=np.int32)
    cand = np.full((B, W, D), -1, dtype=np.int32)
    cand_len = np.zeros((B, W), dtype=np.int32)
    copy_gate = np.zeros(B, dtype=bool)
    for b in range(B):
        if fire is not None and not bool(fire[b]):
            continue
        x = ids[cu[b]:cu[b + 1]]
        n = len(x)
        hits = kgram_matches(x, kappa, limit=W)
        n_match[b] = len(hits)
        copy_gate[b] = len(hits) > 0
        for w, p in enumerate(hits):
            L = min(D, n - 1 - p)
            match_end[b, w] = p
            cand_len[b, w] = L
            for j in range(L):
                cand[b, w, j] = x[p + 1 + j]
    return {"match_end": match_end, "n_match": n_match, "cand": cand,
            "cand_len": cand_len, "copy_gate": copy_gate}
