"""Block-triangular verification attention (oracle; test infrastructure only).

SwitchSD paper §3.3 "Parallel Verification with Block-Triangular Attention"
(write-up §2.6): the W candidates are concatenated after the anchor position
and verified in one target forward pass; a token of candidate w may attend to
(i) the whole original prefix and (ii) the earlier tokens of candidate w, and to
nothing of any other candidate.  Paper §3.3 "Overall Framework": verification
is delegated to the target model and keeps its correctness guarantees, so each
candidate row must see exactly what plain causal decoding of that candidate
would see.

Readings where the pages leave a step open:
* Row layout per sequence: R = 1 + W*D query rows.  Row 0 is the anchor (the
  newest context token, whose K/V is the last prefix entry n-1); row
  1 + w*D + j is token j of candidate w.
* "Earlier tokens within candidate w" includes the token itself, as in any
  causal mask: row (w, j) sees candidate keys (w, 0..j).  The anchor row sees
  the prefix only.
* Standard multi-head conventions, not stated on the pages: scores are
  scale * q.k with scale = 1/sqrt(d) by default; query head h reads key/value
  head floor(h / g) with g = Hq / Hkv; the output row is the head-major
  concatenation (head h in columns h*d .. h*d+d-1).
* Rows that are not real (candidate w >= M, token j >= L_w, or a sequence whose
  gate is closed) are not verified; they are reported as zeros here.
"""
import numpy as np

from .bf16 import as_f64


def allowed_keys(n, W, D, r):
    """Boolean visibility of every key for query row r of one sequence.

    The key axis is [prefix 0..n-1, candidate 0 tokens 0..D-1, candidate 1 ...],
    length n + W*D.  Row 0 (anchor) sees the prefix; row 1 + w*D + j sees the
    prefix plus candidate keys (w, 0) .. (w, j).
    """
    vis = np.zeros(n + W * D, dtype=bool)
    vis[:n] = True
    if r > 0:
        w, j = divmod(r - 1, D)
        start = n + w * D
        vis[start:start + j + 1] = True
    return vis


def real_rows(cand_len_b, gate_b, W, D):
    """Rows of one sequence that carry a real query (see module readings)."""
    if not gate_b:
        return []
    rows = [0]
    for w in range(W):
        for j in range(int(cand_len_b[w])):
            rows.append(1 + w * D + j)
    return rows


def blocktri_attention(q, k_pre, v_pre, cu_len, k_cand, v_cand, cand_len, copy_gate,
                       Hq, Hkv, d, W, D, scale=None, rows=None):
    """Block-triangular attention output for real rows.

    q [B, R, Hq, d]; k_pre, v_pre [sum n, Hkv, d]; k_cand, v_cand [B, W*D, Hkv, d]
    (float32 or bfloat16 bits); cand_len [B, W]; copy_gate [B].
    rows: optional list of (b, r) to evaluate; default every real row.
    Returns (out [B, R, Hq*d] float64 with zeros on rows not evaluated,
             evaluated list of (b, r)).
    """
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    g = Hq // Hkv
    cu = np.asarray(cu_len)
    B = len(cu) - 1
    R = 1 + W * D
    out = np.zeros((B, R, Hq * d))
    todo = {}
    if rows is None:
        for b in range(B):
            rr = real_rows(cand_len[b], copy_gate[b], W, D)
            if rr:
                todo[b] = rr
    else:
        for b, r in rows:
            if r in real_rows(cand_len[b], copy_gate[b], W, D):
                todo.setdefault(b, []).append(r)
    evaluated = []
    for b, rr in todo.items():
        n = int(cu[b + 1] - cu[b])
        qb = as_f64(q[b])                                # [R, Hq, d]
        kp = as_f64(k_pre[cu[b]:cu[b + 1]])              # [n, Hkv, d]
        vp = as_f64(v_pre[cu[b]:cu[b + 1]])
        kc = as_f64(k_cand[b])                           # [W*D, Hkv, d]
        vc = as_f64(v_cand[b])
        vis = np.stack([allowed_keys(n, W, D, r) for r in rr])   # [rows, n + W*D]
        for h in range(Hq):
            kv = h // g
            K = np.concatenate([kp[:, kv, :], kc[:, kv, :]], axis=0)   # key axis of allowed_keys
            V = np.concatenate([vp[:, kv, :], vc[:, kv, :]], axis=0)
            S = (qb[rr, h, :] @ K.T) * scale                 # every score q.k, scaled
            S = np.where(vis, S, -np.inf)                    # keys a row may not see
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P = P / P.sum(axis=1, keepdims=True)
            out[b, rr, h * d:(h + 1) * d] = P @ V
        evaluated.extend((b, r) for r in rr)
    return out, evaluated
