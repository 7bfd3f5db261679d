"""Committing the accepted draft (oracle; test infrastructure only).

SwitchSD paper §3.3 "Parallel Verification" keeps the longest validated
continuation, and the same section (with the write-up's §2.6) says the accepted
tokens then extend the context for the next step.  Greedy decoding also emits
the target's own token after the accepted ones (the prefix-acceptance rule of
the VIA-SD page, "Draft–Verify and Lossy Acceptance"), which becomes the next
anchor.  The verification pass already computed the keys and values of the
accepted candidate tokens; committing them means copying those rows into the
target's KV cache.  The caller computes the new anchor's K/V in its next pass.

Readings:
* The rows committed for sequence b are the candidate rows (best_w, 0..best_len-1)
  of the verify-pass K/V, in that order, at cache rows off_b .. off_b + best_len - 1.
* The tokens that extend the context are cand[best_w][0..best_len-1] followed by
  next_token (best_len + 1 tokens).
* A sequence whose gate was closed (best_w < 0) commits nothing: 0 tokens.
* A commit that would write past the cache capacity writes nothing for that
  sequence and reports -1 tokens.
"""
import numpy as np


def commit_accepted(k_cand, v_cand, cand, best_w, best_len, next_token, W, D,
                    k_cache, v_cache, cache_off):
    """k_cand, v_cand [B, W*D, Hkv, d]; cand [B, W, D]; best_w/best_len/next_token [B];
    k_cache, v_cache [rows, Hkv, d] (updated in place); cache_off [B] first cache
    row to write.  Returns (tokens [B, D+1] int32 padded with -1, n_tokens [B] int32)."""
    B = len(best_w)
    rows = k_cache.shape[0]
    tokens = np.full((B, D + 1), -1, dtype=np.int32)
    n_tokens = np.zeros(B, dtype=np.int32)
    for b in range(B):
        w = int(best_w[b])
        if w < 0:
            continue
        L = int(best_len[b])
        off = int(cache_off[b])
        if off < 0 or off + L > rows:
            n_tokens[b] = -1
            continue
        for j in range(L):
            k_cache[off + j] = k_cand[b, w * D + j]
            v_cache[off + j] = v_cand[b, w * D + j]
            tokens[b, j] = int(cand[b][w][j])
        tokens[b, L] = int(next_token[b])
        n_tokens[b] = L + 1
    return tokens, n_tokens
