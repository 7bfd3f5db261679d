"""The verification pass as a full target forward: embedding, decoder layers, final
norm, LM head (oracle; test infrastructure only).

SwitchSD paper §3.3 "Parallel Verification with Block-Triangular Attention":
the anchor and the W candidates are verified in one forward pass of the target,
candidate tokens seeing the prefix and their own earlier tokens.  The pages
name the targets (Llama-3.1-8B, Qwen3-8B, Llama-3.3-70B; paper §4.1) but not
their layer; the decoder layer here is the Llama-family layer those models
share, with synthetic weights.

Readings:
* Layer (pre-norm): h = RMSNorm(x) * g_attn; q, k, v = projections of h; RoPE on
  q and k; attention (block-triangular, GQA, scale 1/sqrt(d)); x += Wo attn;
  h = RMSNorm(x) * g_mlp; x += W_down (silu(W_gate h) * (W_up h)).  After the
  layers, h = RMSNorm(x) * g_final feeds the LM head.  RMSNorm(x) =
  x / sqrt(mean(x^2) + eps).  Weights are [out][in].
* Positions: prefix entry p has position p (the caches hold keys after RoPE),
  the anchor row n - 1, candidate token j of any candidate n + j.
* RoPE rotates adjacent pairs (2i, 2i + 1) of each head by pos * base^(-2i/d)
  (base 500000, the Llama-3 value; no long-context rescaling).  Which pairs a
  model rotates is a fixed permutation of the head dimensions, absorbed by the
  synthetic weights.
* The anchor's own key and value are prefix entry n - 1 (the caller's cache), so
  the anchor row contributes only its query; candidate rows contribute their
  keys and values to the candidate blocks.
* Storage, the rule of a bf16 Llama layer: every tensor that one operation hands
  to the next as an operand of a bf16 matrix product or of attention is held in
  bf16.  Those are the RMSNorm outputs that feed the q/k/v and the gate/up
  projections, q and k after RoPE and v (so the KV cache holds bf16 keys and
  values), the attention output that feeds W_o, the SwiGLU activation
  silu(gate) * up that feeds W_down, and the final RMSNorm output that feeds the
  LM head.  Each is computed wide, held as the float32 an accumulator would
  hold, and rounded to bf16, to nearest even.  The
  residual stream x, into which W_o and W_down add their outputs, stays wide, and
  so do the logits.  storage_bf16=False keeps every tensor wide.
"""
import numpy as np

from .attention import blocktri_attention
from .bf16 import bf16_bits_to_f64
from .lmhead import lmhead_argmax


def round_bf16(x):
    """float64 -> nearest-even bfloat16 value (as float64)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return bf16_bits_to_f64(u.astype(np.uint16))


def rmsnorm(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def rope(x, pos, base):
    """x [..., d] (one head) rotated by position pos: pair (2i, 2i+1) by pos * base^(-2i/d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    out = np.empty_like(x)
    for i in range(d // 2):
        a = pos * base ** (-2.0 * i / d)
        c, s = np.cos(a), np.sin(a)
        x0, x1 = x[..., 2 * i], x[..., 2 * i + 1]
        out[..., 2 * i] = x0 * c - x1 * s
        out[..., 2 * i + 1] = x0 * s + x1 * c
    return out


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def row_tokens(ids, cu_len, cand, W, D):
    """Token of every verification row: the anchor (last context token) at row 0,
    candidate token j of w at row 1 + w*D + j (-1 beyond the candidate)."""
    B = len(cu_len) - 1
    tok = np.full((B, 1 + W * D), -1, dtype=np.int64)
    for b in range(B):
        tok[b, 0] = ids[cu_len[b + 1] - 1]
        tok[b, 1:] = np.asarray(cand[b]).reshape(-1)
    return tok


def row_positions(cu_len, W, D):
    B = len(cu_len) - 1
    pos = np.zeros((B, 1 + W * D), dtype=np.int64)
    for b in range(B):
        n = int(cu_len[b + 1] - cu_len[b])
        pos[b, 0] = n - 1
        for w in range(W):
            for j in range(D):
                pos[b, 1 + w * D + j] = n + j
    return pos


def _keep(x):
    return np.asarray(x, dtype=np.float64)


def decoder_layer(x, layer, cu_len, cand_len, gate, pos, Hq, Hkv, d, W, D, base, eps, rows=None,
                  storage_bf16=True):
    """One layer on the residual stream x [B, R, hid] (float64).  layer: dict of
    float64 arrays attn_norm, wq, wk, wv, wo, mlp_norm, w_gate, w_up, w_down and
    the prefix caches k_cache, v_cache [sum n, Hkv, d].  Returns the new x.
    storage_bf16=False skips the bf16 rounding of the stored activations."""
    round_bf16_ = round_bf16 if storage_bf16 else _keep
    B, R, hid = x.shape
    h = round_bf16_(rmsnorm(x, layer["attn_norm"], eps))
    q = (h @ layer["wq"].T).reshape(B, R, Hq, d)
    k = (h @ layer["wk"].T).reshape(B, R, Hkv, d)
    v = (h @ layer["wv"].T).reshape(B, R, Hkv, d)
    for b in range(B):
        for r in range(R):
            for hh in range(Hq):
                q[b, r, hh] = rope(q[b, r, hh], pos[b, r], base)
            for hh in range(Hkv):
                k[b, r, hh] = rope(k[b, r, hh], pos[b, r], base)
    q, k, v = round_bf16_(q), round_bf16_(k), round_bf16_(v)
    k_c, v_c = k[:, 1:], v[:, 1:]             # candidate rows' keys and values
    att, _ = blocktri_attention(q, layer["k_cache"], layer["v_cache"], cu_len, k_c, v_c, cand_len,
                                gate, Hq, Hkv, d, W, D, 1.0 / np.sqrt(d), rows=rows)
    att = round_bf16_(att)
    x = x + att @ layer["wo"].T
    h = round_bf16_(rmsnorm(x, layer["mlp_norm"], eps))
    a = round_bf16_(silu(h @ layer["w_gate"].T) * (h @ layer["w_up"].T))
    return x + a @ layer["w_down"].T


def verify_forward(ids, cu_len, cand, cand_len, gate, embed, layers, final_norm, lm_head, Hq, Hkv,
                   d, W, D, base=500000.0, eps=1e-5, rows=None, storage_bf16=True):
    """Embedding, the decoder layers, final norm and the LM head with argmax.

    Returns dict x (final residual [B, R, hid]), h (normalised bf16 rows) and
    argmax / margin / logits of the rows listed (every row when rows is None)."""
    tok = row_tokens(ids, cu_len, cand, W, D)
    pos = row_positions(cu_len, W, D)
    E = np.asarray(embed, dtype=np.float64)
    x = E[np.clip(tok, 0, len(E) - 1)] * (tok >= 0)[..., None]
    for layer in layers:
        x = decoder_layer(x, layer, cu_len, cand_len, gate, pos, Hq, Hkv, d, W, D, base, eps, rows,
                          storage_bf16)
    h = rmsnorm(x, final_norm, eps)
    h = round_bf16(h) if storage_bf16 else h
    B, R, _ = x.shape
    sel = [(b, r) for b in range(B) for r in range(R)] if rows is None else list(rows)
    res = lmhead_argmax(h[[b for b, _ in sel], [r for _, r in sel]], lm_head)
    return {"x": x, "h": h, "rows": sel, **res}
