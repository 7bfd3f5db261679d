"""LM-head projection and greedy argmax (oracle; test infrastructure only).

SwitchSD paper §3.3 "Parallel Verification": the single target forward pass
over anchor + candidates ends in the model's output distribution for every
query row; write-up §3.1: all reported runs decode at temperature T = 0.0, so
the target's choice at each row is the highest-scoring vocabulary entry.

Readings:
* logits[r][v] = sum_k O[r][k] * Wlm[k][v]; the weight is stored transposed,
  lm_head[v][k] (one contiguous row of `hid` weights per vocabulary entry).
* Equal maxima go to the lowest vocabulary index (the pages say nothing about
  ties; this makes the choice independent of evaluation order).
* The top-2 margin (best logit minus the best logit of any other index) says how
  far a row is from changing its choice.
"""
import numpy as np

from .bf16 import as_f64


def lm_logits(O, lm_head):
    """Full logits O . lm_head^T in float64.  O [rows, hid]; lm_head [V, hid]."""
    Of = as_f64(O)
    Wf = lm_head if (isinstance(lm_head, np.ndarray) and lm_head.dtype == np.float64) \
        else as_f64(lm_head)
    return Of @ Wf.T


def argmax_with_margin(logits):
    """Per row: (argmax with lowest index on ties, top-1 logit, top-2 margin)."""
    L = np.asarray(logits, dtype=np.float64)
    if L.ndim == 1:
        L = L[None, :]
    pred = np.argmax(L, axis=1)            # first occurrence of the maximum = lowest index
    top1 = L[np.arange(L.shape[0]), pred]
    rest = L.copy()
    rest[np.arange(L.shape[0]), pred] = -np.inf
    top2 = rest.max(axis=1) if L.shape[1] > 1 else np.full(L.shape[0], -np.inf)
    return pred.astype(np.int64), top1, top1 - top2


def lmhead_argmax(O, lm_head):
    """pred, margin and logits for rows of O (see lm_logits / argmax_with_margin)."""
    logits = lm_logits(O, lm_head)
    pred, top1, margin = argmax_with_margin(logits)
    return {"pred": pred, "top1": top1, "margin": margin, "logits": logits}
