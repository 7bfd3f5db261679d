"""Copy-intent probe (oracle; test infrastructure only).

SwitchSD pages: paper §3.2 "Layer and Threshold Selection" and §3.3 opening
paragraph — at every decoding step the hidden state H_i^(l) of the selected
layer is read and copy drafting is allowed only when the probe score
PR(H_i^(l)) >= tau; write-up §2.3 "Probe 架构" — the probe is a strictly linear
projection without bias, one per layer, trained with binary cross-entropy;
write-up §2.4 — tau ~ 0.4 for Llama-3.1-8B, picked by F1 on a validation split.

Reading (the probe formula itself is missing from both pages): a bias-free
linear map trained with binary cross-entropy outputs a logit, so the score is
the probability PR(h) = sigmoid(w . h), and tau in (0, 1) is a probability
threshold.  The decision is therefore PR(h) >= tau, which is the same test as
w . h >= ln(tau / (1 - tau)).
"""
import math

import numpy as np

from .bf16 import as_f64


def logit(tau):
    """ln(tau / (1 - tau)) in float64: the score threshold on the linear output."""
    return math.log(tau / (1.0 - tau))


def probe_score(h, w, tau):
    """Probe decision for each row of h.

    h: [B, hid] float32, float64 or bfloat16 bits (uint16); w: [hid] float32.
    Returns dict with
      z      [B] float64  linear output w . h (sum over k ascending),
      score  [B] float64  PR(h) = 1 / (1 + exp(-z)),
      fire   [B] bool     score >= tau,
      margin [B] float64  z - ln(tau/(1-tau)) (distance from the decision point),
      S      [B] float64  sum_k |w_k h_k| (scale of the rounding error of z).
    """
    if not (0.0 < tau < 1.0):
        raise ValueError("tau must lie in (0, 1)")
    H = as_f64(h)
    if H.ndim == 1:
        H = H[None, :]
    wv = as_f64(w)
    B, hid = H.shape
    z = np.zeros(B)
    S = np.zeros(B)
    for b in range(B):
        acc = 0.0
        s_abs = 0.0
        for k in range(hid):
            t = wv[k] * H[b, k]
            acc += t
            s_abs += abs(t)
        z[b] = acc
        S[b] = s_abs
    score = 1.0 / (1.0 + np.exp(-z))
    fire = score >= tau
    return {"z": z, "score": score, "fire": fire, "margin": z - logit(tau), "S": S}
