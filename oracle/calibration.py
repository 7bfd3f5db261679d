"""Offline calibration of the copy-intent probe (oracle; test infrastructure only).

SwitchSD paper §3.2 "Problem Formulation": a token position is a copy-mode
instance (Y = 1) when it belongs to a verbatim run of at least n_train = 5 tokens
that appears earlier in the context; every other position is Y = 0.  §3.2 "Layer
and Threshold Selection": after probes are trained on every layer, the layer is
chosen by greedy F1 maximisation on a validation split, and the decision
threshold tau by maximising F1 on the same split.  §4.3.3 reports the F1-optimal
threshold (near 0.4) and the ROC AUC (> 0.99); the write-up's §2.4 restates both.

Readings:
* "Appears earlier": the run x[a..e] (e - a + 1 >= n_train) occurs starting at
  some s < a; the earlier occurrence may overlap the run (periodic text).  Every
  n_train-window inside such a run then also occurs at an earlier start, and a
  single window is itself such a run, so position i is labelled exactly when some
  n_train-window containing i occurs at an earlier start.
* Scores are the probe logits z = w . h; thresholds are taken on z (sigma is
  monotone, so F1 and AUC are the same as on PR = sigma(z)); tau = sigma(z*).
* F1 = 2 TP / (2 TP + FP + FN) with "copy" predicted when z >= t, and 0 when
  TP = 0.  Candidate thresholds are the distinct scores; an F1 tie goes to the
  highest threshold (the most conservative gate).  A layer tie goes to the lowest
  layer.
* ROC AUC is the Mann-Whitney statistic: the probability that a copy position
  scores above a non-copy one, equal scores counting one half.  It is returned as
  the integer 2U with the class counts (AUC = 2U / (2 P N)); undefined (NaN) when
  a class is empty.
"""
import math

import numpy as np

from .bf16 import bf16_bits_to_f64


def copy_labels(ids, cu_len, n_train=5):
    """Per-position copy-mode labels (uint8) of the concatenated contexts."""
    ids = np.asarray(ids)
    lab = np.zeros(len(ids), dtype=np.uint8)
    for b in range(len(cu_len) - 1):
        lo, hi = int(cu_len[b]), int(cu_len[b + 1])
        x = [int(t) for t in ids[lo:hi]]
        n = len(x)
        first = {}
        for a in range(n - n_train + 1):
            key = tuple(x[a:a + n_train])
            if key in first:                 # occurs at an earlier start
                lab[lo + a:lo + a + n_train] = 1
            else:
                first[key] = a
    return lab


def probe_logits(H, w, dtype="f32"):
    """z[l][i] = w[l] . H[l][i] in float64.  H [L, N, hid] (float32 or bf16 bits), w [L, hid]."""
    Hd = bf16_bits_to_f64(H) if dtype == "bf16" else np.asarray(H, dtype=np.float64)
    wd = np.asarray(w, dtype=np.float64)
    return np.einsum("lnk,lk->ln", Hd, wd)


def threshold_sweep(z, y):
    """F1-optimal threshold and ROC AUC of one layer's scores z [N] against labels y [N].

    Returns dict: t (best logit threshold; +inf when no threshold gives TP > 0),
    f1, tp, fp, fn at t, u2 (= 2U), pos, neg, auc."""
    z = np.asarray(z, dtype=np.float64)
    y = np.asarray(y).astype(bool)
    pos, neg = int(y.sum()), int((~y).sum())
    best = {"t": math.inf, "f1": 0.0, "tp": 0, "fp": 0, "fn": pos}
    for t in sorted(set(z.tolist()), reverse=True):       # highest threshold first
        pred = z >= t
        tp = int((pred & y).sum())
        fp = int((pred & ~y).sum())
        fn = pos - tp
        f1 = 2 * tp / (2 * tp + fp + fn) if tp > 0 else 0.0
        if f1 > best["f1"]:                                  # strict: ties keep the higher t
            best = {"t": t, "f1": f1, "tp": tp, "fp": fp, "fn": fn}
    zp, zn = z[y], z[~y]
    u2 = 0
    for v in zp:
        u2 += 2 * int((zn < v).sum()) + int((zn == v).sum())
    auc = u2 / (2 * pos * neg) if pos and neg else float("nan")
    best.update(u2=u2, pos=pos, neg=neg, auc=auc)
    return best


def calibrate(z_layers, y):
    """Per-layer sweep, then the layer with the highest F1 (lowest layer on ties) and
    tau = sigma(t) of that layer."""
    per = [threshold_sweep(z, y) for z in z_layers]
    layer = 0
    for l in range(1, len(per)):
        if per[l]["f1"] > per[layer]["f1"]:
            layer = l
    t = per[layer]["t"]
    if math.isinf(t):
        tau = 1.0 if t > 0 else 0.0        # the limits of sigma
    else:
        tau = 1.0 / (1.0 + math.exp(-t)) if t > -700 else 0.0
    return {"per_layer": per, "layer": layer, "t": t, "tau": tau}
