"""Pins for the oracle's offline probe calibration.

SwitchSD paper §3.2 "Problem Formulation" (copy-mode labels: a position inside a
verbatim run of >= n_train = 5 tokens that appears earlier) and "Layer and
Threshold Selection" (greedy F1 maximisation over layers and thresholds); §4.3.3
(F1-optimal threshold, ROC AUC).

References: hand-built contexts, a brute force over every span and every earlier
start (it does not use the window equivalence the oracle relies on),
scikit-learn's ROC AUC and F1, closed forms for separable, reversed and constant
scores, and Python-loop dot products.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from sklearn.metrics import f1_score, precision_recall_curve, roc_auc_score

import oracle


def _lab(x, n_train=5):
    return oracle.copy_labels(np.array(x), np.array([0, len(x)]), n_train).tolist()


def test_hand_built_labels():
    assert _lab([1, 2, 3, 4, 5, 9, 1, 2, 3, 4, 5]) == [0] * 6 + [1] * 5
    assert _lab([1, 2, 3, 4, 9, 1, 2, 3, 4, 8]) == [0] * 10           # a 4-token repeat only
    assert _lab([7] * 8) == [0] + [1] * 7                             # overlapping earlier run
    assert _lab([1, 2, 3] * 4) == [0] * 3 + [1] * 9                   # period 3
    assert _lab([1, 2, 3, 4]) == [0] * 4                              # shorter than n_train
    # a repeat longer than n_train labels the whole repeated run
    assert _lab([5, 6, 7, 8, 9, 10, 11, 0, 5, 6, 7, 8, 9, 10, 11]) == [0] * 8 + [1] * 7


def test_labels_do_not_cross_sequences():
    ids = np.array([1, 2, 3, 4, 5, 1, 2, 3, 4, 5, 6])
    lab = oracle.copy_labels(ids, np.array([0, 5, 11]))
    assert lab.tolist() == [0] * 5 + [0] * 6


def _brute(x, n_train):
    n = len(x)
    lab = [0] * n
    for a in range(n):
        for e in range(a + n_train - 1, n):
            L = e - a + 1
            if any(x[s:s + L] == x[a:e + 1] for s in range(a)):
                for i in range(a, e + 1):
                    lab[i] = 1
    return lab


@settings(max_examples=200, deadline=None)
@given(st.integers(2, 3), st.integers(2, 6), st.lists(st.integers(0, 2), min_size=0, max_size=40))
def test_labels_match_brute_force_over_all_spans(vocab, n_train, xs):
    x = [v % vocab for v in xs]
    assert _lab(x, n_train) == _brute(x, n_train)


def test_probe_logits_loop_and_bf16():
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(8)
    H = rng.standard_normal((3, 5, 7)).astype(np.float32)
    w = rng.standard_normal((3, 7)).astype(np.float32)
    z = oracle.probe_logits(H, w)
    for l in range(3):
        for i in range(5):
            want = math.fsum(float(H[l, i, k]) * float(w[l, k]) for k in range(7))
            assert z[l, i] == pytest.approx(want, abs=1e-12)
    Hb = f32_to_bf16_bits(np.array([[[1.0, -2.0, 0.5]]], np.float32))
    assert oracle.probe_logits(Hb, np.array([[1.0, 1.0, 4.0]]), "bf16")[0, 0] == 1.0


def test_sweep_closed_forms():
    y = np.array([1, 1, 0, 0, 0])
    r = oracle.threshold_sweep(np.array([3.0, 2.0, 1.0, 0.0, -1.0]), y)       # separable
    assert r["auc"] == 1.0 and r["f1"] == 1.0 and r["t"] == 2.0 and (r["tp"], r["fp"]) == (2, 0)
    r = oracle.threshold_sweep(np.array([-3.0, -2.0, 1.0, 0.0, 5.0]), y)      # reversed
    assert r["auc"] == 0.0
    r = oracle.threshold_sweep(np.zeros(5), y)                                # all equal
    assert r["auc"] == 0.5 and r["u2"] == 6 and r["f1"] == pytest.approx(2 * 2 / (2 * 2 + 3))
    r = oracle.threshold_sweep(np.array([1.0, 2.0]), np.array([0, 0]))        # no copy positions
    assert math.isnan(r["auc"]) and r["f1"] == 0.0 and r["t"] == math.inf


def test_f1_tie_keeps_the_highest_threshold():
    # thresholds 4 (TP 1, FP 0) and 1 (TP 2, FP 2) both give F1 = 2/3, the maximum;
    # the higher one is kept
    z = np.array([4.0, 3.0, 2.0, 1.0])
    y = np.array([1, 0, 0, 1])
    r = oracle.threshold_sweep(z, y)
    assert r["f1"] == pytest.approx(2 / 3) and r["t"] == 4.0 and (r["tp"], r["fp"]) == (1, 0)


@pytest.mark.parametrize("seed", range(5))
def test_sweep_against_sklearn(seed):
    rng = np.random.default_rng(seed)
    n = 400
    y = (rng.random(n) < 0.3).astype(int)
    z = np.round(rng.standard_normal(n) + 1.5 * y, 1)          # rounding makes ties
    r = oracle.threshold_sweep(z, y)
    assert r["auc"] == pytest.approx(roc_auc_score(y, z), abs=1e-12)
    assert r["f1"] == pytest.approx(f1_score(y, (z >= r["t"]).astype(int)), abs=1e-12)
    prec, rec, _ = precision_recall_curve(y, z)
    with np.errstate(invalid="ignore", divide="ignore"):
        f1s = np.where(prec + rec > 0, 2 * prec * rec / (prec + rec), 0.0)
    assert r["f1"] == pytest.approx(np.nanmax(f1s), abs=1e-12)


def test_calibrate_picks_best_layer_lowest_on_ties():
    y = np.array([1, 1, 0, 0])
    z = np.array([[0.0, 1.0, 1.0, 0.0],          # F1 2/3 at best
                  [3.0, 2.0, 1.0, 0.0],          # F1 1
                  [3.0, 2.0, 1.0, 0.0]])         # F1 1 as well: the lower layer wins
    c = oracle.calibrate(z, y)
    assert c["layer"] == 1 and c["t"] == 2.0
    assert c["tau"] == pytest.approx(1 / (1 + math.exp(-2.0)))


def test_calibrate_tau_at_infinite_thresholds():
    # sigma's limits: t = -inf (every score is -inf, all copies) gives tau = 0,
    # no positive at all gives t = +inf and tau = 1
    inf = float("inf")
    r = oracle.calibrate(np.array([[-inf, -inf]]), np.array([1, 1], np.uint8))
    assert r["t"] == -inf and r["tau"] == 0.0 and r["per_layer"][0]["f1"] == 1.0
    r = oracle.calibrate(np.array([[0.3, -2.0]]), np.array([0, 0], np.uint8))
    assert r["t"] == inf and r["tau"] == 1.0
    r = oracle.calibrate(np.array([[math.log(0.4 / 0.6), -5.0]]), np.array([1, 0], np.uint8))
    assert abs(r["tau"] - 0.4) < 1e-15
