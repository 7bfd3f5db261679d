"""Pins for the oracle's probe (SwitchSD paper §3.2 Layer and Threshold Selection;
write-up §2.3 bias-free linear probe, §2.5 gate condition PR(H) >= tau).

The probe's formula is missing from the pages; the reading is PR(h) = sigmoid(w.h).
Each case below fails for a plausible slip: comparing the raw score with tau,
a flipped sign, an added bias, a dropped term or a wrong bf16 widening.
"""
import math
import struct

import numpy as np
import pytest

import oracle
from oracle.bf16 import bf16_bits_to_f64



def _unit(hid, k, c):
    w = np.zeros(hid, dtype=np.float32)
    h = np.zeros((1, hid), dtype=np.float32)
    w[k] = 1.0
    h[0, k] = c
    return w, h


def test_logit_closed_form():
    assert oracle.logit(0.4) == pytest.approx(math.log(2.0 / 3.0), abs=1e-15)
    assert oracle.logit(0.5) == 0.0


@pytest.mark.parametrize("c,fires", [(-0.40, True), (-0.41, False), (0.2, True), (-1.0, False),
                                     (3.0, True)])
def test_unit_vector_closed_form(c, fires):
    # w = e_k, h = c e_k  =>  z = c exactly and PR = 1/(1+e^-c); logit(0.4) = -0.4055
    w, h = _unit(16, 11, c)
    r = oracle.probe_score(h, w, 0.4)
    assert r["z"][0] == np.float64(np.float32(c))
    assert r["score"][0] == pytest.approx(1.0 / (1.0 + math.exp(-float(np.float32(c)))), rel=1e-15)
    assert bool(r["fire"][0]) is fires
    assert r["margin"][0] == pytest.approx(float(np.float32(c)) - math.log(2 / 3), abs=1e-12)


def test_last_and_first_terms_count():
    hid = 33
    for k in (0, hid - 1):
        w, h = _unit(hid, k, 5.0)
        assert oracle.probe_score(h, w, 0.4)["z"][0] == 5.0


def test_hand_example_zero_score():
    # z = 1*0.5 + 2*0.25 + (-1)*1 = 0 -> PR = 0.5; >= is inclusive
    w = np.array([1.0, 2.0, -1.0], dtype=np.float32)
    h = np.array([[0.5, 0.25, 1.0]], dtype=np.float32)
    r = oracle.probe_score(h, w, 0.5)
    assert r["z"][0] == 0.0 and r["score"][0] == 0.5 and bool(r["fire"][0])
    assert not bool(oracle.probe_score(h, w, 0.6)["fire"][0])
    assert r["S"][0] == 2.0


def test_zero_state_means_no_bias():
    # a bias-free probe scores the zero vector at exactly 0.5
    w = np.random.default_rng(0).standard_normal(64).astype(np.float32)
    r = oracle.probe_score(np.zeros((2, 64), np.float32), w, 0.4)
    assert np.all(r["z"] == 0.0) and np.all(r["score"] == 0.5) and np.all(r["fire"])


def test_bf16_widening_known_bits():
    expect = {0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0xC000: -2.0, 0x0000: 0.0,
              0x0001: struct.unpack("<f", struct.pack("<I", 1 << 16))[0], 0x7F7F: 3.3895313892515355e38}
    bits = np.array(list(expect.keys()), dtype=np.uint16)
    got = bf16_bits_to_f64(bits)
    for b, g in zip(bits, got):
        assert g == expect[int(b)]


def test_bf16_state_probe():
    # h = [1.0, 0.5, -2.0] as bf16 bits; w = [1, 1, 1] -> z = -0.5
    h = np.array([[0x3F80, 0x3F00, 0xC000]], dtype=np.uint16)
    w = np.ones(3, dtype=np.float32)
    r = oracle.probe_score(h, w, 0.4)
    assert r["z"][0] == -0.5
    assert not bool(r["fire"][0])          # sigmoid(-0.5) = 0.3775 < 0.4


def test_rejects_tau_outside_unit_interval():
    with pytest.raises(ValueError):
        oracle.probe_score(np.zeros((1, 4), np.float32), np.zeros(4, np.float32), 1.0)


def test_generator_statistics_sanity():
    # not parity: the synthetic anchor state at copy positions is shifted by 3 w/|w|,
    # so z | copy ~ N(3|w|, |w|^2) with |w| ~ 1.  Over many draws the mean is near 3.
    from workloads import generate
    zs = []
    for seed in range(40):
        wl = generate("small_f32", with_tensors=False, seed=5000 + seed, B=1)
        if wl.copy_pos[-1]:
            zs.append(oracle.probe_score(wl.h, wl.w, 0.4)["z"][0])
    assert len(zs) > 10
    assert 2.0 < np.mean(zs) < 4.0
