"""Pins for the oracle's block-triangular attention.

SwitchSD paper §3.3 "Parallel Verification with Block-Triangular Attention"
(write-up §2.6): candidate w's tokens see the whole prefix and earlier tokens of
w only; §3.3 "Overall Framework": verification keeps correctness, i.e. each
candidate row equals what plain causal decoding of that candidate sees.

Independent references used here: a hand-written visibility table, torch's
scaled_dot_product_attention (float64, CPU) with a mask built from
block_diag(tril) in this file, per-candidate causal attention written as a loop,
and closed forms (constant values, a two-key softmax, the GQA head mapping).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import allowed_keys


def test_hand_built_visibility_table():
    # n = 2 (P0, P1 = anchor), W = 2, D = 2; key order [P0, P1, c00, c01, c10, c11]
    want = {0: "110000", 1: "111000", 2: "111100", 3: "110010", 4: "110011"}
    for r, bits in want.items():
        got = "".join("1" if v else "0" for v in allowed_keys(2, 2, 2, r))
        assert got == bits, (r, got)


def _case(seed, B=2, Hq=4, Hkv=2, d=8, W=3, D=4, ns=(7, 5), lens=((4, 2, 0), (1, 4, 3)),
          gates=(True, True)):
    rng = np.random.default_rng(seed)
    R = 1 + W * D
    N = sum(ns)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ns)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(q=f(B, R, Hq, d), k_pre=f(N, Hkv, d), v_pre=f(N, Hkv, d),
                k_cand=f(B, W * D, Hkv, d), v_cand=f(B, W * D, Hkv, d),
                cu_len=cu, cand_len=np.array(lens, dtype=np.int32),
                copy_gate=np.array(gates), Hq=Hq, Hkv=Hkv, d=d, W=W, D=D)


def _run(c, **kw):
    return oracle.blocktri_attention(c["q"], c["k_pre"], c["v_pre"], c["cu_len"], c["k_cand"],
                                     c["v_cand"], c["cand_len"], c["copy_gate"], c["Hq"], c["Hkv"],
                                     c["d"], c["W"], c["D"], **kw)


def test_matches_sdpa_with_block_diag_tril_mask():
    c = _case(1)
    out, ev = _run(c)
    W, D, g = c["W"], c["D"], c["Hq"] // c["Hkv"]
    for b in range(2):
        n = int(c["cu_len"][b + 1] - c["cu_len"][b])
        # mask over [prefix | candidates]: anchor row sees prefix; candidate block is
        # block_diag of W lower-triangular D x D blocks
        tri = torch.block_diag(*[torch.tril(torch.ones(D, D, dtype=torch.bool))] * W)
        mask = torch.zeros(1 + W * D, n + W * D, dtype=torch.bool)
        mask[:, :n] = True
        mask[1:, n:] = tri
        q = torch.from_numpy(c["q"][b]).double().permute(1, 0, 2)            # [Hq, R, d]
        kp = torch.from_numpy(c["k_pre"][c["cu_len"][b]:c["cu_len"][b + 1]]).double()
        vp = torch.from_numpy(c["v_pre"][c["cu_len"][b]:c["cu_len"][b + 1]]).double()
        K = torch.cat([kp, torch.from_numpy(c["k_cand"][b]).double()], 0).permute(1, 0, 2)
        V = torch.cat([vp, torch.from_numpy(c["v_cand"][b]).double()], 0).permute(1, 0, 2)
        K = K.repeat_interleave(g, dim=0)
        V = V.repeat_interleave(g, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask)
        ref = ref.permute(1, 0, 2).reshape(1 + W * D, -1).numpy()
        for (bb, r) in ev:
            if bb == b:
                np.testing.assert_allclose(out[b, r], ref[r], rtol=0, atol=1e-12)


def test_equals_independent_causal_pass_per_candidate():
    # row (w, j) == causal attention of sequence prefix + c_w[0..j] run alone (loop form)
    c = _case(2)
    out, ev = _run(c)
    d, g = c["d"], c["Hq"] // c["Hkv"]
    for (b, r) in ev:
        if r == 0:
            continue
        w, j = divmod(r - 1, c["D"])
        lo, hi = c["cu_len"][b], c["cu_len"][b + 1]
        for h in range(c["Hq"]):
            kv = h // g
            keys = [c["k_pre"][t, kv].astype(np.float64) for t in range(lo, hi)]
            vals = [c["v_pre"][t, kv].astype(np.float64) for t in range(lo, hi)]
            for jj in range(j + 1):
                keys.append(c["k_cand"][b, w * c["D"] + jj, kv].astype(np.float64))
                vals.append(c["v_cand"][b, w * c["D"] + jj, kv].astype(np.float64))
            qv = c["q"][b, r, h].astype(np.float64)
            s = [float(qv @ k) / math.sqrt(d) for k in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            o = sum(ei * v for ei, v in zip(e, vals)) / sum(e)
            np.testing.assert_allclose(out[b, r, h * d:(h + 1) * d], o, rtol=0, atol=1e-12)


def test_constant_values_give_that_value():
    c = _case(3)
    c["v_pre"][:] = 2.5
    c["v_cand"][:] = 2.5
    out, ev = _run(c)
    for (b, r) in ev:
        np.testing.assert_allclose(out[b, r], 2.5, rtol=0, atol=1e-13)


def test_two_key_softmax_by_hand_catches_scale():
    # n = 1, W = 1, D = 1, L = 1, d = 4 -> scale 1/2.  anchor row sees only P0 -> O = v0.
    # row (0,0) sees P0 and c00: q.k0 = 0, q.k1 = 2 ln 3 -> scaled scores 0, ln 3
    # -> weights 1/4, 3/4 -> O = v0/4 + 3 v1/4
    q = np.zeros((1, 2, 1, 4), np.float32)
    q[0, 1, 0, 0] = 1.0
    k_pre = np.zeros((1, 1, 4), np.float32)
    k_c = np.zeros((1, 1, 1, 4), np.float32)
    k_c[0, 0, 0, 0] = np.float32(2 * math.log(3.0))
    v_pre = np.array([[[4.0, 0.0, -8.0, 1.0]]], np.float32)
    v_c = np.array([[[[0.0, 4.0, 8.0, 1.0]]]], np.float32)
    out, _ = oracle.blocktri_attention(q, k_pre, v_pre, np.array([0, 1]), k_c, v_c,
                                       np.array([[1]]), np.array([True]), 1, 1, 4, 1, 1)
    np.testing.assert_allclose(out[0, 0], v_pre[0, 0], atol=1e-15)
    w1 = 3.0 * float(np.exp(np.float64(np.float32(2 * math.log(3.0))) / 2 - math.log(3.0)))
    expect = (v_pre[0, 0] + w1 * v_c[0, 0, 0]) / (1 + w1)
    np.testing.assert_allclose(out[0, 1], expect, atol=1e-12)
    np.testing.assert_allclose(out[0, 1], [1.0, 3.0, 4.0, 1.0], atol=1e-6)


def test_gqa_head_mapping_and_head_major_layout():
    # Hq = 4, Hkv = 2: heads 0,1 read kv head 0 (values 3), heads 2,3 read kv head 1 (values 7)
    c = _case(4)
    c["v_pre"][:, 0, :] = 3.0
    c["v_pre"][:, 1, :] = 7.0
    c["v_cand"][:, :, 0, :] = 3.0
    c["v_cand"][:, :, 1, :] = 7.0
    out, ev = _run(c)
    d = c["d"]
    for (b, r) in ev:
        for h, val in enumerate([3.0, 3.0, 7.0, 7.0]):
            np.testing.assert_allclose(out[b, r, h * d:(h + 1) * d], val, atol=1e-13)


def test_candidates_are_isolated_and_anchor_ignores_candidates():
    c = _case(5)
    base, ev = _run(c)
    for w_bad in range(c["W"]):
        c2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
        sl = slice(w_bad * c["D"], (w_bad + 1) * c["D"])
        c2["k_cand"][:, sl] += 3.0
        c2["v_cand"][:, sl] -= 5.0
        out, _ = _run(c2)
        for (b, r) in ev:
            w = None if r == 0 else (r - 1) // c["D"]
            if w != w_bad:
                assert np.array_equal(out[b, r], base[b, r])


def test_unreal_rows_and_closed_gate_are_zero():
    c = _case(6, gates=(True, False))
    out, ev = _run(c)
    assert all(b == 0 for b, _ in ev)
    assert np.all(out[1] == 0)
    real = {r for _, r in ev}
    for r in range(1 + c["W"] * c["D"]):
        if r not in real:
            assert np.all(out[0, r] == 0)
    assert len(real) == 1 + int(c["cand_len"][0].sum())


def test_row_subset_matches_full():
    c = _case(7)
    full, ev = _run(c)
    sub, ev2 = _run(c, rows=[(1, 0), (0, 6), (1, 9), (0, 12)])   # (0,12): w=2 has L=0
    assert set(ev2) == {(1, 0), (0, 6), (1, 9)}
    for (b, r) in ev2:       # BLAS may order sums differently for another row count
        np.testing.assert_allclose(sub[b, r], full[b, r], rtol=0, atol=1e-13)
