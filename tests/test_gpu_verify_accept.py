"""GPU parity of ssd_blocktri_verify_accept (the verification pass and the accept in
the verification's launches) and of the greedy LM head's folded argmax.

Bars:
* verify_accept against blocktri_verify followed by accept_longest on the same
  inputs: attention output, argmax and every accept output equal bit for bit (the
  two paths share their kernels; only the launch that runs the accept differs), on
  two calls in a row with different inputs.
* the argmax against the oracle's LM head on the device's attention output
  (check_verify's bars), and the accept outputs against the oracle's accept on the
  device's argmax, bit for bit.
* exact ties: two vocabulary rows with identical weights give identical logits;
  where they hold a row's maximum, the argmax is the lower of the two indices,
  whether they sit in one workgroup's tile or in two.
* NaN logits never win: with the weights of the most frequent winners set to NaN,
  the argmax is the oracle's over the remaining columns; with every weight NaN,
  every row reports -1 and nothing is accepted.
Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import copy_draft_verification_amd as cdv
import oracle
from parity_lib import ARGMAX_MARGIN, DEV, Dev, check_verify, host, widen_out
from workloads import f32_to_bf16_bits, generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cdv.load()


def _retrieve(wl, d):
    s = wl.spec
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, None)
    torch.cuda.synchronize()
    return g


def _both(wl, d, g):
    """verify_accept, then the two separate calls; returns both results (host)."""
    s = wl.spec
    a1, m1, acc1 = cdv.blocktri_verify_accept(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand"],
                                              g["cand_len"], g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    a0, m0 = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                 g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    acc0 = cdv.accept_longest(g["cand"], g["cand_len"], g["copy_gate"], m0, s.W, s.D)
    torch.cuda.synchronize()
    assert torch.equal(a0, a1) and torch.equal(m0, m1)
    for k in acc0:
        assert torch.equal(acc0[k], acc1[k]), k
    o = oracle.accept_longest(host(g["cand"]), host(g["cand_len"]), host(g["copy_gate"]).astype(bool),
                              host(m1), s.W, s.D)
    for k in ("accept_len", "best_w", "best_len", "next_token"):
        assert np.array_equal(host(acc1[k]), o[k]), k
    return m1, acc1


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),                                        # fp32: reduce and accept launches
    ("small_f32", {}),
    ("small_bf16", {"lm_std": 1.0}),
    ("small_bf16", {"anchor": "natural", "B": 6, "seed": 2101, "lm_std": 1.0}),
    ("small_bf16", {"B": 32, "n": (200, 400), "seed": 2203, "lm_std": 1.0}),  # 8 sequences per wave
    ("small_bf16", {"W": 64, "D": 1, "lm_std": 1.0}),
    ("small_bf16", {"W": 1, "D": 64, "lm_std": 1.0}),
    ("llama8b_b1", {"lm_std": 1.0}),
])
def test_verify_accept_matches_separate_calls(name, over):
    wl = generate(name, **over)
    s = wl.spec
    print(f"[case] verify_accept {s.name} {over} B={s.B} W={s.W} D={s.D} V={s.V} dtype={s.dtype}",
          flush=True)
    d = Dev(wl)
    g = _retrieve(wl, d)
    # the argmax against the oracle (sampled rows at the full shape)
    rows = None
    if s.V > 10000:
        rng = np.random.default_rng(3)
        rows = [(0, int(r)) for r in rng.choice(wl.R, 24, replace=False)] + [(0, 0)]
    check_verify(wl, d, g, rows_att=rows, rows_lm=rows, logits=s.V <= 10000)
    m, acc = _both(wl, d, g)
    print(f"[ok] best_len {host(acc['best_len']).tolist()[:8]} "
          f"gates {int(host(g['copy_gate']).sum())}", flush=True)


def test_verify_accept_twice_with_other_inputs():
    # the second call must not see the first call's keys or finished-workgroup count
    for seed, B in ((2301, 3), (2302, 5)):
        wl = generate("small_bf16", B=B, seed=seed, lm_std=1.0)
        print(f"[case] verify_accept seed={seed} B={B}", flush=True)
        d = Dev(wl)
        g = _retrieve(wl, d)
        check_verify(wl, d, g)
        _both(wl, d, g)


def test_verify_accept_all_gates_closed():
    wl = generate("small_bf16")
    s = wl.spec
    print("[case] verify_accept with every gate closed", flush=True)
    d = Dev(wl)
    fire = torch.zeros(s.B, dtype=torch.uint8, device=DEV)
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, fire)
    m, acc = _both(wl, d, g)
    assert torch.all(m == -1)
    assert host(acc["best_w"]).tolist() == [-1] * s.B


# The bf16 LM head starts vocabulary tile t's contraction at k-slab t mod (hid / 64)
# (8 at hidden size 512), so two tiles sum in the same order, and give equal logits
# for equal weights, when their indices agree mod 8: tiles 0 and 8 (rows 100 and
# 2148), 2 and 10 (rows 700 and 2748).
@pytest.mark.parametrize("pairs", [((5, 6),), ((100, 2148),), ((40, 41), (700, 2748))])
def test_argmax_exact_ties_take_the_lower_index(pairs):
    wl = generate("small_bf16", lm_std=0.02)
    s = wl.spec
    print(f"[case] argmax ties, duplicated vocabulary rows {pairs}", flush=True)
    lm = wl.lm_head
    for lo, hi in pairs:
        # x64 (exact in bf16): the pair holds the maximum of about half the rows
        lm[lo] = f32_to_bf16_bits(oracle.bf16_bits_to_f64(lm[lo]).astype(np.float32) * np.float32(64.0))
        lm[hi] = lm[lo]
    d = Dev(wl)
    g = _retrieve(wl, d)
    logits = torch.empty(s.B, wl.R, s.V, dtype=torch.float32, device=DEV)
    a, m = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                               g["copy_gate"], d.lm, s.W, s.D, wl.scale, logits_out=logits)
    torch.cuda.synchronize()
    L, am = host(logits), host(m)
    hits = 0
    for b in range(s.B):
        for r in range(wl.R):
            if am[b, r] < 0:
                continue
            row = L[b, r]
            for lo, hi in pairs:
                assert row[lo] == row[hi]
                if row[lo] == row.max():
                    assert am[b, r] == lo, (b, r, am[b, r], lo)
                    hits += 1
            assert row[am[b, r]] == row.max()
            assert am[b, r] == int(np.argmax(row))
    print(f"[ok] rows won by a duplicated pair: {hits}", flush=True)
    assert hits > 0


def _nan_rows(lm, rows):
    if lm.dtype == np.uint16:
        lm[rows] = np.uint16(0x7FC0)       # bf16 quiet NaN
    else:
        lm[rows] = np.float32(np.nan)


@pytest.mark.parametrize("name", ["tiny", "small_f32", "small_bf16"])
def test_nan_logits_never_win(name):
    wl = generate(name, lm_std=1.0)
    s = wl.spec
    print(f"[case] NaN vocabulary rows, {name}", flush=True)
    # the winners without NaN, from a first pass
    d = Dev(wl)
    g = _retrieve(wl, d)
    _, m0 = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    torch.cuda.synchronize()
    won = host(m0)[host(m0) >= 0]
    top, counts = np.unique(won, return_counts=True)
    hit = top[np.argsort(-counts)][:4].tolist()
    _nan_rows(wl.lm_head, hit + [s.V - 1])
    d = Dev(wl)
    attn, m, acc = cdv.blocktri_verify_accept(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc,
                                              g["cand"], g["cand_len"], g["copy_gate"], d.lm,
                                              s.W, s.D, wl.scale)
    torch.cuda.synchronize()
    am = host(m)
    O = widen_out(attn).reshape(s.B, wl.R, s.Hq * s.d)
    real = am >= 0
    assert real.sum() == (host(m0) >= 0).sum()
    L = oracle.lm_logits(O[real], wl.lm_head)
    assert np.all(np.isnan(L[:, hit]))
    L[np.isnan(L)] = -np.inf
    pred, _, margin = oracle.argmax_with_margin(L)
    ok = margin >= ARGMAX_MARGIN
    assert np.array_equal(am[real][ok], pred[ok])
    assert not np.isin(am[real], hit).any()
    o = oracle.accept_longest(host(g["cand"]), host(g["cand_len"]), host(g["copy_gate"]).astype(bool),
                              am, s.W, s.D)
    for k in ("accept_len", "best_w", "best_len", "next_token"):
        assert np.array_equal(host(acc[k]), o[k]), k
    print(f"[ok] NaN rows {hit}; rows checked {int(ok.sum())} of {int(real.sum())}", flush=True)


@pytest.mark.parametrize("name", ["tiny", "small_bf16"])
def test_all_nan_logits_give_minus_one(name):
    wl = generate(name)
    s = wl.spec
    print(f"[case] every vocabulary row NaN, {name}", flush=True)
    _nan_rows(wl.lm_head, slice(None))
    d = Dev(wl)
    g = _retrieve(wl, d)
    _, m, acc = cdv.blocktri_verify_accept(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand"],
                                           g["cand_len"], g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    torch.cuda.synchronize()
    assert np.all(host(m) == -1)
    o = oracle.accept_longest(host(g["cand"]), host(g["cand_len"]), host(g["copy_gate"]).astype(bool),
                              host(m), s.W, s.D)
    for k in ("accept_len", "best_w", "best_len", "next_token"):
        assert np.array_equal(host(acc[k]), o[k]), k
