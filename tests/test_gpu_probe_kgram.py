"""GPU parity of the fused probe + retrieval call (ssd_probe_kgram_retrieve) against
the oracle's probe_score and kgram_retrieve, and against the two separate calls.

Bars (those of the separate calls):
* z: |z_gpu - z| <= 1e-5 * sum|w_k h_k|; the decision equals the oracle's outside
  that tie zone (tie-zone cases are counted).
* retrieval: match positions, counts, candidates, lengths and gate equal, bit for
  bit, the oracle's retrieval gated by the GPU's own decision (which equals the
  oracle's wherever it is compared), and the separate kgram call's outputs.
Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch

import copy_draft_verification_amd as cdv
import oracle
from parity_lib import DEV, PROBE_TIE, Dev, host
from workloads import generate, generate_with_ids, spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cdv.load()


def _fused_vs_oracle(wl, d, W=None, D=None, kappa=None):
    s = wl.spec
    W, D, kappa = W or s.W, D or s.D, kappa or s.kappa
    print(f"[case] probe+kgram {s.name} B={s.B} hid={s.hid} dtype={s.dtype} "
          f"n={np.diff(wl.cu_len).tolist()[:8]} kappa={kappa} W={W} D={D}", flush=True)
    z, fire, g = cdv.probe_kgram_retrieve(d.h, d.w, s.tau, d.ids, d.cu, kappa, W, D)
    torch.cuda.synchronize()
    po = oracle.probe_score(wl.h, wl.w, s.tau)
    zz, ff = host(z).astype(np.float64), host(fire).astype(bool)
    tie = np.abs(po["margin"]) < PROBE_TIE * po["S"]
    assert np.all(np.abs(zz - po["z"]) <= PROBE_TIE * po["S"]), (zz, po["z"])
    assert np.array_equal(ff[~tie], po["fire"][~tie])
    ko = oracle.kgram_retrieve(wl.ids, wl.cu_len, kappa, W, D, ff)
    for k in ("match_end", "n_match", "cand", "cand_len"):
        assert np.array_equal(host(g[k]), ko[k]), k
    assert np.array_equal(host(g["copy_gate"]).astype(bool), ko["copy_gate"])
    # the separate retrieval call, gated by the fused call's decision
    g2 = cdv.kgram_retrieve(d.ids, d.cu, kappa, W, D, fire)
    torch.cuda.synchronize()
    for k in g:
        assert torch.equal(g[k], g2[k]), k
    print(f"[ok] fired {int(ff.sum())}/{s.B} ties {int(tie.sum())} "
          f"gates {int(ko['copy_gate'].sum())} M={ko['n_match'].tolist()[:8]}", flush=True)
    return ff, ko


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("small_bf16", {}),
    ("small_f32", {}),
    ("small_bf16", {"anchor": "natural", "B": 6, "seed": 2101}),
    ("small_bf16", {"hid": 1001}),            # hidden not a multiple of 8
    ("small_f32", {"hid": 13, "B": 5}),
    ("llama8b_b1", {}),
    ("llama8b_b32", {"anchor": "natural"}),
    ("qwen3_8b_b8", {}),
    ("small_bf16", {"B": 600, "n": (50, 5000), "anchor": "natural"}),  # 256-lane workgroups
])
def test_fused_probe_kgram(name, over):
    wl = generate(name, with_tensors=False, **over)
    _fused_vs_oracle(wl, Dev(wl, tensors=False))


def test_fused_closed_and_open_probes():
    # both decisions occur: anchor states moved 4 units along +w or -w (z ~ N(0, 1)
    # otherwise; the threshold is ln(0.4 / 0.6) = -0.41)
    ids = [([1, 2, 3, 4, 5, 6, 7] * 30)[:205]] * 4
    wl = generate_with_ids(spec("small_f32"), ids, anchor_copy=[False] * 4)
    u = wl.w / np.linalg.norm(wl.w)
    for b, sign in enumerate((1, -1, 1, -1)):
        wl.h[b] += np.float32(4.0 * sign) * u
    ff, ko = _fused_vs_oracle(wl, Dev(wl, tensors=False))
    assert ff.tolist() == [True, False, True, False]
    assert ko["copy_gate"].tolist() == [True, False, True, False]


def test_fused_edge_contexts():
    rng = np.random.default_rng(7)
    ids = [
        [1, 2, 3],                                   # n <= kappa: no scan, probe still scored
        [5] * 40,
        list(range(300)),
        list(rng.integers(0, 3, 517)),
        [9] * 6,                                     # n = kappa + 1
        [4],                                         # one token
    ]
    wl = generate_with_ids(spec("small_f32"), ids)
    _fused_vs_oracle(wl, Dev(wl, tensors=False))


@pytest.mark.parametrize("W,D,kappa", [(3, 7, 2), (1, 1, 1), (64, 64, 5), (10, 20, 64)])
def test_fused_other_limits(W, D, kappa):
    rng = np.random.default_rng(W * 100 + D + 7)
    ids = [list(rng.integers(0, 4, int(rng.integers(1, 400)))) for _ in range(5)]
    ids.append([7] * 150)
    wl = generate_with_ids(spec("small_bf16", W=W, D=D), ids)
    _fused_vs_oracle(wl, Dev(wl, tensors=False), W=W, D=D, kappa=kappa)


def test_fused_long_context_matches_far_back():
    # several chunks of scanning after the probe, before the one earlier occurrence
    n = 20000
    x = list(range(1000, 1000 + n))
    x[100:105] = x[n - 5:]
    wl = generate_with_ids(spec("small_f32"), [x, x[:9000] + x[n - 5:]])
    ff, ko = _fused_vs_oracle(wl, Dev(wl, tensors=False))
    assert ff.all() and ko["match_end"][0, 0] == 104 and ko["n_match"][0] == 1


def test_fused_refuses_bad_arguments():
    wl = generate("small_bf16", with_tensors=False)
    s = wl.spec
    d = Dev(wl, tensors=False)
    print("[case] probe+kgram argument checks", flush=True)
    with pytest.raises(cdv.SwitchSDError):
        cdv.probe_kgram_retrieve(d.h, d.w, 1.5, d.ids, d.cu, s.kappa, s.W, s.D)
    with pytest.raises(cdv.SwitchSDError):
        cdv.probe_kgram_retrieve(d.h, d.w, s.tau, d.ids, d.cu, 0, s.W, s.D)
    with pytest.raises(cdv.SwitchSDError):
        cdv.probe_kgram_retrieve(d.h, d.w, s.tau, d.ids, d.cu[:-1].contiguous(), s.kappa, s.W, s.D)
    with pytest.raises(cdv.SwitchSDError):
        cdv.probe_kgram_retrieve(d.h, d.w, s.tau, d.ids, d.cu, s.kappa, s.W, s.D,
                                 z_out=torch.empty(s.B + 1, device=DEV))
