"""GPU parity of verification at T > 0 (ssd_blocktri_verify_sample, ssd_accept_sample)
against the oracle (oracle/sampling.py).

The sampling pass runs the same attention and LM-head contraction as the greedy
pass, so the greedy pass with logits_out supplies the device's own logits L (whose
parity with the float64 oracle the greedy tests establish).  On those logits:
* trie (n_children, children, child_w): bit-exact against oracle.candidate_trie.
* lse and child logits / T: |gpu - oracle| <= 1e-5 * (1 + |value|) (float32
  exp / log / sum against float64 on the same float32 logits).
* residual draw per real row: equal to the oracle's Gumbel-max draw (float64 noise
  from the same Philox words) wherever the oracle's top-2 score gap is >= 1e-4;
  closer rows are counted.
* the walk: on the device's own row statistics, best_w / best_len / next_token equal
  the oracle's walk exactly unless a test on the path has |u - r| < 1e-5 (counted).
* the law of the first emitted token over many seeds: chi-square against
  softmax(anchor logits / T).
Every test prints its case before touching the GPU."""
import numpy as np
import pytest
import torch
from scipy.stats import chisquare

import copy_draft_verification_amd as cdv
import oracle
from oracle import sampling as S
from oracle.attention import real_rows
from parity_lib import DEV, Dev, check_kgram, check_probe, host, up, widen_out
from workloads import generate

pytestmark = pytest.mark.gpu

STAT_TOL = 1e-5
DRAW_MARGIN = 1e-4
WALK_TIE = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cdv.load()


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _retrieve(wl):
    d = Dev(wl)
    fire, _, _ = check_probe(wl, d)
    g, _ = check_kgram(wl, d, fire, host(fire).astype(bool))
    return d, g


def _sample(wl, d, g, T, seed):
    s = wl.spec
    attn, rows = cdv.blocktri_verify_sample(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand"],
                                            g["cand_len"], g["copy_gate"], d.lm, s.W, s.D,
                                            wl.scale, T, seed)
    acc = cdv.accept_sample(rows, g["copy_gate"], s.W, s.D, seed)
    torch.cuda.synchronize()
    return attn, {k: host(v) for k, v in rows.items()}, {k: host(v) for k, v in acc.items()}


def _greedy_logits(wl, d, g):
    s = wl.spec
    L = torch.empty(s.B, wl.R, s.V, dtype=torch.float32, device=DEV)
    attn, _ = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                  g["copy_gate"], d.lm, s.W, s.D, wl.scale, logits_out=L)
    torch.cuda.synchronize()
    return attn, host(L)


def _check_rows(wl, g, rows, L, T, seed, row_sample=None):
    """Trie exact; lse / child logits tight; residual draws equal outside the margin."""
    s = wl.spec
    B, R, W, D = s.B, wl.R, s.W, s.D
    cand, cl, gate = host(g["cand"]), host(g["cand_len"]), host(g["copy_gate"]).astype(bool)
    close = 0
    checked = 0
    for b in range(B):
        kids = S.candidate_trie(cand[b], cl[b], gate[b], W, D)
        real = set(real_rows(cl[b], gate[b], W, D))
        for r in range(R):
            nc = int(rows["n_children"][b, r])
            want = kids[r]
            assert nc == len(want), (b, r, nc, want)
            assert [(int(rows["children"][b, r, k]), int(rows["child_w"][b, r, k])) for k in range(nc)] == want
            if r not in real:
                assert rows["lse"][b, r] == -np.inf and rows["resample"][b, r] == -1
                continue
            if row_sample is not None and (b, r) not in row_sample and nc == 0:
                continue
            t = L[b, r].astype(np.float64) / T
            mx = t.max()
            lse = mx + np.log(np.exp(t - mx).sum())
            assert abs(rows["lse"][b, r] - lse) <= STAT_TOL * (1 + abs(lse)), (b, r)
            for k, (x, _) in enumerate(want):
                assert abs(rows["child_logit"][b, r, k] - t[x]) <= STAT_TOL * (1 + abs(t[x])), (b, r, k)
            y = t + S.gumbel_row(seed, b * R + r, s.V)
            for x, _ in want:
                y[x] = -np.inf
            order = np.argsort(-y, kind="stable")
            if y[order[0]] - y[order[1]] < DRAW_MARGIN:
                close += 1
                continue
            assert rows["resample"][b, r] == order[0], (b, r)
            checked += 1
    return checked, close


def _walk_on_device_stats(wl, g, rows, seed):
    """The oracle walk on the device's own statistics, with the same uniforms."""
    s = wl.spec
    R, W, D = wl.R, s.W, s.D
    gate = host(g["copy_gate"]).astype(bool)
    out, ties = [], 0
    for b in range(s.B):
        if not gate[b]:
            out.append((-1, 0, -1))
            continue
        row, j, bw = 0, 0, 0
        while True:
            gr = b * R + row
            nc = int(rows["n_children"][b, row])
            lse = float(rows["lse"][b, row])
            tried, moved = 0.0, False
            for k in range(nc):
                p = float(np.exp(np.float64(rows["child_logit"][b, row, k]) - lse))
                r = S.accept_ratio(p, tried)
                u = S.accept_uniform(seed, gr, k)
                if abs(u - r) < WALK_TIE:
                    ties += 1
                if u < r:
                    w = int(rows["child_w"][b, row, k])
                    bw, row, j, moved = w, 1 + w * D + j, j + 1, True
                    break
                tried += p
            if not moved:
                out.append((bw, j, int(rows["resample"][b, row])))
                break
    return out, ties


def _check_walk(wl, g, rows, acc, seed):
    want, ties = _walk_on_device_stats(wl, g, rows, seed)
    got = list(zip(acc["best_w"].tolist(), acc["best_len"].tolist(), acc["next_token"].tolist()))
    if ties == 0:
        assert got == want, (got, want)
    return ties


@pytest.mark.parametrize("name,over,T", [
    ("small_bf16", {"lm_std": 1.0}, 1.0),
    ("small_bf16", {"lm_std": 1.0}, 0.25),
    ("small_bf16", {}, 1.0),
    ("small_bf16", {"anchor": "natural", "B": 6, "seed": 2101, "lm_std": 1.0}, 0.7),
    ("small_bf16", {"W": 3, "D": 7, "lm_std": 1.0}, 1.0),
    ("small_bf16", {"W": 64, "D": 1, "lm_std": 1.0}, 1.0),
    ("small_bf16", {"W": 1, "D": 64, "lm_std": 1.0}, 2.0),
])
def test_sample_rows_and_walk(name, over, T):
    wl = generate(name, **over)
    seed = 0x1234_5678_9ABC_DEF0 + len(over)
    _case(f"sample {name} {over} T={T} B={wl.spec.B} W={wl.spec.W} D={wl.spec.D} V={wl.spec.V}")
    d, g = _retrieve(wl)
    attn0, L = _greedy_logits(wl, d, g)
    attn, rows, acc = _sample(wl, d, g, T, seed)
    assert torch.equal(attn.view(torch.int16), attn0.view(torch.int16))   # same attention
    checked, close = _check_rows(wl, g, rows, L, T, seed)
    ties = _check_walk(wl, g, rows, acc, seed)
    print(f"[ok] draws checked {checked} close {close} walk ties {ties} "
          f"best_len {acc['best_len'].tolist()}", flush=True)


def test_walk_deep_paths_on_crafted_statistics():
    # the device walk on statistics that accept often: child logits / T set so that
    # p(child) is 0.2 .. 0.9 (lse = 0), on the device's own trie of a workload whose
    # candidates share prefixes
    wl = generate("small_bf16", W=12, D=9, lm_std=1.0)
    _case(f"deep walks W={wl.spec.W} D={wl.spec.D}")
    d, g = _retrieve(wl)
    _, rows_dev = cdv.blocktri_verify_sample(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand"],
                                             g["cand_len"], g["copy_gate"], d.lm, wl.spec.W,
                                             wl.spec.D, wl.scale, 1.0, 5)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    total_len = 0
    for trial in range(8):
        cl = np.log(rng.uniform(0.2, 0.9, rows_dev["child_logit"].shape)).astype(np.float32)
        rows_dev["child_logit"].copy_(torch.from_numpy(cl))
        rows_dev["lse"].zero_()
        seed = 1000 + trial
        acc = cdv.accept_sample(rows_dev, g["copy_gate"], wl.spec.W, wl.spec.D, seed)
        torch.cuda.synchronize()
        rows = {k: host(v) for k, v in rows_dev.items()}
        acc = {k: host(v) for k, v in acc.items()}
        ties = _check_walk(wl, g, rows, acc, seed)
        assert ties == 0
        total_len += int(acc["best_len"].sum())
    assert total_len > 8                 # the walks did go deep


def test_first_token_follows_the_target():
    # over many seeds, the first emitted token (the first accepted token, else the
    # residual draw at the anchor) follows softmax(anchor logits / T)
    wl = generate("small_bf16", B=1, lm_std=1.0)
    T = 1.5
    _case(f"first-token law over seeds, V={wl.spec.V} T={T}")
    d, g = _retrieve(wl)
    _, L = _greedy_logits(wl, d, g)
    p = S.softmax_T(L[0, 0].astype(np.float64), T)
    n = 3000
    cells = {}
    s = wl.spec
    cand = host(g["cand"])
    rows = None
    for seed in range(n):
        _, rows = cdv.blocktri_verify_sample(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand"],
                                             g["cand_len"], g["copy_gate"], d.lm, s.W, s.D,
                                             wl.scale, T, seed, rows=rows)
        acc = cdv.accept_sample(rows, g["copy_gate"], s.W, s.D, seed)
        bl, nt, bw = (int(acc["best_len"][0]), int(acc["next_token"][0]), int(acc["best_w"][0]))
        first = int(cand[0, bw, 0]) if bl > 0 else nt
        cells[first] = cells.get(first, 0) + 1
    torch.cuda.synchronize()
    # pool tokens into bins of expected count >= 20
    order = np.argsort(-p)
    bins, cur, mass = [], [], 0.0
    for x in order:
        cur.append(int(x))
        mass += p[x]
        if mass * n >= 20:
            bins.append(cur)
            cur, mass = [], 0.0
    if cur:
        bins[-1].extend(cur)
    obs = np.array([sum(cells.get(x, 0) for x in b_) for b_ in bins], dtype=float)
    exp = np.array([p[b_].sum() * n for b_ in bins])
    assert obs.sum() == n
    assert chisquare(obs, exp).pvalue > 1e-4


def test_all_gates_closed_sample():
    wl = generate("small_bf16")
    _case("sampling with every gate closed")
    d = Dev(wl)
    s = wl.spec
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D,
                           torch.zeros(s.B, dtype=torch.uint8, device=DEV))
    attn, rows, acc = _sample(wl, d, g, 1.0, 3)
    assert np.all(acc["best_w"] == -1) and np.all(acc["next_token"] == -1)
    assert np.all(acc["best_len"] == 0)
    assert np.all(rows["n_children"] == 0) and np.all(rows["resample"] == -1)
    assert np.all(widen_out(attn) == 0.0)


@pytest.mark.slow
def test_full_llama8b_b1_sample():
    wl = generate("llama8b_b1")
    T, seed = 1.0, 0xC0FFEE
    _case(f"sample llama8b_b1 T={T} (every node row and 48 sampled rows)")
    d, g = _retrieve(wl)
    _, L = _greedy_logits(wl, d, g)
    _, rows, acc = _sample(wl, d, g, T, seed)
    rng = np.random.default_rng(1)
    sample = {(0, int(r)) for r in rng.integers(0, wl.R, 48)}
    checked, close = _check_rows(wl, g, rows, L, T, seed, row_sample=sample)
    ties = _check_walk(wl, g, rows, acc, seed)
    print(f"[ok] draws checked {checked} close {close} walk ties {ties}", flush=True)
