"""GPU parity of kappa-gram retrieval on long contexts and on the large-array scan:
the HIP path (through the C ABI) against the oracle, bit for bit (match positions,
match counts, candidates, candidate lengths, gates).  Every test prints its case
before touching the GPU."""
import numpy as np
import pytest
import torch

import copy_draft_verification_amd as cdv
import oracle
from parity_lib import host, up
from workloads import SCAN_N, SCAN_SIZES, scan_ids_device, scan_ids_planted

pytestmark = pytest.mark.gpu

KEYS = ("match_end", "n_match", "cand", "cand_len", "copy_gate")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cdv.load()


def _compare(g, ko, label):
    for k in KEYS:
        got = host(g[k])
        exp = ko[k].astype(got.dtype) if k == "copy_gate" else ko[k]
        bad = np.argwhere(got != exp)
        assert bad.size == 0, f"{label}: {k} differs first at {bad[0].tolist()}"


# Ragged long contexts: the anchor's kappa-gram planted at 0..14 earlier end positions
# across the context (some at or across multiples of 8192), so scans stop after W
# matches in various chunks, or read the whole context with fewer than W matches.
# Lengths around chunk multiples exercise the last (partial) chunk and its halo.
LENGTHS = [40000, 8192, 8193, 8194, 16384, 16390, 24576 + 3, 9, 6, 5000, 65536, 30001,
           8192 * 3 - 1, 12345, 100000, 20000]


@pytest.mark.parametrize("kappa,W,D", [(5, 10, 20), (1, 10, 20), (2, 3, 7), (3, 64, 64),
                                       (9, 10, 20), (64, 5, 20)])
def test_scan_planted_long_contexts(kappa, W, D):
    print(f"[case] scan planted kappa={kappa} W={W} D={D} B={len(LENGTHS)}", flush=True)
    ids, cu = scan_ids_planted(LENGTHS, kappa=kappa, seed=4100 + kappa)
    g = cdv.kgram_retrieve(up(ids), up(cu), kappa, W, D)
    torch.cuda.synchronize()
    ko = oracle.kgram_retrieve(ids, cu, kappa, W, D)
    _compare(g, ko, f"kappa={kappa}")
    print(f"[ok] M={ko['n_match'].tolist()}", flush=True)


# Many contexts (512 and more run on 256-lane workgroups, whose chunks are 2048
# end positions): random lengths plus lengths around multiples of 2048, matches
# planted at or across those multiples.
MANY = ([int(x) for x in np.random.default_rng(4301).integers(5, 12000, 560)]
        + [2048, 2049, 2050, 4096, 4096 + 3, 6144 - 1, 2048 * 5 + 1, 2047, 66, 67, 68, 4100])


@pytest.mark.parametrize("kappa,W,D", [(5, 10, 20), (1, 10, 20), (3, 64, 64), (64, 5, 20)])
def test_scan_planted_many_contexts(kappa, W, D):
    print(f"[case] scan planted, many contexts, kappa={kappa} W={W} D={D} B={len(MANY)}", flush=True)
    ids, cu = scan_ids_planted(MANY, kappa=kappa, seed=4400 + kappa, boundary=2048)
    g = cdv.kgram_retrieve(up(ids), up(cu), kappa, W, D)
    torch.cuda.synchronize()
    ko = oracle.kgram_retrieve(ids, cu, kappa, W, D)
    _compare(g, ko, f"many kappa={kappa}")
    print(f"[ok] contexts with a match {int((ko['n_match'] > 0).sum())}, "
          f"with W {int((ko['n_match'] >= W).sum())}", flush=True)


def test_scan_small_vocabulary_many_matches():
    # vocabulary of 3: every chunk holds many matches, W of them are kept
    rng = np.random.default_rng(4200)
    ns = [30000, 17, 8200, 16400]
    ids = np.concatenate([rng.integers(0, 3, n).astype(np.int32) for n in ns])
    cu = np.zeros(len(ns) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ns)
    for kappa, W in ((5, 10), (12, 64), (1, 64)):
        print(f"[case] scan vocab 3 kappa={kappa} W={W}", flush=True)
        g = cdv.kgram_retrieve(up(ids), up(cu), kappa, W, 20)
        torch.cuda.synchronize()
        _compare(g, oracle.kgram_retrieve(ids, cu, kappa, W, 20), f"vocab3 kappa={kappa}")


def test_scan_full_size_sampled():
    # the largest scan launch (2^28 ids, 16384 contexts of 16384), as timed; the
    # anchor's kappa-gram is copied into 24 sampled contexts at chosen depths
    total = SCAN_SIZES[-1]
    print(f"[case] scan full size total={total} n={SCAN_N}", flush=True)
    ids, cu = scan_ids_device(total, device="cuda")
    B = cu.numel() - 1
    rng = np.random.default_rng(4300)
    sample = rng.choice(B, 64, replace=False)
    kappa, W, D = 5, 10, 20
    for i, b in enumerate(sample[:24].tolist()):
        base = b * SCAN_N
        suffix = ids[base + SCAN_N - kappa:base + SCAN_N].clone()
        for p in rng.choice(np.arange(kappa - 1, SCAN_N - 1 - kappa), int(rng.integers(1, 14)),
                            replace=False).tolist():
            ids[base + p - kappa + 1:base + p + 1] = suffix
    g = cdv.kgram_retrieve(ids, cu, kappa, W, D)
    torch.cuda.synchronize()
    nm = host(g["n_match"])
    assert nm.min() >= 0 and nm.max() <= W
    for b in sample.tolist():
        x = host(ids[b * SCAN_N:(b + 1) * SCAN_N])
        ko = oracle.kgram_retrieve(x, np.array([0, SCAN_N], dtype=np.int32), kappa, W, D)
        for k in KEYS:
            got = host(g[k][b:b + 1])
            exp = ko[k].astype(got.dtype) if k == "copy_gate" else ko[k]
            assert np.array_equal(got, exp), f"context {b}: {k}"
    print(f"[ok] sampled 64 of {B}; planted M={nm[sample[:24]].tolist()}; "
          f"contexts with a match: {int((nm > 0).sum())}", flush=True)
