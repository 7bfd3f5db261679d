"""GPU parity of the offline probe calibration (copy labels, batched probe logits,
threshold / AUC sweep and layer choice) against the float64 oracle.

Bars:
* labels: bit-exact.
* probe logits: |z_gpu - z| <= (c + 7) * 2^-24 * sum_k |w_k h_k|.  Each lane runs one
  fused multiply-add chain over c products, then six shuffle adds: a recursive sum of at
  most c + 7 rounded steps, whose error is bounded by that many unit roundoffs times the
  sum of magnitudes.  A lane takes every 64th element (c = ceil(hid / 64)), or, when
  hid % 8 == 0, every 64th group of eight (c = 8 * ceil(hid / 512), e.g. 16 at hid = 520).
* sweep: run on the GPU's own fp32 scores, the oracle (float64, exact on those values)
  must give the same threshold, TP / FP / FN / P and 2U exactly, the same layer; AUC and
  tau within the rounding of a double to float.
Every test prints its case before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import copy_draft_verification_amd as cdv
import oracle
from parity_lib import DEV, host, up
from workloads import generate, generate_calibration

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cdv.load()


def _case(msg):
    print(f"[case] {msg}", flush=True)


_FULL = {}


def _full():
    """The 32-layer, 4096-position, 4096-wide bf16 calibration set (generated once)."""
    if "c" not in _FULL:
        _FULL["c"] = generate_calibration("calib_llama8b")
    return _FULL["c"]


# ------------------------------------------------------------------ labels
def _labels_gpu(ids, cu_len, n_train=5):
    lab = cdv.copy_labels(up(np.asarray(ids, np.int32)), up(np.asarray(cu_len, np.int32)), n_train)
    torch.cuda.synchronize()
    return host(lab)


def _check_labels(ids, cu_len, n_train=5):
    got = _labels_gpu(ids, cu_len, n_train)
    want = oracle.copy_labels(ids, cu_len, n_train)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} label mismatches, first at {bad[:8].tolist()}"
    return want


def _concat(lists):
    ids = np.concatenate([np.asarray(x, np.int32) for x in lists])
    cu = np.zeros(len(lists) + 1, np.int32)
    cu[1:] = np.cumsum([len(x) for x in lists])
    return ids, cu


@pytest.mark.parametrize("name", ["calib_small_bf16", "calib_small_f32", "calib_llama8b"])
def test_copy_labels_calibration_contexts(name):
    c = _full() if name == "calib_llama8b" else generate_calibration(name)
    _case(f"labels {name} B={c.spec.B} n={np.diff(c.cu_len).tolist()}")
    y = _check_labels(c.ids, c.cu_len)
    assert 0 < int(y.sum()) < len(y)


@pytest.mark.parametrize("name,over", [("tiny", {}),
                                       ("small_bf16", {"anchor": "natural", "B": 6, "seed": 2101})])
def test_copy_labels_decode_contexts(name, over):
    wl = generate(name, **over)
    _case(f"labels {name} {over} B={wl.spec.B}")
    _check_labels(wl.ids, wl.cu_len)


@pytest.mark.parametrize("n_train", [1, 2, 5, 9, 64])
def test_copy_labels_edge_contexts(n_train):
    rng = np.random.default_rng(11)
    lists = [
        [7],                                          # one token
        [3, 4, 5],                                    # shorter than most windows
        [9] * 70,                                     # constant: overlapping earlier start
        [1, 2, 3] * 30,                               # period 3
        rng.integers(0, 4, 300).tolist(),             # tiny vocabulary: many repeats
        rng.integers(0, 10 ** 6, 200).tolist(),       # no repeats at all
        [5, 6, 7, 8, 9, 1, 5, 6, 7, 8, 9],            # one repeat of a 5-run
    ]
    # a window that occurs in two contexts but only once in each is not a copy
    lists += [[40, 41, 42, 43, 44, 45], [40, 41, 42, 43, 44, 45]]
    ids, cu = _concat(lists)
    _case(f"labels edge n_train={n_train} n={np.diff(cu).tolist()}")
    y = _check_labels(ids, cu, n_train)
    if n_train == 5:
        assert y[cu[-3]:].sum() == 0


def test_copy_labels_long_context():
    # one 262144-token context: a table of 2^19 slots, many probe collisions
    c = generate_calibration("calib_small_bf16", B=1, n=(262144, 262144), V=5000, hid=8, L=1)
    _case("labels one context n=262144")
    _check_labels(c.ids, c.cu_len)


# ------------------------------------------------------------------ probe logits
def _logit_bound(H, w, dtype):
    Hd = oracle.bf16_bits_to_f64(H) if dtype == "bf16" else np.asarray(H, np.float64)
    mag = np.einsum("lnk,lk->ln", np.abs(Hd), np.abs(np.asarray(w, np.float64)))
    hid = H.shape[-1]
    chain = 8 * math.ceil(hid / 512) if hid % 8 == 0 else math.ceil(hid / 64)
    return (chain + 7) * 2.0 ** -24 * mag


def _check_logits(H, w, dtype, z_gpu):
    want = oracle.probe_logits(H, w, dtype)
    err = np.abs(z_gpu.astype(np.float64) - want)
    tol = _logit_bound(H, w, dtype)
    assert np.all(err <= tol), f"max err/tol {float(np.max(err / tol)):.3g}"
    return float(np.max(err / tol))


@pytest.mark.parametrize("name", ["calib_small_bf16", "calib_small_f32"])
def test_probe_logits_small(name):
    c = generate_calibration(name)
    _case(f"logits {name} H={c.H.shape}")
    z = host(cdv.probe_logits(up(c.H), up(c.w)))
    r = _check_logits(c.H, c.w, c.spec.dtype, z)
    print(f"[ok] max err/tol {r:.3g}", flush=True)


@pytest.mark.parametrize("hid", [1, 7, 13, 8, 520, 1000, 4096, 4104, 16384])
def test_probe_logits_odd_hidden(hid):
    # hid % 8 != 0 takes the per-element path; hid % 8 == 0 up to 4096 the one-round,
    # next-row-prefetch path (rows shorter than a round read zeros past their end);
    # 4104 and 16384 the multi-round path; 16384 fills the LDS copy of w
    c = generate_calibration("calib_small_f32", hid=hid, L=2, B=1, n=(97, 97))
    _case(f"logits hid={hid} H={c.H.shape}")
    _check_logits(c.H, c.w, "f32", host(cdv.probe_logits(up(c.H), up(c.w))))
    cb = generate_calibration("calib_small_bf16", hid=hid, L=2, B=1, n=(97, 97))
    _check_logits(cb.H, cb.w, "bf16", host(cdv.probe_logits(up(cb.H), up(cb.w))))


@pytest.mark.slow
def test_probe_logits_full_size_sampled():
    c = _full()
    _case(f"logits calib_llama8b H={c.H.shape} (sampled)")
    z = host(cdv.probe_logits(up(c.H), up(c.w)))
    rng = np.random.default_rng(5)
    L, N, _ = c.H.shape
    for l, i in zip(rng.integers(0, L, 256), rng.integers(0, N, 256)):
        _check_logits(c.H[l:l + 1, i:i + 1], c.w[l:l + 1], "bf16", z[l:l + 1, i:i + 1])
    # the last row of the last layer and the first of the first
    _check_logits(c.H[-1:, -1:], c.w[-1:], "bf16", z[-1:, -1:])
    _check_logits(c.H[:1, :1], c.w[:1], "bf16", z[:1, :1])


# ------------------------------------------------------------------ sweep
def _check_sweep(z, y):
    """z [L, N] float32 (host), y [N] uint8: GPU calibrate vs the oracle on the same z."""
    z = np.ascontiguousarray(z, np.float32)
    out = cdv.calibrate(up(z), up(np.asarray(y, np.uint8)))
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in out.items()}
    want = oracle.calibrate(z.astype(np.float64), y)
    for l, p in enumerate(want["per_layer"]):
        tag = f"layer {l}"
        assert got["thr"][l] == p["t"] or (math.isinf(p["t"]) and math.isinf(got["thr"][l])), tag
        assert got["counts"][l].tolist() == [p["tp"], p["fp"], p["fn"], p["pos"]], tag
        assert int(got["u2"][l]) == p["u2"], tag
        if math.isnan(p["auc"]):
            assert math.isnan(got["auc"][l]), tag
        else:
            assert abs(got["auc"][l] - p["auc"]) <= 2.0 ** -23 * p["auc"] + 1e-30, tag
    assert int(got["best_layer"][0]) == want["layer"]
    assert abs(float(got["tau"][0]) - want["tau"]) <= 2.0 ** -23 * want["tau"]
    return want


@pytest.mark.parametrize("name", ["calib_small_bf16", "calib_small_f32"])
def test_calibrate_chain_small(name):
    c = generate_calibration(name)
    _case(f"calibrate chain {name}")
    yd = cdv.copy_labels(up(c.ids), up(c.cu_len))
    zd = cdv.probe_logits(up(c.H), up(c.w))
    torch.cuda.synchronize()
    y = host(yd)
    assert np.array_equal(y, oracle.copy_labels(c.ids, c.cu_len))
    _check_logits(c.H, c.w, c.spec.dtype, host(zd))
    want = _check_sweep(host(zd), y)
    print(f"[ok] layer {want['layer']} tau {want['tau']:.4f} "
          f"f1 {want['per_layer'][want['layer']]['f1']:.4f}", flush=True)


def _rand_labels(rng, n, p):
    return (rng.random(n) < p).astype(np.uint8)


@pytest.mark.parametrize("N,L,levels", [(1, 1, 0), (2, 2, 0), (777, 3, 0), (1500, 2, 0), (3000, 2, 40), (8192, 2, 0),
                                        (8193, 2, 0), (20000, 2, 0), (20000, 2, 300),
                                        (5000, 4, 3)])
def test_calibrate_sweep_shapes(N, L, levels):
    # levels > 0: scores on a grid of that many values, so groups of equal scores span
    # threads, chunks of the scan and the sort's LDS chunks
    rng = np.random.default_rng(N * 31 + L)
    _case(f"sweep N={N} L={L} levels={levels}")
    y = _rand_labels(rng, N, 0.2)
    z = rng.standard_normal((L, N)).astype(np.float32) + 1.5 * y
    if levels:
        z = np.round(z * levels / 8) / (levels / 8)
    _check_sweep(z.astype(np.float32), y)


def test_calibrate_sweep_degenerate():
    rng = np.random.default_rng(3)
    N = 1000
    _case("sweep degenerate: no positives / all positives / one score / signed zeros")
    z = rng.standard_normal((2, N)).astype(np.float32)
    _check_sweep(z, np.zeros(N, np.uint8))                 # t = +inf, AUC undefined
    _check_sweep(z, np.ones(N, np.uint8))                  # lowest threshold, AUC undefined
    _check_sweep(np.full((2, N), 0.25, np.float32), _rand_labels(rng, N, 0.3))
    zz = np.where(rng.random((2, N)) < 0.5, -0.0, 0.0).astype(np.float32)
    zz[:, :100] = 1.0
    _check_sweep(zz, _rand_labels(rng, N, 0.3))            # -0 and +0 are one threshold
    big = rng.choice(np.array([-3e38, 3e38, -1e-45, 1e-45, 0.0], np.float32), (2, N))
    _check_sweep(big, _rand_labels(rng, N, 0.5))           # extremes and subnormals


def test_calibrate_layer_tie_keeps_lowest():
    rng = np.random.default_rng(9)
    N = 3000
    _case("sweep identical layers")
    y = _rand_labels(rng, N, 0.25)
    z1 = (rng.standard_normal(N) + 2 * y).astype(np.float32)
    z = np.stack([z1 * 0.0 - 1.0, z1, z1, z1])               # layer 0 weak, 1..3 identical
    want = _check_sweep(z, y)
    assert want["layer"] == 1


@pytest.mark.slow
def test_calibrate_full_size():
    c = _full()
    _case(f"calibrate calib_llama8b L={c.spec.L} N={c.H.shape[1]}")
    yd = cdv.copy_labels(up(c.ids), up(c.cu_len))
    zd = cdv.probe_logits(up(c.H), up(c.w))
    torch.cuda.synchronize()
    y = host(yd)
    assert np.array_equal(y, oracle.copy_labels(c.ids, c.cu_len))
    want = _check_sweep(host(zd), y)
    print(f"[ok] layer {want['layer']} tau {want['tau']:.4f}", flush=True)
