"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the same
seeded inputs.  Bars are stated in parity_lib.  Every test prints the case it runs
before touching the GPU."""
import numpy as np
import pytest
import torch

import copy_draft_verification_amd as cdv
import oracle
from parity_lib import (DEV, Dev, check_accept, check_kgram, check_probe, check_verify, host,
                        up)
from workloads import generate, generate_with_ids, spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cdv.load()


def _chain(wl, rows_att=None, rows_lm=None, logits=True):
    print(f"[case] {wl.spec.name} B={wl.spec.B} n={np.diff(wl.cu_len).tolist()[:8]} "
          f"V={wl.spec.V} dtype={wl.spec.dtype} lm_std={wl.spec.lm_std} q_scale={wl.spec.q_scale}",
          flush=True)
    d = Dev(wl)
    fire_dev, po, ties = check_probe(wl, d)
    fire_host = host(fire_dev).astype(bool)
    g, ko = check_kgram(wl, d, fire_dev, fire_host)
    attn, am, st = check_verify(wl, d, g, rows_att=rows_att, rows_lm=rows_lm, logits=logits)
    check_accept(wl, g, am)
    st.update(ties=ties, gates=int(ko["copy_gate"].sum()), M=ko["n_match"].tolist()[:8])
    print(f"[ok] {wl.spec.name} {st}", flush=True)
    return st


# ------------------------------------------------------------------ small shapes, every row
def test_tiny_fp32_chain():
    st = _chain(generate("tiny"))
    assert st["gates"] == 1 and st["M"] == [3]


@pytest.mark.parametrize("variant", [{}, {"lm_std": 1.0}, {"q_scale": 4.0}])
def test_small_bf16_chain(variant):
    st = _chain(generate("small_bf16", **variant))
    if variant.get("lm_std") == 1.0:
        assert st["margin_excluded"] <= 0.1 * st["argmax_rows"]


@pytest.mark.parametrize("variant", [{}, {"lm_std": 1.0}, {"q_scale": 4.0, "Hq": 4, "Hkv": 2, "hid": 256},
                                     {"d": 128, "hid": 256, "lm_std": 1.0}])  # d = 128: two elements per lane
def test_small_fp32_chain(variant):
    _chain(generate("small_f32", **variant))


@pytest.mark.parametrize("W,D", [(3, 7), (16, 5), (1, 64), (64, 1), (12, 33)])
def test_bf16_chain_other_candidate_shapes(W, D):
    # the candidate mask is evaluated in registers from W, D and the row index, and
    # the candidate keys form blocks of 64 that W*D need not fill
    st = _chain(generate("small_bf16", W=W, D=D, lm_std=1.0, q_scale=4.0))
    assert st["att_rows"] > 0


def test_bf16_chain_many_key_splits():
    # one sequence whose rows fit one tile of one KV head: the 12000-token context is
    # cut into 23 key splits, 21 of which hold keys; the merge combines 21 prefix
    # partials and the candidate slot, which comes last (24 slots: the merge's first
    # round of eight slot outputs and two more rounds)
    st = _chain(generate("small_bf16", B=1, n=(12000, 12000), W=1, D=20, lm_std=1.0, q_scale=4.0))
    assert st["att_rows"] > 0


@pytest.mark.parametrize("W,D", [(3, 7), (64, 1)])
def test_f32_chain_other_candidate_shapes(W, D):
    _chain(generate("small_f32", W=W, D=D, lm_std=1.0))


def test_small_natural_anchors():
    # natural anchor mode: gates open and close by the data; short accidental repeats
    _chain(generate("small_bf16", anchor="natural", B=6, seed=2101, lm_std=1.0))


# ------------------------------------------------------------------ edge cases
def test_edge_contexts_bf16():
    rng = np.random.default_rng(7)
    ids = [
        [1, 2, 3],                                   # n <= kappa: no match
        [5] * 40,                                    # constant: L = 1..W
        list(range(300)),                            # all distinct: no match
        ([1, 2, 3, 4, 5, 6, 7] * 30)[:205],          # periodic, ragged
        list(rng.integers(0, 3, 517)),               # tiny vocabulary: many matches
        [9] * 6,                                     # n = kappa + 1
    ]
    wl = generate_with_ids(spec("small_bf16", lm_std=1.0), ids)
    _chain(wl)


def test_edge_contexts_fp32_probe_closed():
    ids = [[4, 4, 4, 4, 4, 4, 4, 4], list(range(50)) + list(range(45, 50))]
    wl = generate_with_ids(spec("small_f32"), ids, anchor_copy=[False, True])
    d = Dev(wl)
    # force the first probe shut and the second open, whatever the scores
    fire = torch.tensor([0, 1], dtype=torch.uint8, device=DEV)
    g, ko = check_kgram(wl, d, fire, np.array([False, True]))
    assert ko["n_match"].tolist() == [0, 1]
    attn, am, st = check_verify(wl, d, g)
    a, ao = check_accept(wl, g, am)
    assert ao["best_w"].tolist()[0] == -1 and ao["next_token"].tolist()[0] == -1
    assert np.all(host(am)[0] == -1) and torch.all(attn[0] == 0)


def test_all_gates_closed():
    wl = generate("small_bf16")
    d = Dev(wl)
    fire = torch.zeros(wl.spec.B, dtype=torch.uint8, device=DEV)
    g, ko = check_kgram(wl, d, fire, np.zeros(wl.spec.B, dtype=bool))
    attn, am, st = check_verify(wl, d, g)
    assert st["att_rows"] == 0 and torch.all(am == -1)
    check_accept(wl, g, am)


def _pack_host(w, K):
    """The packed weight layout from its definition: 16-byte chunk
    c = (((t*K/64 + s)*4 + wv)*8 + 4a + j)*64 + 32h + l holds row 256t + 64wv + 32a + l,
    columns 64s + 16j + 8h .. +7; rows past the end are zero."""
    N = w.shape[0]
    T = -(-N // 256)
    wp = np.zeros((T * 256, K), dtype=np.uint16)
    wp[:N] = w
    x = wp.reshape(T, 4, 2, 32, K // 64, 4, 2, 8)        # t, wv, a, l | s, j, h, e
    return x.transpose(0, 4, 1, 2, 5, 6, 3, 7).reshape(-1)


def _pair_rows_host(gate, up):
    """The gate / up pair as the rows of one matrix: row 256t + 64wv + 32a + l is
    feature 128t + 32wv + l of the gate (a = 0) or of the up matrix (a = 1)."""
    inter, K = gate.shape
    T = -(-inter // 128)
    g = np.zeros((T * 128, K), dtype=np.uint16)
    u = np.zeros((T * 128, K), dtype=np.uint16)
    g[:inter], u[:inter] = gate, up
    out = np.stack([g.reshape(T, 4, 32, K), u.reshape(T, 4, 32, K)], axis=2)   # t, wv, a, l
    return out.reshape(T * 256, K)


def _bits(rng, shape):
    bits = rng.integers(0, 1 << 16, shape, dtype=np.uint16)
    return bits, torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("N,K", [(1000, 512), (256, 1024), (513, 256)])
def test_pack_weight_layout_bitwise(N, K):
    print(f"[case] pack_weight N={N} K={K}", flush=True)
    bits, w = _bits(np.random.default_rng(N + K), (N, K))
    packed = cdv.pack_weight(w)
    torch.cuda.synchronize()
    got = packed.data.cpu().numpy().view(np.uint16)
    assert got.size == -(-N // 256) * 256 * K
    assert np.array_equal(got, _pack_host(bits, K))


@pytest.mark.parametrize("inter,K", [(1024, 256), (300, 512), (128, 768)])
def test_pack_gate_up_layout_bitwise(inter, K):
    print(f"[case] pack_gate_up inter={inter} K={K}", flush=True)
    rng = np.random.default_rng(inter * 7 + K)
    gbits, g = _bits(rng, (inter, K))
    ubits, u = _bits(rng, (inter, K))
    packed = cdv.pack_gate_up(g, u)
    torch.cuda.synchronize()
    got = packed.data.cpu().numpy().view(np.uint16)
    assert got.size == -(-inter // 128) * 256 * K
    assert np.array_equal(got, _pack_host(_pair_rows_host(gbits, ubits), K))


@pytest.mark.parametrize("name,over", [
    ("small_bf16", {"lm_std": 1.0}),                              # V = 3001: a partial last tile
    ("small_bf16", {"B": 32, "n": (200, 400), "seed": 2203, "lm_std": 1.0}),  # several row chunks
    ("llama8b_b1", {"lm_std": 1.0}),
])
def test_row_major_bf16_lm_head_matches_packed(name, over):
    # SSD_BF16_ROWS: the plain [V, hid] matrix gives the packed layout's results bit for
    # bit (the same MFMA operands reach every lane, only the load addressing differs)
    wl = generate(name, **over)
    s = wl.spec
    print(f"[case] row-major LM head, {name} {over}", flush=True)
    d = Dev(wl)
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D)
    plain = up(wl.lm_head)
    assert plain.dtype == torch.bfloat16 and not isinstance(plain, cdv.PackedWeight)
    logits = s.V <= 10000
    outs = []
    for lm in (d.lm, plain):
        L = torch.empty(s.B, wl.R, s.V, dtype=torch.float32, device=DEV) if logits else None
        a, m = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                   g["copy_gate"], lm, s.W, s.D, wl.scale, logits_out=L)
        a2, m2, acc = cdv.blocktri_verify_accept(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc,
                                                 g["cand"], g["cand_len"], g["copy_gate"], lm,
                                                 s.W, s.D, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(m, m2)
        outs.append((m, L, acc))
    assert torch.equal(outs[0][0], outs[1][0])
    if logits:
        real = host(outs[0][0]) >= 0
        assert np.array_equal(host(outs[0][1])[real], host(outs[1][1])[real])
    for k in outs[0][2]:
        assert torch.equal(outs[0][2][k], outs[1][2][k]), k
    print(f"[ok] argmax equal on {int((host(outs[0][0]) >= 0).sum())} real rows", flush=True)


def test_row_major_bf16_lm_head_is_refused_by_sampling():
    wl = generate("small_bf16")
    d = Dev(wl)
    g = cdv.kgram_retrieve(d.ids, d.cu, wl.spec.kappa, wl.spec.W, wl.spec.D)
    with pytest.raises(cdv.SwitchSDError, match="packed"):
        cdv.blocktri_verify_sample(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand"],
                                   g["cand_len"], g["copy_gate"], up(wl.lm_head), wl.spec.W,
                                   wl.spec.D, wl.scale, 1.0, 7)


def _nan_tail(t, extra_rows):
    """t [rows, ...] copied into the head of a longer buffer whose tail is NaN; returns
    the view of the head (same shape, same values, NaN right after its end)."""
    big = torch.full((t.shape[0] + extra_rows, *t.shape[1:]), float("nan"), dtype=t.dtype,
                     device=t.device)
    big[: t.shape[0]] = t
    return big[: t.shape[0]]


@pytest.mark.parametrize("name", ["small_bf16", "small_f32"])
def test_keys_past_the_end_are_never_read(name):
    # The last sequence's context and the last candidate block end inside a 64-key
    # block (n and W*D = 200 are not multiples of 64).  NaN right after the caches
    # and the candidate keys would reach the output through 0 * NaN if the kernel
    # read past the last key instead of taking zeros.
    wl = generate(name, lm_std=1.0)
    n_last = int(wl.cu_len[-1] - wl.cu_len[-2])
    print(f"[case] {name} NaN past the caches, n_last={n_last}", flush=True)
    assert n_last % 64 != 0 and (wl.spec.W * wl.spec.D) % 64 != 0
    d = Dev(wl)
    d.kp, d.vp = _nan_tail(d.kp, 128), _nan_tail(d.vp, 128)
    B, WD = wl.spec.B, wl.spec.W * wl.spec.D
    d.kc = _nan_tail(d.kc.reshape(B * WD, *d.kc.shape[2:]), 128).reshape(d.kc.shape)
    d.vc = _nan_tail(d.vc.reshape(B * WD, *d.vc.shape[2:]), 128).reshape(d.vc.shape)
    fire = torch.ones(B, dtype=torch.uint8, device=DEV)
    g, ko = check_kgram(wl, d, fire, np.ones(B, dtype=bool))
    assert bool(ko["copy_gate"][-1])
    attn, am, st = check_verify(wl, d, g)
    assert torch.isfinite(attn.float()).all()
    assert st["att_rows"] > 0


@pytest.mark.parametrize("W,D,kappa", [(3, 7, 2), (1, 1, 1), (64, 64, 5), (10, 20, 64)])
def test_kgram_accept_other_limits(W, D, kappa):
    rng = np.random.default_rng(W * 100 + D)
    ids = [list(rng.integers(0, 4, int(rng.integers(1, 400)))) for _ in range(5)]
    ids.append([7] * 150)
    wl = generate_with_ids(spec("small_f32", W=W, D=D), ids)
    print(f"[case] kgram W={W} D={D} kappa={kappa}", flush=True)
    d = Dev(wl, tensors=False)
    g, ko = check_kgram(wl, d, None, None, W=W, D=D, kappa=kappa)
    # accept on planted predictions that follow the candidates for a random length
    B, R = len(ids), 1 + W * D
    am = rng.integers(0, 4, (B, R)).astype(np.int32)
    cand, cl = ko["cand"], ko["cand_len"]
    for b in range(B):
        if ko["n_match"][b]:
            am[b, 0] = cand[b, 0, 0]
        for w in range(W):
            stop = int(rng.integers(0, D + 1))
            for j in range(min(stop, D - 1)):
                if cand[b, w, j + 1] >= 0:
                    am[b, 1 + w * D + j] = cand[b, w, j + 1]
    check_accept(wl, g, up(am), W=W, D=D)


def test_kgram_long_context_matches_far_back():
    # 3 chunks of scanning before the first (and only) earlier occurrence at p = 104
    n = 20000
    x = list(range(1000, 1000 + n))
    x[100:105] = x[n - 5:]
    wl = generate_with_ids(spec("small_f32"), [x, x[:9000] + x[n - 5:]])
    print("[case] kgram long context", flush=True)
    d = Dev(wl, tensors=False)
    g, ko = check_kgram(wl, d, None, None)
    assert ko["match_end"][0, 0] == 104 and ko["n_match"][0] == 1


def test_accept_planted_agreements():
    wl = generate("small_bf16")
    s = wl.spec
    d = Dev(wl, tensors=False)
    g, ko = check_kgram(wl, d, None, None)
    rng = np.random.default_rng(3)
    R = wl.R
    for trial in range(20):
        am = rng.integers(0, 50, (s.B, R)).astype(np.int32)
        for b in range(s.B):
            am[b, 0] = ko["cand"][b, rng.integers(0, s.W), 0]
            for w in range(s.W):
                stop = int(rng.integers(0, s.D + 1))
                for j in range(min(stop, s.D - 1)):
                    am[b, 1 + w * s.D + j] = ko["cand"][b, w, j + 1]
        a, ao = check_accept(wl, g, up(am))
    assert ao["best_len"].max() > 0


# ------------------------------------------------------------------ metamorphic
def test_candidate_isolation_bitwise():
    wl = generate("small_bf16", lm_std=1.0)
    s = wl.spec
    d = Dev(wl)
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, None)
    a0, m0 = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                 g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    a0, m0 = a0.clone(), m0.clone()
    wbad = 3
    kc2, vc2 = d.kc.clone(), d.vc.clone()
    kc2[:, wbad * s.D:(wbad + 1) * s.D] += 1.0
    vc2[:, wbad * s.D:(wbad + 1) * s.D] *= -2.0
    a1, m1 = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, kc2, vc2, g["cand_len"],
                                 g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    torch.cuda.synchronize()
    rows = [r for r in range(wl.R) if r == 0 or (r - 1) // s.D != wbad]
    assert torch.equal(a0[:, rows], a1[:, rows]) and torch.equal(m0[:, rows], m1[:, rows])
    bad = [1 + wbad * s.D + j for j in range(s.D)]
    assert not torch.equal(a0[:, bad], a1[:, bad])


def test_runs_are_deterministic():
    wl = generate("small_bf16", B=2)
    s = wl.spec
    d = Dev(wl)
    outs = []
    for _ in range(2):
        z, f = cdv.probe_score(d.h, d.w, s.tau)
        g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, f)
        a, m = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                   g["copy_gate"], d.lm, s.W, s.D, wl.scale)
        acc = cdv.accept_longest(g["cand"], g["cand_len"], g["copy_gate"], m, s.W, s.D)
        torch.cuda.synchronize()
        outs.append([z.clone(), a.clone(), m.clone()] + [v.clone() for v in g.values()]
                    + [v.clone() for v in acc.values()])
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_max_n_only_sizes_the_launch():
    # an under-estimated max_n must not change results (the last split runs to n_b)
    wl = generate("small_bf16", lm_std=1.0)
    s = wl.spec
    d = Dev(wl)
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, None)
    outs = []
    # 32 * max_n gives 22 key splits, most of them past every context: the merge skips
    # the slots past each context (it counts the splits from n_b) and still reads the
    # candidate slot, the last one, in its third round of eight slot outputs
    for mn in (wl.max_n, 64, 4 * wl.max_n, 32 * wl.max_n):
        a, m = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, mn, d.kc, d.vc, g["cand_len"],
                                   g["copy_gate"], d.lm, s.W, s.D, wl.scale)
        torch.cuda.synchronize()
        outs.append((widen(a), host(m)))
    for a, m in outs[1:]:
        assert np.max(np.abs(a - outs[0][0])) <= 2e-2
        agree = np.mean(m == outs[0][1])
        assert agree > 0.97


def widen(t):
    from parity_lib import widen_out
    return widen_out(t)


# ------------------------------------------------------------------ full sizes
def _sample_rows(wl, k, seed):
    rng = np.random.default_rng(seed)
    rows = [(b, 0) for b in range(wl.spec.B)]
    rows += [(int(rng.integers(0, wl.spec.B)), int(rng.integers(1, wl.R))) for _ in range(k)]
    return rows


def test_full_llama8b_b1_every_row():
    _chain(generate("llama8b_b1"), logits=False)


def test_full_llama8b_b1_wide_head_every_row():
    st = _chain(generate("llama8b_b1", lm_std=1.0), logits=True)
    assert st["margin_excluded"] <= 0.1 * st["argmax_rows"]


def test_full_llama8b_b1_peaked_every_row():
    # queries x4: each row's softmax concentrates on a few keys and |O| is of order 1,
    # so the 2e-2 bar sees a leaked or dropped candidate key.  Every row of the 8B
    # shape: g = 4 packed heads, 7 row tiles, the prefix split over several key slots
    wl = generate("llama8b_b1", q_scale=4.0, lm_std=1.0)
    st = _chain(wl, rows_lm=_sample_rows(wl, 24, 3), logits=False)
    assert st["att_rows"] == wl.R and st["err_att"] <= 2e-2


def test_full_llama70b_peaked_one_sequence():
    # the 70B share's tiling (g = 8, 13 row tiles of packed heads) over one 32768-token
    # context, peaked queries, every row
    wl = generate("llama70b_b4", B=1, q_scale=4.0, lm_std=1.0)
    st = _chain(wl, rows_lm=_sample_rows(wl, 12, 4), logits=False)
    assert st["att_rows"] == wl.R


@pytest.mark.parametrize("name,over", [("llama8b_b32", {}), ("llama8b_b32", {"anchor": "natural"}),
                                       ("qwen3_8b_b8", {}), ("llama70b_b4", {"lm_std": 1.0})])
def test_full_configs_sampled(name, over):
    wl = generate(name, **over)
    _chain(wl, rows_att=_sample_rows(wl, 24, 1), rows_lm=_sample_rows(wl, 12, 2), logits=False)


def test_lm_events_time_the_contraction():
    # events handed to blocktri_verify bracket the LM-head kernel; results are unchanged
    wl = generate("small_bf16", lm_std=1.0)
    s = wl.spec
    d = Dev(wl)
    print(f"[case] lm events {s.name} B={s.B}", flush=True)
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, None)
    a0, m0 = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                 g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    a0, m0 = a0.clone(), m0.clone()
    fresh = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    with pytest.raises(cdv.SwitchSDError):
        cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                            g["copy_gate"], d.lm, s.W, s.D, wl.scale, events=fresh)
    for e in fresh:
        e.record()
    a1, m1 = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                 g["copy_gate"], d.lm, s.W, s.D, wl.scale, events=fresh)
    torch.cuda.synchronize()
    assert fresh[0].elapsed_time(fresh[1]) > 0.0
    assert torch.equal(a0, a1) and torch.equal(m0, m1)


@pytest.mark.parametrize("name,over", [("tiny", {}), ("small_bf16", {}),
                                       ("small_bf16", {"anchor": "natural", "B": 6, "seed": 2101}),
                                       ("llama8b_b1", {})])
def test_commit_accepted_bitwise(name, over):
    # commit after a device chain: cache rows and context tokens equal the oracle's
    # copy of the same accept outputs, bit for bit; one sequence does not fit
    wl = generate(name, **over)
    s = wl.spec
    print(f"[case] commit {s.name} B={s.B} W={s.W} D={s.D}", flush=True)
    d = Dev(wl)
    z, fire = cdv.probe_score(d.h, d.w, s.tau)
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, fire)
    attn, am = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                   g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    acc = cdv.accept_longest(g["cand"], g["cand_len"], g["copy_gate"], am, s.W, s.D)
    torch.cuda.synchronize()
    B, D = s.B, s.D
    rows = int(wl.cu_len[-1]) + B * D
    off = np.array([int(wl.cu_len[b + 1]) + b * D for b in range(B)], dtype=np.int64)
    bl = host(acc["best_len"])
    if B > 1 and bl[-1] > 1:
        off[-1] = rows - 1          # needs best_len rows: does not fit
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    k_cache = torch.randn(rows, s.Hkv, s.d, device=DEV, generator=gen).to(d.kc.dtype)
    v_cache = torch.randn(rows, s.Hkv, s.d, device=DEV, generator=gen).to(d.kc.dtype)
    raw = (lambda t: host(t.view(torch.int16)).view(np.uint16)) if d.kc.dtype == torch.bfloat16 \
        else host
    kc_ref, vc_ref = raw(k_cache).copy(), raw(v_cache).copy()
    out = cdv.commit_accepted(d.kc, d.vc, g["cand"], acc["best_w"], acc["best_len"],
                              acc["next_token"], s.W, D, k_cache, v_cache, up(off))
    torch.cuda.synchronize()
    tok, nt = oracle.commit_accepted(raw(d.kc), raw(d.vc), host(g["cand"]), host(acc["best_w"]),
                                     bl, host(acc["next_token"]), s.W, D, kc_ref, vc_ref, off)
    assert np.array_equal(host(out["tokens"]), tok)
    assert np.array_equal(host(out["n_tokens"]), nt)
    assert np.array_equal(raw(k_cache), kc_ref) and np.array_equal(raw(v_cache), vc_ref)
    print(f"[ok] commit n_tokens={nt.tolist()[:8]}", flush=True)
