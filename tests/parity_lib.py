"""Helpers for GPU-vs-oracle parity: run each stage of the HIP path through the C ABI
and compare it with the oracle on the same seeded inputs.

Bars (stated once, used everywhere):
* probe decision, match positions, candidates, candidate lengths, gate, accept
  lengths, best candidate, next token: bit-exact.  A probe decision whose
  oracle score lies within 1e-5 * sum|w_k h_k| of the threshold is a tie-zone
  case (float32 vs float64 rounding can flip it) and is counted, not compared.
* probe score z: |z_gpu - z| <= 1e-5 * sum|w_k h_k|.
* attention output: |O_gpu - O| <= 1e-5 (float32 inputs), 2e-2 (bfloat16), and,
  relative to the largest reference output of the case, max|O_gpu - O| / max|O|
  <= 1e-4 (float32), 2e-2 (bfloat16).  Under N(0,1) queries and keys |O| shrinks
  like sqrt(e/n), so at long contexts the absolute bar alone would pass a mask
  error; the relative bar and the peaked-query cases (queries x4, softmax
  concentrated on a few keys, |O| of order 1) do not.
* logits: |l_gpu - l| <= 5e-2.
* argmax: equal wherever the oracle's top-2 margin is >= 1e-2; rows below that
  margin are counted as margin-excluded.
"""
import numpy as np
import torch

import copy_draft_verification_amd as cdv
import oracle
from oracle.attention import real_rows
from workloads import to_torch

DEV = "cuda:0"
TOL_ATT = {"f32": 1e-5, "bf16": 2e-2}
REL_ATT = {"f32": 1e-4, "bf16": 2e-2}
TOL_LOGIT = 5e-2
ARGMAX_MARGIN = 1e-2
PROBE_TIE = 1e-5


def up(a):
    return to_torch(a, DEV)


def host(t):
    return t.detach().cpu().numpy()


def widen_out(t):
    """GPU attention output -> float64 numpy with the exact stored values."""
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.detach().cpu().view(torch.int16).numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


class Dev:
    """Device copies of one workload."""

    def __init__(self, wl, tensors=True):
        self.wl = wl
        self.ids, self.cu = up(wl.ids), up(wl.cu_len)
        self.h, self.w = up(wl.h), up(wl.w)
        if tensors:
            self.q, self.kp, self.vp = up(wl.q), up(wl.k_pre), up(wl.v_pre)
            self.kc, self.vc = up(wl.k_cand), up(wl.v_cand)
            # the bf16 calls read the LM head packed (once, as at model load)
            lm = up(wl.lm_head)
            self.lm = cdv.pack_weight(lm) if lm.dtype == torch.bfloat16 else lm


def check_probe(wl, d):
    s = wl.spec
    z, fire = cdv.probe_score(d.h, d.w, s.tau)
    torch.cuda.synchronize()
    o = oracle.probe_score(wl.h, wl.w, s.tau)
    zz, ff = host(z).astype(np.float64), host(fire).astype(bool)
    tie = np.abs(o["margin"]) < PROBE_TIE * o["S"]
    assert np.all(np.abs(zz - o["z"]) <= PROBE_TIE * o["S"]), (zz, o["z"])
    assert np.array_equal(ff[~tie], o["fire"][~tie])
    return fire, o, int(tie.sum())


def check_kgram(wl, d, fire_dev, fire_host, W=None, D=None, kappa=None):
    s = wl.spec
    W, D, kappa = W or s.W, D or s.D, kappa or s.kappa
    g = cdv.kgram_retrieve(d.ids, d.cu, kappa, W, D, fire_dev)
    torch.cuda.synchronize()
    o = oracle.kgram_retrieve(wl.ids, wl.cu_len, kappa, W, D, fire_host)
    for k in ("match_end", "n_match", "cand", "cand_len"):
        assert np.array_equal(host(g[k]), o[k]), k
    assert np.array_equal(host(g["copy_gate"]).astype(bool), o["copy_gate"])
    return g, o


def check_verify(wl, d, g, rows_att=None, rows_lm=None, logits=True, events=None):
    """Run blocktri_verify on the device retrieval outputs; compare with the oracle.

    rows_att / rows_lm: None = every real row; else lists of (b, r) to sample.
    Returns (attn_out, argmax, stats)."""
    s = wl.spec
    B, R, V = s.B, wl.R, s.V
    logits_out = torch.empty(B, R, V, dtype=torch.float32, device=DEV) if logits else None
    attn, am = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                   g["copy_gate"], d.lm, s.W, s.D, wl.scale,
                                   logits_out=logits_out, events=events)
    torch.cuda.synchronize()
    cand_len, gate = host(g["cand_len"]), host(g["copy_gate"]).astype(bool)
    real = {(b, r) for b in range(B) for r in real_rows(cand_len[b], gate[b], s.W, s.D)}
    O = widen_out(attn).reshape(B, R, s.Hq * s.d)
    amh = host(am)
    # rows that are not real: zero output, argmax -1
    for b in range(B):
        for r in range(R):
            if (b, r) not in real:
                assert amh[b, r] == -1
    unreal = np.ones((B, R), dtype=bool)
    for (b, r) in real:
        unreal[b, r] = False
    assert np.all(O[unreal] == 0.0)
    # attention
    ref, ev = oracle.blocktri_attention(wl.q, wl.k_pre, wl.v_pre, wl.cu_len, wl.k_cand, wl.v_cand,
                                        cand_len, gate, s.Hq, s.Hkv, s.d, s.W, s.D, wl.scale,
                                        rows=rows_att)
    err_att = ref_max = 0.0
    for (b, r) in ev:
        e = np.max(np.abs(O[b, r] - ref[b, r]))
        err_att = max(err_att, e)
        ref_max = max(ref_max, float(np.max(np.abs(ref[b, r]))))
    rel_att = err_att / ref_max if ref_max > 0 else 0.0
    print(f"[att] rows {len(ev)} max|O-O*| {err_att:.3e} max|O*| {ref_max:.3e} "
          f"relative {rel_att:.3e}", flush=True)
    assert err_att <= TOL_ATT[s.dtype], err_att
    assert rel_att <= REL_ATT[s.dtype], rel_att
    # LM head on the device's own attention output
    lm_rows = sorted(real) if rows_lm is None else [x for x in rows_lm if x in real]
    excluded = 0
    err_logit = 0.0
    if lm_rows:
        Osel = O[[b for b, _ in lm_rows], [r for _, r in lm_rows]]
        res = oracle.lmhead_argmax(Osel, wl.lm_head)
        got = np.array([amh[b, r] for b, r in lm_rows])
        ok = res["margin"] >= ARGMAX_MARGIN
        excluded = int((~ok).sum())
        assert np.array_equal(got[ok], res["pred"][ok]), np.nonzero(got[ok] != res["pred"][ok])
        if logits:
            L = host(logits_out)
            Lsel = L[[b for b, _ in lm_rows], [r for _, r in lm_rows]].astype(np.float64)
            err_logit = float(np.max(np.abs(Lsel - res["logits"])))
            assert err_logit <= TOL_LOGIT, err_logit
    return attn, am, {"err_att": err_att, "rel_att": rel_att, "err_logit": err_logit, "argmax_rows": len(lm_rows),
                      "margin_excluded": excluded, "att_rows": len(ev)}


def check_accept(wl, g, am, W=None, D=None):
    s = wl.spec
    W, D = W or s.W, D or s.D
    a = cdv.accept_longest(g["cand"], g["cand_len"], g["copy_gate"], am, W, D)
    torch.cuda.synchronize()
    o = oracle.accept_longest(host(g["cand"]), host(g["cand_len"]),
                              host(g["copy_gate"]).astype(bool), host(am), W, D)
    for k in ("accept_len", "best_w", "best_len", "next_token"):
        assert np.array_equal(host(a[k]), o[k]), k
    return a, o
