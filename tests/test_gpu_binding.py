"""The binding refuses outputs, workspaces and inputs whose dtype, shape or device
does not match the call, before anything is launched (a wrong buffer would become
out-of-bounds device writes).  The binding only marshals; these are its checks."""
import pytest
import torch

import copy_draft_verification_amd as cdv
from parity_lib import DEV, Dev
from workloads import generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def case():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cdv.load()
    wl = generate("small_bf16", lm_std=1.0)
    print(f"[case] binding checks on {wl.spec.name} B={wl.spec.B}", flush=True)
    d = Dev(wl)
    s = wl.spec
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, None)
    torch.cuda.synchronize()
    return wl, d, g


def _verify(wl, d, g, **kw):
    s = wl.spec
    args = dict(q=d.q, k_pre=d.kp, v_pre=d.vp, cu_len=d.cu, max_n=wl.max_n, k_cand=d.kc,
                v_cand=d.vc, cand_len=g["cand_len"], copy_gate=g["copy_gate"], lm_head=d.lm,
                W=s.W, D=s.D, scale=wl.scale)
    args.update(kw)
    return cdv.blocktri_verify(**args)


def _bad_outputs(wl):
    s = wl.spec
    B, R, V, hid = s.B, wl.R, s.V, s.Hq * s.d
    f = lambda *sh, dt: torch.empty(*sh, dtype=dt, device=DEV)  # noqa: E731
    return [
        ("attn_out", f(B, R, hid, dt=torch.float32)),            # wrong dtype
        ("attn_out", f(B, R - 1, hid, dt=torch.bfloat16)),       # short
        ("attn_out", f(B, hid, R, dt=torch.bfloat16).transpose(1, 2)),  # not contiguous
        ("attn_out", torch.empty(B, R, hid, dtype=torch.bfloat16)),     # host memory
        ("argmax_out", f(B, R, dt=torch.int64)),
        ("argmax_out", f(B, R + 1, dt=torch.int32)),
        ("logits_out", f(B, R, V, dt=torch.bfloat16)),
        ("logits_out", f(B, R, V - 1, dt=torch.float32)),
        ("workspace", f(16, dt=torch.uint8)),                    # too small
        ("workspace", f(1 << 20, dt=torch.float32)),             # not bytes
    ]


def test_verify_refuses_bad_outputs(case):
    wl, d, g = case
    for name, t in _bad_outputs(wl):
        with pytest.raises(cdv.SwitchSDError):
            _verify(wl, d, g, **{name: t})


def test_verify_refuses_bad_inputs(case):
    wl, d, g = case
    s = wl.spec
    bad = [("k_cand", d.kc[:, :-1].contiguous()),           # fewer than W*D candidate keys
           ("v_cand", d.vc[:-1].contiguous()),               # fewer sequences
           ("cand_len", g["cand_len"][:, :-1].contiguous()),
           ("cu_len", d.cu[:-1].contiguous()),
           ("copy_gate", g["copy_gate"][:-1].contiguous()),
           ("k_pre", d.kp[..., :64].contiguous()),           # head dim differs from q's
           ("v_pre", d.vp[:-1].contiguous()),                # differs from k_pre
           ("q", d.q[:, :-1].contiguous())]                  # rows != 1 + W*D
    for name, t in bad:
        with pytest.raises(cdv.SwitchSDError):
            _verify(wl, d, g, **{name: t})
    with pytest.raises(cdv.SwitchSDError):
        _verify(wl, d, g, W=s.W + 1)


def test_good_outputs_are_accepted(case):
    wl, d, g = case
    s = wl.spec
    B, R, hid = s.B, wl.R, s.Hq * s.d
    a0, m0 = _verify(wl, d, g)
    attn = torch.empty(B, R, hid, dtype=torch.bfloat16, device=DEV)
    am = torch.empty(B, R, dtype=torch.int32, device=DEV)
    a1, m1 = _verify(wl, d, g, attn_out=attn, argmax_out=am)
    torch.cuda.synchronize()
    assert a1 is attn and m1 is am
    assert torch.equal(a0, a1) and torch.equal(m0, m1)


def test_other_calls_refuse_bad_outputs(case):
    wl, d, g = case
    s = wl.spec
    B = s.B
    with pytest.raises(cdv.SwitchSDError):
        cdv.probe_score(d.h, d.w, s.tau, z_out=torch.empty(B + 1, device=DEV))
    with pytest.raises(cdv.SwitchSDError):
        cdv.probe_score(d.h, d.w[:-1].contiguous(), s.tau)
    out = {k: v.clone() for k, v in g.items()}
    out["cand"] = torch.empty(B, s.W, s.D - 1, dtype=torch.int32, device=DEV)
    with pytest.raises(cdv.SwitchSDError):
        cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, None, out=out)
    am = torch.zeros(B, wl.R, dtype=torch.int32, device=DEV)
    with pytest.raises(cdv.SwitchSDError):
        cdv.accept_longest(g["cand"], g["cand_len"], g["copy_gate"], am[:, :-1].contiguous(),
                           s.W, s.D)
    acc = {"accept_len": torch.empty(B, s.W, dtype=torch.int32, device=DEV),
           "best_w": torch.empty(B, dtype=torch.int64, device=DEV),
           "best_len": torch.empty(B, dtype=torch.int32, device=DEV),
           "next_token": torch.empty(B, dtype=torch.int32, device=DEV)}
    with pytest.raises(cdv.SwitchSDError):
        cdv.accept_longest(g["cand"], g["cand_len"], g["copy_gate"], am, s.W, s.D, out=acc)


def test_allocations_follow_the_given_stream(case):
    # with stream= and no workspace, the binding allocates on that stream; results on a
    # side stream equal those on the default stream
    wl, d, g = case
    a0, m0 = _verify(wl, d, g)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    a1, m1 = _verify(wl, d, g, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(a0, a1) and torch.equal(m0, m1)
