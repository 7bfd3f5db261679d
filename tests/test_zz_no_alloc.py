"""The no-allocation verification entry point (ssd_blocktri_verify_noalloc) against
ssd_blocktri_verify on the same inputs, through the C ABI: attention output and
argmax equal bit for bit (the same kernels run on the same inputs), on two calls in
a row, the second with a smaller input (the library's scratch keeps the first
call's contents), and a call whose partials exceed the scratch is refused."""
import numpy as np
import pytest
import torch

import copy_draft_verification_amd as cdv
from parity_lib import DEV, Dev
from workloads import generate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    cdv.load()


def _both(wl):
    s = wl.spec
    d = Dev(wl)
    g = cdv.kgram_retrieve(d.ids, d.cu, s.kappa, s.W, s.D, None)
    a0, m0 = cdv.blocktri_verify(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                 g["copy_gate"], d.lm, s.W, s.D, wl.scale)
    attn = torch.full_like(a0, float("nan"))
    am = torch.full_like(m0, -7)
    cdv.blocktri_verify_noalloc(d.q, d.kp, d.vp, d.cu, wl.max_n, d.kc, d.vc, g["cand_len"],
                                g["copy_gate"], d.lm, s.W, s.D, wl.scale, attn, am)
    torch.cuda.synchronize()
    return (a0, m0), (attn, am)


@pytest.mark.parametrize("first,second", [("llama8b_b1", "small_bf16"), ("small_bf16", "tiny")])
def test_noalloc_equals_workspace_call_twice(first, second):
    for name, over in ((first, {"lm_std": 1.0}), (second, {"lm_std": 1.0})):
        wl = generate(name, **over)
        print(f"[case] noalloc {name} B={wl.spec.B} dtype={wl.spec.dtype}", flush=True)
        (a0, m0), (a1, m1) = _both(wl)
        assert torch.equal(m0, m1)
        assert torch.equal(a0.view(torch.int16) if a0.dtype == torch.bfloat16 else a0,
                           a1.view(torch.int16) if a1.dtype == torch.bfloat16 else a1)
        assert int((m1 >= 0).sum()) > 0


def test_noalloc_refuses_partials_beyond_the_scratch():
    # 32 sequences of the 70B share's width need far more than 64 MiB of partials
    B, W, D, Hq, Hkv, d, V, n = 32, 10, 20, 64, 8, 128, 1024, 32768
    need = cdv.verify_workspace_bytes(B, n, W, D, Hq, Hkv, d, V, torch.bfloat16)
    assert need > 64 << 20
    print(f"[case] noalloc refused: need {need} bytes", flush=True)
    R = 1 + W * D
    q = torch.zeros(B, R, Hq, d, dtype=torch.bfloat16, device=DEV)
    kp = torch.zeros(B * 64, Hkv, d, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(B, W * D, Hkv, d, dtype=torch.bfloat16, device=DEV)
    cu = torch.arange(0, B * 64 + 1, 64, dtype=torch.int32, device=DEV)
    cl = torch.zeros(B, W, dtype=torch.int32, device=DEV)
    gate = torch.zeros(B, dtype=torch.uint8, device=DEV)
    lm = cdv.pack_weight(torch.zeros(V, Hq * d, dtype=torch.bfloat16, device=DEV))
    attn = torch.empty(B, R, Hq * d, dtype=torch.bfloat16, device=DEV)
    am = torch.empty(B, R, dtype=torch.int32, device=DEV)
    with pytest.raises(cdv.SwitchSDError, match="workspace"):
        cdv.blocktri_verify_noalloc(q, kp, kp, cu, n, kc, kc, cl, gate, lm, W, D, 0.088, attn, am)
