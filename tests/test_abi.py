"""The C-ABI library loads and exports every entry point include/switchsd.h declares,
and host-side validation rejects bad arguments before any launch (no GPU needed:
every call below returns from validation without touching the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "switchsd.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from copy_draft_verification_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libswitchsd.so not built (run __graft_entry__.build())")
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) >= {"ssd_probe_score", "ssd_kgram_retrieve", "ssd_blocktri_verify",
                          "ssd_accept_longest", "ssd_verify_workspace_bytes", "ssd_abi_version",
                          "ssd_status_string", "ssd_commit_accepted", "ssd_copy_labels",
                          "ssd_copy_labels_workspace_bytes", "ssd_probe_logits",
                          "ssd_calibrate", "ssd_calibrate_workspace_bytes",
                          "ssd_blocktri_verify_sample", "ssd_accept_sample",
                          "ssd_verify_forward", "ssd_verify_forward_workspace_bytes",
                          "ssd_pack_weight", "ssd_pack_weight_bytes", "ssd_pack_gate_up",
                          "ssd_pack_gate_up_bytes", "ssd_probe_kgram_retrieve",
                          "ssd_blocktri_verify_noalloc", "ssd_blocktri_verify_accept"}
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_matches_header(lib):
    m = re.search(r"#define SSD_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.ssd_abi_version() == int(m.group(1))


def test_status_strings(lib):
    assert lib.ssd_status_string(0) == b"ok"
    assert lib.ssd_status_string(3).startswith(b"workspace")
    assert lib.ssd_status_string(99) == b"unknown status"


def test_workspace_query(lib):
    f = lib.ssd_verify_workspace_bytes
    assert f(1, 4096, 10, 20, 32, 8, 128, 128256, 1) > 0
    assert f(0, 4096, 10, 20, 32, 8, 128, 128256, 1) == 0          # B < 1
    assert f(1, 4096, 10, 20, 32, 7, 128, 128256, 1) == 0          # Hq % Hkv
    assert f(1, 4096, 10, 20, 32, 8, 64, 128256, 1) == 0           # bf16 needs d = 128
    assert f(1, 4096, 65, 20, 32, 8, 128, 128256, 1) == 0          # W above limit
    assert f(1, 512, 10, 20, 1, 1, 64, 1000, 0) > 0                # fp32, d = 64
    small = f(1, 512, 10, 20, 1, 1, 64, 1000, 0)
    assert f(8, 512, 10, 20, 1, 1, 64, 1000, 0) > small
    # bf16 byte offsets are 32-bit: (max_n + 64) * Hkv * d * 2 and B * R * Hq * d * 2
    # must stay below 0x7ffffff0
    assert f(1, 1048511, 10, 20, 32, 8, 128, 1000, 1) > 0           # (n + 64) * 2 KiB
    assert f(1, 1048512, 10, 20, 32, 8, 128, 1000, 1) == 0
    assert f(1304, 4096, 10, 20, 32, 8, 128, 1000, 1) > 0           # 1304 * 201 * 8 KiB
    assert f(1305, 4096, 10, 20, 32, 8, 128, 1000, 1) == 0
    assert f(1305, 4096, 10, 20, 32, 8, 64, 1000, 0) > 0            # fp32 path: no limit
    # the row-major bf16 LM head needs the packed one's workspace
    assert f(1, 4096, 10, 20, 32, 8, 128, 128256, 2) == f(1, 4096, 10, 20, 32, 8, 128, 128256, 1)
    assert f(1, 4096, 10, 20, 32, 8, 128, 128256, 3) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x1008)


def test_pack_validation(lib):
    nb = lib.ssd_pack_weight_bytes
    assert nb(128256, 4096) == 128256 * 4096 * 2                 # 501 full tiles of 256 rows
    assert nb(1000, 512) == 1024 * 512 * 2                       # last tile zero-padded
    assert nb(0, 4096) == 0 and nb(10, 0) == 0
    assert nb(10, 4095) == 0 and nb(10, 4160) == 0               # K % 256
    assert nb(10, (1 << 20) + 256) == 0
    pb = lib.ssd_pack_gate_up_bytes
    assert pb(14336, 4096) == 2 * 14336 * 4096 * 2               # 112 tiles of 128 features
    assert pb(300, 256) == 3 * 256 * 256 * 2                     # 3 tiles, zero-padded
    assert pb(0, 256) == 0 and pb(128, 100) == 0
    f = lib.ssd_pack_weight
    good = [FAKE, 1000, 512, FAKE, 1024 * 512 * 2, None]
    for i, bad in ((0, None), (3, None), (1, 0), (2, 0), (0, ctypes.c_void_p(0x1008)),
                   (3, ctypes.c_void_p(0x1004))):
        a = list(good)
        a[i] = bad
        assert f(*a) == 1, (i, bad)
    a = list(good)
    a[2] = 320
    assert f(*a) == 2                                            # K % 256
    a = list(good)
    a[4] = 1024 * 512 * 2 - 16
    assert f(*a) == 3                                            # packed buffer too small
    fp = lib.ssd_pack_gate_up
    goodp = [FAKE, FAKE, 300, 256, FAKE, 3 * 256 * 256 * 2, None]
    for i, bad in ((0, None), (1, None), (4, None), (2, 0), (1, ctypes.c_void_p(0x1002))):
        a = list(goodp)
        a[i] = bad
        assert fp(*a) == 1, (i, bad)
    a = list(goodp)
    a[5] = 3 * 256 * 256 * 2 - 16
    assert fp(*a) == 3


def test_probe_validation(lib):
    f = lib.ssd_probe_score
    assert f(None, 0, FAKE, 1, 8, 0.4, None, FAKE, None) == 1
    assert f(FAKE, 0, FAKE, 0, 8, 0.4, None, FAKE, None) == 1
    assert f(FAKE, 0, FAKE, 1, 8, 1.0, None, FAKE, None) == 1
    assert f(FAKE, 0, FAKE, 1, 8, 0.0, None, FAKE, None) == 1
    assert f(FAKE, 0, FAKE, 1, 8, float("nan"), None, FAKE, None) == 1
    assert f(FAKE, 7, FAKE, 1, 8, 0.4, None, FAKE, None) == 1


def test_kgram_validation(lib):
    f = lib.ssd_kgram_retrieve
    args = [FAKE, FAKE, 1, 5, 10, 20, None, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    for i, bad in ((2, 0), (3, 0), (3, 65), (4, 0), (4, 65), (5, 0), (5, 65), (0, None), (7, None)):
        a = list(args)
        a[i] = bad
        assert f(*a) == 1, (i, bad)


def test_probe_kgram_validation(lib):
    f = lib.ssd_probe_kgram_retrieve
    args = [FAKE, 1, FAKE, 4096, 0.4, None, FAKE, FAKE, FAKE, 1, 5, 10, 20, FAKE, FAKE, FAKE, FAKE,
            FAKE, None]
    for i, bad in ((0, None), (2, None), (6, None), (7, None), (8, None), (13, None), (17, None),
                   (1, 7), (3, 0), (4, 0.0), (4, 1.0), (4, float("nan")), (9, 0), (10, 0),
                   (10, 65), (11, 0), (11, 65), (12, 0), (12, 65)):
        a = list(args)
        a[i] = bad
        assert f(*a) == 1, (i, bad)


def _verify_args(**over):
    a = dict(q=FAKE, k_pre=FAKE, v_pre=FAKE, cu_len=FAKE, max_n=4096, k_cand=FAKE, v_cand=FAKE,
             cand_len=FAKE, copy_gate=FAKE, lm_head=FAKE, B=1, W=10, D=20, Hq=32, Hkv=8, d=128,
             V=128256, dtype=1, scale=0.088, attn_out=FAKE, argmax_out=FAKE, logits_out=None,
             ws=FAKE, ws_bytes=1 << 40, ev0=None, ev1=None, stream=None)
    a.update(over)
    return list(a.values())


def test_verify_validation(lib):
    f = lib.ssd_blocktri_verify
    assert f(*_verify_args(q=None)) == 1
    assert f(*_verify_args(Hkv=5)) == 1
    assert f(*_verify_args(scale=0.0)) == 1
    assert f(*_verify_args(scale=float("inf"))) == 1
    assert f(*_verify_args(d=64)) == 2                     # unsupported for bf16
    assert f(*_verify_args(dtype=0, d=96)) == 2
    assert f(*_verify_args(Hq=3, Hkv=1)) == 2               # bf16 hidden size not a multiple of 256
    # fp32 has no such limit: the shape passes and the (too small) workspace is refused
    assert f(*_verify_args(dtype=0, Hq=3, Hkv=1, ws_bytes=16)) == 3
    assert f(*_verify_args(ws_bytes=16)) == 3
    assert f(*_verify_args(ws=None)) == 3
    # the kernels move q, K, V, the weights and the output in 16-byte pieces
    for k in ("q", "k_pre", "v_pre", "k_cand", "v_cand", "lm_head", "attn_out"):
        assert f(*_verify_args(**{k: MISALIGNED})) == 1, k
        assert f(*_verify_args(dtype=0, d=64, **{k: MISALIGNED})) == 1, k
    # B*R*Hq must stay below 2^31 (32-bit index math in the merges)
    assert f(*_verify_args(dtype=0, d=64, B=2 ** 20, W=64, D=64, Hq=1, Hkv=1)) == 2
    # SSD_BF16_ROWS (bf16, row-major LM head) takes bf16's shape rules
    assert f(*_verify_args(dtype=2, d=64)) == 2
    assert f(*_verify_args(dtype=2, Hq=3, Hkv=1)) == 2
    assert f(*_verify_args(dtype=2, ws_bytes=16)) == 3
    assert f(*_verify_args(dtype=2, lm_head=MISALIGNED)) == 1
    assert f(*_verify_args(dtype=3)) == 1


def _verify_accept_args(**over):
    a = dict(q=FAKE, k_pre=FAKE, v_pre=FAKE, cu_len=FAKE, max_n=4096, k_cand=FAKE, v_cand=FAKE,
             cand=FAKE, cand_len=FAKE, copy_gate=FAKE, lm_head=FAKE, B=1, W=10, D=20, Hq=32, Hkv=8,
             d=128, V=128256, dtype=1, scale=0.088, attn_out=FAKE, argmax_out=FAKE,
             accept_len=FAKE, best_w=FAKE, best_len=FAKE, next_token=FAKE, ws=FAKE,
             ws_bytes=1 << 40, ev0=None, ev1=None, stream=None)
    a.update(over)
    return list(a.values())


def test_verify_accept_validation(lib):
    f = lib.ssd_blocktri_verify_accept
    for k in ("cand", "accept_len", "best_w", "best_len", "next_token", "q", "argmax_out"):
        assert f(*_verify_accept_args(**{k: None})) == 1, k
    assert f(*_verify_accept_args(W=65)) == 1
    assert f(*_verify_accept_args(D=0)) == 1
    assert f(*_verify_accept_args(scale=0.0)) == 1
    assert f(*_verify_accept_args(d=64)) == 2
    assert f(*_verify_accept_args(ws_bytes=16)) == 3
    assert f(*_verify_accept_args(k_pre=MISALIGNED)) == 1
    assert f(*_verify_accept_args(dtype=2, ws_bytes=16)) == 3
    assert f(*_verify_accept_args(dtype=2, d=64)) == 2


def test_accept_validation(lib):
    f = lib.ssd_accept_longest
    good = [FAKE, FAKE, FAKE, FAKE, 1, 10, 20, FAKE, FAKE, FAKE, FAKE, None]
    for i, bad in ((0, None), (4, 0), (5, 0), (5, 65), (6, 65), (10, None)):
        a = list(good)
        a[i] = bad
        assert f(*a) == 1, (i, bad)


def test_commit_validation(lib):
    f = lib.ssd_commit_accepted
    good = dict(kc=FAKE, vc=FAKE, cand=FAKE, bw=FAKE, bl=FAKE, nt=FAKE, B=2, W=10, D=20, Hkv=8,
                d=128, dtype=1, k_cache=FAKE, v_cache=FAKE, rows=1 << 20, off=FAKE, tok=FAKE,
                ntok=FAKE, stream=None)

    def call(**over):
        a = dict(good)
        a.update(over)
        return f(*a.values())

    for k in ("kc", "vc", "cand", "bw", "bl", "nt", "k_cache", "v_cache", "off", "tok", "ntok"):
        assert call(**{k: None}) == 1, k
    for k, bad in (("B", 0), ("W", 0), ("W", 65), ("D", 0), ("D", 65), ("Hkv", 0), ("d", 0),
                   ("rows", 0), ("dtype", 5)):
        assert call(**{k: bad}) == 1, (k, bad)
    assert call(Hkv=1, d=3) == 2                        # 6-byte rows: not 16-byte pieces
    assert call(dtype=0, Hkv=1, d=2) == 2               # 8-byte fp32 rows


def test_copy_labels_validation(lib):
    f = lib.ssd_copy_labels
    ws = lib.ssd_copy_labels_workspace_bytes
    assert ws(0) == 0 and ws(1 << 30) == 0
    assert ws(1000) >= 2048 * 8 + 1000                  # table of >= 2n slots + repeat flags
    good = dict(ids=FAKE, cu=FAKE, B=2, n=1000, n_train=5, labels=FAKE, ws=FAKE, wsb=ws(1000),
                stream=None)

    def call(**over):
        a = dict(good)
        a.update(over)
        return f(*a.values())

    for k in ("ids", "cu", "labels"):
        assert call(**{k: None}) == 1, k
    for k, bad in (("B", 0), ("n", 0), ("n", 1 << 30), ("n_train", 0), ("n_train", 65)):
        assert call(**{k: bad}) == 1, (k, bad)
    assert call(ws=None) == 3
    assert call(wsb=ws(1000) - 1) == 3


def test_probe_logits_validation(lib):
    f = lib.ssd_probe_logits
    good = dict(h=FAKE, dtype=1, w=FAKE, L=32, N=4096, hid=4096, z=FAKE, stream=None)

    def call(**over):
        a = dict(good)
        a.update(over)
        return f(*a.values())

    for k in ("h", "w", "z"):
        assert call(**{k: None}) == 1, k
    for k, bad in (("L", 0), ("L", 65536), ("N", 0), ("N", 1 << 36), ("hid", 0), ("dtype", 2)):
        assert call(**{k: bad}) == 1, (k, bad)
    assert call(hid=16385) == 2


def test_calibrate_validation(lib):
    f = lib.ssd_calibrate
    ws = lib.ssd_calibrate_workspace_bytes
    assert ws(32, 4096) == 32 * 4096 * 8
    assert ws(2, 10) == 2 * 1024 * 8                    # at least 1024 keys per layer
    assert ws(3, 20000) == 3 * 32768 * 8                # padded to a power of two per layer
    assert ws(0, 10) == 0 and ws(1, 0) == 0 and ws(1, (1 << 28) + 1) == 0
    good = dict(z=FAKE, labels=FAKE, L=4, N=5000, thr=FAKE, counts=FAKE, u2=FAKE, auc=FAKE,
                best=FAKE, tau=FAKE, ws=FAKE, wsb=ws(4, 5000), stream=None)

    def call(**over):
        a = dict(good)
        a.update(over)
        return f(*a.values())

    for k in ("z", "labels", "thr", "counts", "u2", "auc", "best", "tau"):
        assert call(**{k: None}) == 1, k
    for k, bad in (("L", 0), ("L", 65536), ("N", 0), ("N", (1 << 28) + 1)):
        assert call(**{k: bad}) == 1, (k, bad)
    assert call(ws=None) == 3
    assert call(wsb=ws(4, 5000) - 8) == 3


def _sample_args(**over):
    a = dict(q=FAKE, k_pre=FAKE, v_pre=FAKE, cu_len=FAKE, max_n=4096, k_cand=FAKE, v_cand=FAKE,
             cand=FAKE, cand_len=FAKE, copy_gate=FAKE, lm_head=FAKE, B=1, W=10, D=20, Hq=32, Hkv=8,
             d=128, V=128256, dtype=1, scale=0.088, temperature=1.0, seed=7, attn_out=FAKE,
             n_children=FAKE, children=FAKE, child_w=FAKE, child_logit=FAKE, lse=FAKE,
             resample=FAKE, ws=FAKE, ws_bytes=16, ev0=None, ev1=None, stream=None)
    a.update(over)
    return list(a.values())


def test_verify_sample_validation(lib):
    f = lib.ssd_blocktri_verify_sample
    for k in ("q", "cand", "n_children", "children", "child_w", "child_logit", "lse", "resample"):
        assert f(*_sample_args(**{k: None})) == 1, k
    for t in (0.0, -1.0, float("inf"), float("nan"), 1e-45):
        assert f(*_sample_args(temperature=t)) == 1, t           # 1e-45: 1/T overflows
    assert f(*_sample_args(dtype=0, d=64, Hq=1, Hkv=1)) == 2      # sampling is bf16 only
    assert f(*_sample_args(d=64)) == 2
    assert f(*_sample_args(dtype=2)) == 2                         # sampling needs the packed head
    assert f(*_sample_args()) == 3                                # workspace too small
    assert f(*_sample_args(seed=(1 << 64) - 1)) == 3              # any 64-bit seed is accepted
    assert f(*_sample_args(v_cand=MISALIGNED)) == 1


def test_accept_sample_validation(lib):
    f = lib.ssd_accept_sample
    good = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 10, 20, 7, FAKE, FAKE, FAKE, None]
    for i, bad in ((0, None), (4, None), (5, None), (6, 0), (7, 0), (7, 65), (8, 0), (8, 65),
                   (12, None)):
        a = list(good)
        a[i] = bad
        assert f(*a) == 1, (i, bad)


def test_verify_forward_validation(lib):
    f = lib.ssd_verify_forward
    ws = lib.ssd_verify_forward_workspace_bytes
    assert ws(1, 4096, 10, 20, 32, 8, 128, 14336, 128256) > 0
    assert ws(1, 4096, 10, 20, 32, 8, 64, 14336, 128256) == 0        # d != 128
    assert ws(1, 4096, 10, 20, 32, 8, 128, 14335, 128256) == 0       # inter % 256
    assert ws(372, 4096, 10, 20, 32, 8, 128, 14336, 128256) > 0      # 372 * 201 * 28 KiB
    assert ws(373, 4096, 10, 20, 32, 8, 128, 14336, 128256) == 0
    good = dict(ids=FAKE, cu=FAKE, max_n=4096, cand=FAKE, cl=FAKE, gate=FAKE, embed=FAKE,
                layers=None, n_layers=0, final_norm=FAKE, lm=FAKE, B=1, W=10, D=20, Hq=32, Hkv=8,
                d=128, inter=14336, V=128256, base=500000.0, eps=1e-5, am=FAKE, x=None, ws=FAKE,
                wsb=16, ev0=None, ev1=None, stream=None)

    def call(**over):
        a = dict(good)
        a.update(over)
        return f(*a.values())

    for k in ("ids", "cand", "embed", "final_norm", "lm", "am"):
        assert call(**{k: None}) == 1, k
    assert call(x=ctypes.c_void_p(0x1004)) == 1          # x_out not 16-byte aligned
    assert call(n_layers=-1) == 1
    assert call(n_layers=2) == 1                          # layers missing
    for k, bad in (("base", 1.0), ("base", float("nan")), ("eps", 0.0), ("Hkv", 5), ("W", 65)):
        assert call(**{k: bad}) == 1, (k, bad)
    assert call(d=64) == 2 and call(Hq=72) == 2           # hid = 9216 > 8192
    assert call() == 3                                    # workspace too small
