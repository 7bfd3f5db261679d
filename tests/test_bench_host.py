"""Host logic of bench.py, on the CPU: the algorithmic work it divides by (the
roofline's numerator), the counter-file lookup behind `traffic`, and the refusal
of more than one GPU.  The figures are the closed forms of the work the paper's
§3.3 verification needs (the LM head streams every weight once; attention
counts 4 Hq d flops per visible (row, key) pair), written out independently here."""
import hashlib
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import generate  # noqa: E402


def _spec(name):
    return generate(name, with_tensors=False).spec


def test_lm_algorithmic_llama8b_b1_closed_form():
    s = _spec("llama8b_b1")
    rows = 1 + s.W * s.D                       # every gate open, every candidate full
    byts, flops = bench.lm_algorithmic(s, rows)
    assert byts == 128256 * 4096 * 2 + rows * 4096 * 2 + rows * 4 == 1052320548
    assert flops == 2.0 * rows * 4096 * 128256


def test_lm_algorithmic_closed_gates_is_zero():
    s = _spec("llama8b_b1")
    assert bench.lm_algorithmic(s, 0) == (0, 0.0)


def test_attn_algorithmic_llama8b_b1_closed_form():
    s = _spec("llama8b_b1")
    n = np.array([4096])
    cand_len = np.full((1, s.W), s.D)
    byts, flops = bench.attn_algorithmic(s, n, np.array([1]), cand_len)
    r_real = 1 + s.W * s.D
    kv = s.Hkv * s.d * 2 * 2                   # K and V per key, bf16
    assert byts == 4096 * kv + 2 * r_real * s.Hq * s.d * 2 + s.W * s.D * kv
    # each real row sees the whole prefix; candidate token j of w also sees w's
    # first j+1 tokens
    pairs = r_real * 4096 + s.W * (s.D * (s.D + 1) // 2)
    assert flops == 4.0 * s.Hq * s.d * pairs == 13523288064.0


def test_attn_algorithmic_skips_closed_gates_and_short_candidates():
    s = _spec("llama8b_b1")
    n = np.array([1000, 2000])
    cand_len = np.array([[3] + [0] * (s.W - 1), [s.D] * s.W])
    b_open, f_open = bench.attn_algorithmic(s, n[1:], np.array([1]), cand_len[1:])
    b_both, f_both = bench.attn_algorithmic(s, n, np.array([0, 1]), cand_len)
    assert (b_both, f_both) == (b_open, f_open)
    _, f_short = bench.attn_algorithmic(s, n[:1], np.array([1]), cand_len[:1])
    assert f_short == 4.0 * s.Hq * s.d * ((1 + 3) * 1000 + 3 * 4 // 2)


def test_measured_traffic_follows_the_source(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "traffic.txt"
    prof.write_text("# comment = ignored\nworkload = wl\nkernel = k\n"
                    f"source_sha256 = {sha}\ntraffic_bytes_per_launch = 123456\n")
    assert bench.measured_traffic("wl", str(prof), str(src)) == 123456
    assert bench.measured_traffic("other", str(prof), str(src)) is None
    src.write_text("// kernel v2\n")
    assert bench.measured_traffic("wl", str(prof), str(src)) is None
    assert bench.measured_traffic("wl", str(tmp_path / "missing.txt"), str(src)) is None


def test_committed_lm_traffic_matches_the_current_kernel():
    """The committed counter summary was taken on the LM head as it is now (else
    bench.py would report traffic null)."""
    t = bench.measured_traffic("llama8b_b1")
    assert t is not None and 1.0 <= t / 1052320548 < 1.05


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
