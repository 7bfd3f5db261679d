"""Benchmark of one SwitchSD copy-speculation step on one MI355X.

A step is the whole hot path over one batch, all on one HIP stream with no host
synchronisation inside: probe_score -> kgram_retrieve -> blocktri_verify
(block-triangular attention, LM head, argmax) -> accept_longest.  Inputs are
synthetic (seeded) and resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b_b1]
                    [--no-cpu-baseline]

Prints one JSON line: copy-steps/s (whole job), verified candidate tokens/s,
the LM-head kernel's roofline position (HIP events around that kernel in the
timed region) and the CPU oracle timed on the host on a bounded sample.

    python bench.py --calibration [--steps K] [--warmup W]

measures the offline probe calibration instead: one pass is copy labels, probe
logits at every position of every layer, and the per-layer F1 / AUC sweep with the
layer choice, over a 32-layer, 4096-position, 4096-wide bf16 set.

    python bench.py --scan [--steps K] [--warmup W]

times kappa-gram retrieval alone over 2^24, 2^26 and 2^28 Zipf ids in contexts of
16384 (every context scanned to its start unless W matches stop it earlier).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0     # dense bf16
FP32_PEAK_TFS = 157.3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="llama8b_b1")
    p.add_argument("--anchor", default=None, choices=("full", "natural"),
                   help="anchor mode of the synthetic contexts (default: the workload's own)")
    p.add_argument("--W", type=int, default=None, help="candidates per sequence (default: the workload's)")
    p.add_argument("--D", type=int, default=None, help="tokens per candidate (default: the workload's)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=20.0)
    p.add_argument("--temperature", type=float, default=0.0,
                   help="> 0: verify by sampling at this temperature (blocktri_verify_sample + "
                        "accept_sample) instead of greedy")
    p.add_argument("--seed", type=int, default=0x5EED, help="sampling seed (with --temperature)")
    p.add_argument("--forward", type=int, default=0, metavar="LAYERS",
                   help="> 0: verify with a full target forward of this many synthetic "
                        "Llama-3.1-8B layers (ssd_verify_forward) instead of the single-layer share")
    p.add_argument("--calibration", action="store_true",
                   help="time the offline probe calibration pass instead of the decoding step")
    p.add_argument("--scan", action="store_true",
                   help="time kappa-gram retrieval alone on large id arrays (2^24, 2^26, 2^28 ids "
                        "in contexts of 16384) instead of the decoding step")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (the reference point that scales the "
                        "HBM byte counters) and exit")
    return p.parse_args()


COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_bf16_kernel.llama8b_b1.traffic.txt")
SAMPLE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_bf16_kernel_sample.llama8b_b1.traffic.txt")
LM_SOURCE = os.path.join(ROOT, "copy_draft_verification_amd", "csrc", "lmhead.hip")
CAL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "probe_logits_kernel.calib_llama8b.traffic.txt")
CAL_SOURCE = os.path.join(ROOT, "copy_draft_verification_amd", "csrc", "calib.hip")
SCAN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kgram_kernel.scan_2e28.traffic.txt")
SCAN_SOURCE = os.path.join(ROOT, "copy_draft_verification_amd", "csrc", "kgram.hip")


def calibrate_copy():
    """A plain device copy of COPY_BYTES, five times: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    over this run give the counters' reading for a known number of bytes."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(5):
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[copy] {i} copied {COPY_BYTES} bytes", file=sys.stderr, flush=True)


def measured_traffic(workload, path=TRAFFIC_FILE, source=LM_SOURCE):
    """HBM bytes per launch of a kernel from its committed counter summary, or None
    when it does not cover this workload or the kernel source changed since."""
    import hashlib
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    with open(source, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if kv.get("workload") != workload or kv.get("source_sha256") != sha:
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def lm_algorithmic(s, R_tot):
    """LM-head work the method itself needs: the weights once, the real rows in,
    one int per row out; 2 flops per weight per real row.  With no real row (every
    gate closed) there is nothing to contract and nothing to read."""
    elt = 2 if s.dtype == "bf16" else 4
    byts = (s.V * s.hid * elt + R_tot * s.hid * elt + 4 * R_tot) if R_tot > 0 else 0
    flops = 2.0 * R_tot * s.hid * s.V
    return byts, flops


def cpu_baseline(wl, budget_s):
    """Time the oracle (as it stands) on the host for one step of this workload.

    Integer stages and the probe run on every sequence.  Attention and the LM head
    run on a seeded sample of real rows sized to the budget, and their time is
    scaled to all real rows of the step."""
    import oracle
    from oracle.attention import real_rows
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    s = wl.spec
    t0 = time.perf_counter()
    pr = oracle.probe_score(wl.h, wl.w, s.tau)
    kg = oracle.kgram_retrieve(wl.ids, wl.cu_len, s.kappa, s.W, s.D, pr["fire"])
    t_int = time.perf_counter() - t0
    real = [(b, r) for b in range(s.B) for r in real_rows(kg["cand_len"][b], kg["copy_gate"][b], s.W, s.D)]
    if not real:
        return None
    rng = np.random.default_rng(0)
    # attention: grow the sample until about a third of the budget is spent
    k_att = min(len(real), 8)
    while True:
        idx = rng.choice(len(real), k_att, replace=False)
        rows = [real[i] for i in idx]
        t0 = time.perf_counter()
        out, ev = oracle.blocktri_attention(wl.q, wl.k_pre, wl.v_pre, wl.cu_len, wl.k_cand, wl.v_cand,
                                            kg["cand_len"], kg["copy_gate"], s.Hq, s.Hkv, s.d, s.W,
                                            s.D, wl.scale, rows=rows)
        t_att = time.perf_counter() - t0
        if t_att > budget_s / 3 or k_att == len(real):
            break
        k_att = min(len(real), k_att * 4)
    # LM head: every real row in one call when the step has at most 1024 of them
    # (the weight widening is part of the oracle's call); otherwise a 256-row sample
    # whose whole-call time is scaled by rows (this overstates the CPU time)
    k_lm = n_real = len(real)
    if n_real > 1024:
        k_lm = 256
    rows_lm = real if k_lm == n_real else [real[i] for i in rng.choice(n_real, k_lm, replace=False)]
    if k_att < n_real or rows_lm is not real:
        out, _ = oracle.blocktri_attention(wl.q, wl.k_pre, wl.v_pre, wl.cu_len, wl.k_cand, wl.v_cand,
                                           kg["cand_len"], kg["copy_gate"], s.Hq, s.Hkv, s.d, s.W,
                                           s.D, wl.scale, rows=rows_lm)
    O = out[[b for b, _ in rows_lm], [r for _, r in rows_lm]]
    t0 = time.perf_counter()
    lm = oracle.lmhead_argmax(O, wl.lm_head)
    t_lm = time.perf_counter() - t0
    am = np.full((s.B, wl.R), -1, dtype=np.int64)
    for (b, r), p in zip(rows_lm, lm["pred"]):
        am[b, r] = p
    t0 = time.perf_counter()
    oracle.accept_longest(kg["cand"], kg["cand_len"], kg["copy_gate"], am, s.W, s.D)
    t_acc = time.perf_counter() - t0
    t_step = t_int + t_att * n_real / k_att + t_lm * n_real / k_lm + t_acc
    return {"value": s.B / t_step, "unit": "copy-steps/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"{s.name}: probe+kgram+accept on all {s.B} sequences; attention on {k_att} "
                       f"of {n_real} real rows ({t_att:.2f}s), LM head+argmax on {k_lm} rows "
                       f"({t_lm:.2f}s, includes widening the {s.V}x{s.hid} weights to float64); "
                       f"scaled to all rows: {t_step:.2f}s per step"),
            "measured_s": round(t_int + t_att + t_lm + t_acc, 2)}


def calibration_cpu_baseline(c, budget_s):
    """The oracle's calibration on whole layers of the same set (labels once, then
    probe logits and the sweep layer by layer) until the budget is spent; the
    per-layer time is scaled to all layers."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    L = c.H.shape[0]
    t0 = time.perf_counter()
    y = oracle.copy_labels(c.ids, c.cu_len)
    t_lab = time.perf_counter() - t0
    t_layers, done = 0.0, 0
    for l in range(L):
        t0 = time.perf_counter()
        z = oracle.probe_logits(c.H[l:l + 1], c.w[l:l + 1], c.spec.dtype)
        oracle.threshold_sweep(z[0], y)
        t_layers += time.perf_counter() - t0
        done += 1
        if t_lab + t_layers > budget_s:
            break
    t_pass = t_lab + t_layers * L / done
    return {"value": 1.0 / t_pass, "unit": "calibration-passes/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"{c.spec.name}: labels of all {c.H.shape[1]} positions ({t_lab:.2f}s), "
                       f"probe logits + F1/AUC sweep on {done} of {L} layers ({t_layers:.2f}s), "
                       f"scaled to all layers: {t_pass:.2f}s per pass"),
            "measured_s": round(t_lab + t_layers, 2)}


def bench_calibration(a):
    """Offline probe calibration: labels -> probe logits -> sweep + layer choice, no
    host synchronisation inside a pass.  The roofline entry is the probe
    logit GEMV (it streams every layer's states once from HBM)."""
    import torch
    import copy_draft_verification_amd as cdv
    from workloads import generate_calibration, to_torch

    c = generate_calibration("calib_llama8b")
    s = c.spec
    L, N, hid = c.H.shape
    dev = "cuda:0"
    up = lambda x: to_torch(x, dev)  # noqa: E731
    ids, cu, H, w = up(c.ids), up(c.cu_len), up(c.H), up(c.w)
    lab = torch.empty(N, dtype=torch.uint8, device=dev)
    lws = torch.empty(cdv.copy_labels_workspace_bytes(N), dtype=torch.uint8, device=dev)
    z = torch.empty(L, N, dtype=torch.float32, device=dev)
    cws = torch.empty(cdv.calibrate_workspace_bytes(L, N), dtype=torch.uint8, device=dev)
    out = {"thr": torch.empty(L, dtype=torch.float32, device=dev),
           "counts": torch.empty(L, 4, dtype=torch.int32, device=dev),
           "u2": torch.empty(L, dtype=torch.int64, device=dev),
           "auc": torch.empty(L, dtype=torch.float32, device=dev),
           "best_layer": torch.empty(1, dtype=torch.int32, device=dev),
           "tau": torch.empty(1, dtype=torch.float32, device=dev)}
    stream = torch.cuda.current_stream()
    # the labels depend only on the token ids: they run on a second stream (default
    # priority) beside the probe-logit GEMV and are joined before the sweep
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def one(ev=None):
        fork.record(stream)
        side.wait_event(fork)
        cdv.copy_labels(ids, cu, 5, labels=lab, workspace=lws, stream=side)
        join.record(side)
        if ev is not None:
            ev[0].record(stream)
        cdv.probe_logits(H, w, z_out=z, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        stream.wait_event(join)
        cdv.calibrate(z, lab, out=out, workspace=cws, stream=stream)

    print(f"[bench] calibration {s.name} L={L} N={N} hid={hid} warmup={a.warmup} steps={a.steps}",
          file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        one()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(a.steps):
        one(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_begin.elapsed_time(t_end) / a.steps
    k_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    elt = 2 if s.dtype == "bf16" else 4
    k_bytes = L * N * hid * elt + L * hid * 4 + L * N * 4
    achieved = k_bytes / (k_ms * 1e-3) / 1e9
    print(f"[bench] {ms:.4f} ms/pass, probe-logits kernel {k_ms:.4f} ms ({achieved:.0f} GB/s), "
          f"layer {int(out['best_layer'][0])} tau {float(out['tau'][0]):.4f}", file=sys.stderr, flush=True)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(s.name, CAL_TRAFFIC_FILE, CAL_SOURCE),
            "kernel": "probe_logits_kernel", "kernel_ms": round(k_ms, 4),
            "algorithmic_bytes": int(k_bytes)}
    cpu = None
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = calibration_cpu_baseline(c, a.cpu_budget_s)
    line = {
        "metric": "probe calibration passes/sec (labels + per-layer probe logits + F1/AUC sweep)",
        "value": round(1.0 / (ms * 1e-3), 2),
        "unit": "calibration-passes/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": s.name, "L": L, "N": N, "hid": hid, "n_train": 5,
                   "parallelism": "single-gpu"},
        "scored_positions_per_s": round(L * N / (ms * 1e-3), 1),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def scan_algorithmic(n, kappa, W, D, n_match, last_end, cand_len):
    """Bytes the retrieval itself must move: each context's ids from the anchor back
    to the start of the W-th match (all n when fewer than W matches exist), the
    offsets, the gathered candidate ids, and the outputs."""
    n = np.asarray(n, dtype=np.int64)
    full = n_match >= W
    scanned = np.where(full, n - last_end + kappa - 1, n)
    B = len(n)
    out = B * (4 * W + 4 + 4 * W * D + 4 * W + 1)
    return int(4 * scanned.sum() + 4 * (B + 1) + 4 * int(cand_len.sum()) + out)


def bench_scan(a):
    """kappa-gram retrieval over many long contexts (the step's retrieval call alone,
    every probe fired).  Each launch is timed with HIP events; between launches a
    1 GiB buffer is overwritten (outside the timed launches) so that the ids come
    from HBM, not from the 256 MB last-level cache."""
    import torch
    import copy_draft_verification_amd as cdv
    import oracle
    from workloads import SCAN_N, SCAN_SIZES, scan_ids_device

    kappa, W, D = 5, 10, 20
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    rows = []
    for total in SCAN_SIZES:
        ids, cu = scan_ids_device(total, device=dev)
        B = cu.numel() - 1
        out = {"match_end": torch.empty(B, W, dtype=torch.int32, device=dev),
               "n_match": torch.empty(B, dtype=torch.int32, device=dev),
               "cand": torch.empty(B, W, D, dtype=torch.int32, device=dev),
               "cand_len": torch.empty(B, W, dtype=torch.int32, device=dev),
               "copy_gate": torch.empty(B, dtype=torch.uint8, device=dev)}
        print(f"[bench] scan total={total} B={B} n={SCAN_N} warmup={a.warmup} steps={a.steps}",
              file=sys.stderr, flush=True)
        for _ in range(a.warmup):
            cdv.kgram_retrieve(ids, cu, kappa, W, D, out=out)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(a.steps)]
        for e0, e1 in evs:
            flush.zero_()
            e0.record(stream)
            cdv.kgram_retrieve(ids, cu, kappa, W, D, out=out)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
        nm = out["n_match"].cpu().numpy()
        last = out["match_end"][:, W - 1].cpu().numpy().astype(np.int64)
        byts = scan_algorithmic(np.full(B, SCAN_N), kappa, W, D, nm, last, out["cand_len"].cpu().numpy())
        k_ms = float(ms.mean())
        gbs = byts / (k_ms * 1e-3) / 1e9
        rows.append({"ids": total, "contexts": B, "kernel_ms": round(k_ms, 4),
                     "kernel_ms_median": round(float(np.median(ms)), 4),
                     "algorithmic_bytes": byts, "GB/s": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "contexts_with_match": int((nm > 0).sum())})
        print(f"[bench] scan total={total}: {k_ms:.4f} ms ({gbs:.0f} GB/s, "
              f"{gbs / HBM_PEAK_GBS:.1%} of HBM), contexts with a match {int((nm > 0).sum())}",
              file=sys.stderr, flush=True)
        last_ids, last_cu, last_out = ids, cu, out
        if total != SCAN_SIZES[-1]:
            del ids, cu, out
            torch.cuda.empty_cache()
    top = rows[-1]
    cpu = None
    if not a.no_cpu_baseline:
        # the oracle on whole contexts of the largest launch, as many as fit the budget
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        B = last_cu.numel() - 1
        done, t_cpu = 0, 0.0
        one = np.array([0, SCAN_N], dtype=np.int32)
        while t_cpu < min(a.cpu_budget_s, 10.0) and done < B:
            x = last_ids[done * SCAN_N:(done + 1) * SCAN_N].cpu().numpy()
            t0 = time.perf_counter()
            oracle.kgram_retrieve(x, one, kappa, W, D)
            t_cpu += time.perf_counter() - t0
            done += 1
        per_launch = t_cpu / done * B
        cpu = {"value": round(top["ids"] / per_launch / 1e9, 6), "unit": "Gids/s", "cores": 1,
               "kind": "oracle",
               "sample": (f"kappa-gram retrieval of {done} of the {B} contexts of {SCAN_N} ids "
                          f"({t_cpu:.2f}s), scaled to the whole launch: {per_launch:.1f}s"),
               "measured_s": round(t_cpu, 2)}
    roof = {"bound": "hbm", "achieved": top["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": top["frac"],
            "traffic": measured_traffic(f"scan_{top['ids']}", SCAN_TRAFFIC_FILE, SCAN_SOURCE),
            "kernel": "kgram_kernel", "kernel_ms": top["kernel_ms"],
            "algorithmic_bytes": top["algorithmic_bytes"]}
    line = {
        "metric": "kappa-gram retrieval: context ids scanned/sec (large-array sweep)",
        "value": round(top["ids"] / (top["kernel_ms"] * 1e-3) / 1e9, 3),
        "unit": "Gids/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": top["kernel_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": f"scan_{top['ids']}", "contexts": top["contexts"], "n": SCAN_N,
                   "V": 128256, "zipf": 1.1, "kappa": kappa, "W": W, "D": D,
                   "parallelism": "single-gpu"},
        "sweep": rows,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_forward(a):
    """The copy step with the verification pass as a full target forward: probe ->
    kgram -> verify_forward (a.forward synthetic Llama-3.1-8B layers) -> accept.
    The weights are drawn on the GPU by torch's seeded generator (14 GB at 32
    layers would take minutes on the host); the contexts are the llama8b_b1 ones."""
    import torch
    import copy_draft_verification_amd as cdv
    from workloads import generate, to_torch

    wl = generate("llama8b_b1", with_tensors=False)
    s = wl.spec
    inter, nl = 14336, a.forward
    dev = "cuda:0"
    up = lambda x: to_torch(x, dev)  # noqa: E731
    g = torch.Generator(device=dev)
    g.manual_seed(a.seed)
    hid, Hq, Hkv, d, V = s.hid, s.Hq, s.Hkv, s.d, s.V
    N = int(wl.cu_len[-1])

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device=dev) * std).to(torch.bfloat16)

    def norm():
        return (1.0 + 0.1 * torch.randn(hid, generator=g, device=dev)).to(torch.bfloat16)

    # each layer's projections are packed as it is drawn (as at model load); the plain
    # copies are released once packed
    layers = [cdv.pack_layer({"attn_norm": norm(), "wqkv": randn((Hq + 2 * Hkv) * d, hid, std=hid ** -0.5),
                              "wo": randn(hid, Hq * d, std=(Hq * d) ** -0.5), "mlp_norm": norm(),
                              "w_gate": randn(inter, hid, std=hid ** -0.5),
                              "w_up": randn(inter, hid, std=hid ** -0.5),
                              "w_down": randn(hid, inter, std=inter ** -0.5),
                              "k_cache": randn(N, Hkv, d), "v_cache": randn(N, Hkv, d)})
              for _ in range(nl)]
    embed, final_norm = randn(V, hid), norm()
    lm = cdv.pack_weight(randn(V, hid, std=hid ** -0.5))   # packed once, as at model load
    ids, cu, h, w = up(wl.ids), up(wl.cu_len), up(wl.h), up(wl.w)
    B, R = s.B, 1 + s.W * s.D
    z = torch.empty(B, dtype=torch.float32, device=dev)
    fire = torch.empty(B, dtype=torch.uint8, device=dev)
    kout = {"match_end": torch.empty(B, s.W, dtype=torch.int32, device=dev),
            "n_match": torch.empty(B, dtype=torch.int32, device=dev),
            "cand": torch.empty(B, s.W, s.D, dtype=torch.int32, device=dev),
            "cand_len": torch.empty(B, s.W, dtype=torch.int32, device=dev),
            "copy_gate": torch.empty(B, dtype=torch.uint8, device=dev)}
    am = torch.empty(B, R, dtype=torch.int32, device=dev)
    ws = torch.empty(cdv.verify_forward_workspace_bytes(B, wl.max_n, s.W, s.D, Hq, Hkv, d, inter, V),
                     dtype=torch.uint8, device=dev)
    aout = {"accept_len": torch.empty(B, s.W, dtype=torch.int32, device=dev),
            "best_w": torch.empty(B, dtype=torch.int32, device=dev),
            "best_len": torch.empty(B, dtype=torch.int32, device=dev),
            "next_token": torch.empty(B, dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream()

    def step(ev=None):
        cdv.probe_score(h, w, s.tau, z_out=z, fire_out=fire, stream=stream)
        cdv.kgram_retrieve(ids, cu, s.kappa, s.W, s.D, fire, out=kout, stream=stream)
        cdv.verify_forward(ids, cu, wl.max_n, kout["cand"], kout["cand_len"], kout["copy_gate"], embed,
                           layers, final_norm, lm, s.W, s.D, Hq, Hkv, d, inter, argmax_out=am,
                           workspace=ws, events=ev, stream=stream)
        cdv.accept_longest(kout["cand"], kout["cand_len"], kout["copy_gate"], am, s.W, s.D, out=aout,
                           stream=stream)

    print(f"[bench] forward llama8b_b1 layers={nl} warmup={a.warmup} steps={a.steps}",
          file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        e1.record(stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(a.steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / a.steps
    f_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    gate = kout["copy_gate"].cpu().numpy().astype(bool)
    cl = kout["cand_len"].cpu().numpy()
    rows = int(gate.sum()) + int(cl[gate].sum())
    per_layer = 2 * ((Hq + 2 * Hkv) * d * hid + hid * Hq * d + 3 * inter * hid) + 2 * 2 * N * Hkv * d
    byts = nl * per_layer + 2 * V * hid + rows * hid * 2 * 2 + 4 * rows
    achieved = byts / (f_ms * 1e-3) / 1e9
    print(f"[bench] {ms:.3f} ms/step, forward {f_ms:.3f} ms ({achieved:.0f} GB/s of weights, caches "
          f"and rows), real rows {rows}", file=sys.stderr, flush=True)
    line = {
        "metric": "copy-steps/sec with a full target forward as the verifier (Llama-3.1-8B shape)",
        "value": round(B / (ms * 1e-3), 2),
        "unit": "copy-steps/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama8b_b1", "layers": nl, "hid": hid, "Hq": Hq, "Hkv": Hkv, "d": d,
                   "inter": inter, "V": V, "W": s.W, "D": s.D, "n": int(N), "parallelism": "single-gpu"},
        "verified_cand_tokens_per_s": round(int(cl[gate].sum()) / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "verify_forward (every kernel of the forward)", "kernel_ms": round(f_ms, 4),
                     "algorithmic_bytes": int(byts)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported in this build "
              f"(the path shards over sequences with no exchange; see the sharding notes).",
              file=sys.stderr)
        sys.exit(2)
    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.calibration:
        bench_calibration(a)
        return
    if a.scan:
        bench_scan(a)
        return
    if a.forward > 0:
        bench_forward(a)
        return
    import torch
    import copy_draft_verification_amd as cdv
    from workloads import generate, to_torch

    over = {k: v for k, v in (("anchor", a.anchor), ("W", a.W), ("D", a.D)) if v is not None}
    wl = generate(a.workload, **over)
    s = wl.spec
    dev = "cuda:0"
    up = lambda x: to_torch(x, dev)  # noqa: E731
    ids, cu, h, w = up(wl.ids), up(wl.cu_len), up(wl.h), up(wl.w)
    q, kp, vp, kc, vc, lm = (up(wl.q), up(wl.k_pre), up(wl.v_pre), up(wl.k_cand), up(wl.v_cand),
                             up(wl.lm_head))
    B, R = s.B, wl.R
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    if tdt == torch.bfloat16:
        lm = cdv.pack_weight(lm)   # packed once, as at model load (outside the timed region)
    # every output and the workspace are allocated once, outside the timed region
    z = torch.empty(B, dtype=torch.float32, device=dev)
    fire = torch.empty(B, dtype=torch.uint8, device=dev)
    kout = {"match_end": torch.empty(B, s.W, dtype=torch.int32, device=dev),
            "n_match": torch.empty(B, dtype=torch.int32, device=dev),
            "cand": torch.empty(B, s.W, s.D, dtype=torch.int32, device=dev),
            "cand_len": torch.empty(B, s.W, dtype=torch.int32, device=dev),
            "copy_gate": torch.empty(B, dtype=torch.uint8, device=dev)}
    attn = torch.empty(B, R, s.Hq * s.d, dtype=tdt, device=dev)
    am = torch.empty(B, R, dtype=torch.int32, device=dev)
    ws = torch.empty(cdv.verify_workspace_bytes(B, wl.max_n, s.W, s.D, s.Hq, s.Hkv, s.d, s.V, tdt),
                     dtype=torch.uint8, device=dev)
    aout = {"accept_len": torch.empty(B, s.W, dtype=torch.int32, device=dev),
            "best_w": torch.empty(B, dtype=torch.int32, device=dev),
            "best_len": torch.empty(B, dtype=torch.int32, device=dev),
            "next_token": torch.empty(B, dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream()
    T = a.temperature
    if T > 0:
        srows = {"n_children": torch.empty(B, R, dtype=torch.int32, device=dev),
                 "children": torch.empty(B, R, s.W, dtype=torch.int32, device=dev),
                 "child_w": torch.empty(B, R, s.W, dtype=torch.int32, device=dev),
                 "child_logit": torch.empty(B, R, s.W, dtype=torch.float32, device=dev),
                 "lse": torch.empty(B, R, dtype=torch.float32, device=dev),
                 "resample": torch.empty(B, R, dtype=torch.int32, device=dev)}

    def step(lm_events=None, i=0):
        cdv.probe_score(h, w, s.tau, z_out=z, fire_out=fire, stream=stream)
        cdv.kgram_retrieve(ids, cu, s.kappa, s.W, s.D, fire, out=kout, stream=stream)
        if T > 0:
            seed = a.seed + i
            cdv.blocktri_verify_sample(q, kp, vp, cu, wl.max_n, kc, vc, kout["cand"],
                                       kout["cand_len"], kout["copy_gate"], lm, s.W, s.D, wl.scale,
                                       T, seed, attn_out=attn, rows=srows, workspace=ws,
                                       events=lm_events, stream=stream)
            cdv.accept_sample(srows, kout["copy_gate"], s.W, s.D, seed,
                              out={k: aout[k] for k in ("best_w", "best_len", "next_token")},
                              stream=stream)
            return
        cdv.blocktri_verify(q, kp, vp, cu, wl.max_n, kc, vc, kout["cand_len"], kout["copy_gate"], lm,
                            s.W, s.D, wl.scale, attn_out=attn, argmax_out=am, workspace=ws,
                            events=lm_events, stream=stream)
        cdv.accept_longest(kout["cand"], kout["cand_len"], kout["copy_gate"], am, s.W, s.D,
                           out=aout, stream=stream)

    print(f"[bench] workload={s.name} B={B} n={np.diff(wl.cu_len).tolist()[:4]} V={s.V} "
          f"warmup={a.warmup} steps={a.steps}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    lm_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(a.steps)]
    # torch creates an event on its first record(): record each pair once here, outside
    # the timed region, so that the library can record the handles around the kernel
    for e0, e1 in lm_ev:
        e0.record(stream)
        e1.record(stream)
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(a.steps):
        step(lm_ev[i], i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_begin.elapsed_time(t_end) / a.steps
    lm_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in lm_ev]))
    gate = kout["copy_gate"].cpu().numpy().astype(bool)
    cl = kout["cand_len"].cpu().numpy()
    sum_L = int(cl[gate].sum())
    R_tot = int(gate.sum()) + sum_L
    print(f"[bench] {ms:.4f} ms/step, lm-head kernel {lm_ms:.4f} ms, gates={int(gate.sum())} "
          f"sumL={sum_L}", file=sys.stderr, flush=True)

    lm_bytes, lm_flops = lm_algorithmic(s, R_tot)
    # the contraction runs over every row of the batch (B*R), padded rows included;
    # the algorithmic figures count real rows only
    achieved = lm_bytes / (lm_ms * 1e-3) / 1e9
    tflops = lm_flops / (lm_ms * 1e-3) / 1e12
    mfma_peak = MFMA_BF16_PEAK_TFS if s.dtype == "bf16" else FP32_PEAK_TFS
    hbm_time = lm_bytes / (HBM_PEAK_GBS * 1e9)
    mfma_time = lm_flops / (mfma_peak * 1e12)
    if hbm_time >= mfma_time:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(tflops / mfma_peak, 4)}
    # the committed counters were taken on the workload's own full anchors and W, D
    from workloads import spec as base_spec
    b0 = base_spec(s.name)
    same = (s.anchor, s.W, s.D) == (b0.anchor, b0.W, b0.D)
    roof.update({"traffic": measured_traffic(s.name, SAMPLE_TRAFFIC_FILE if T > 0 else TRAFFIC_FILE)
                 if same else None,
                 "kernel": ("lmhead_bf16_kernel" if s.dtype == "bf16" else "lmhead_f32_kernel") +
                           ("<sample>" if T > 0 else ""),
                 "kernel_ms": round(lm_ms, 4), "algorithmic_bytes": int(lm_bytes),
                 "algorithmic_flops": lm_flops, "mfma_tflops": round(tflops, 1)})

    cpu = None
    if not a.no_cpu_baseline and T == 0:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, a.cpu_budget_s)

    line = {
        "metric": "copy-steps/sec & verified cand tokens/sec @8B shape; % HBM/MFMA peak",
        "value": round(B / (ms * 1e-3), 2),
        "unit": "copy-steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": s.name, "anchor": s.anchor, "B": B, "n": [int(x) for x in np.diff(wl.cu_len)[:4]],
                   "hid": s.hid, "Hq": s.Hq, "Hkv": s.Hkv, "d": s.d, "V": s.V, "kappa": s.kappa,
                   "W": s.W, "D": s.D, "tau": s.tau, "temperature": T, "parallelism": "single-gpu"},
        "verified_cand_tokens_per_s": round(sum_L / (ms * 1e-3), 1),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
