"""Seeded generators for the copy-speculation workloads (no method arithmetic).

Every array is drawn from numpy's PCG64 through a SeedSequence keyed by
(seed, tensor tag, sequence index), so any tensor of any workload can be
regenerated on its own.  Floating-point tensors are produced in float32 and,
for bfloat16 workloads, rounded once to bfloat16 (round to nearest even) and
stored as uint16 bit patterns: both the oracle and the GPU path then read the
very same bf16 values.

Token-id structure (per sequence of length n):
* base ids: Zipf(s) over vocabulary ranks 1..V, P(k) ~ k^-s, drawn by inverse
  CDF; id = k - 1.
* planted verbatim repeats: a destination span is overwritten with a copy of a
  source span lying wholly before it; destinations never overlap.  Positions
  inside destinations are "copy positions" (the paper's copy-mode label of §3.2
  needs runs of >= 5 tokens; planted spans are >= 5 long).
* anchor: the last position n-1.  In "full" anchor mode the sequence ends in a
  copy of a block that already occurs W+1 times earlier, so a full set of W
  candidates exists; in "natural" mode the anchor is inside a repeat only with
  the sequence's copy probability, and otherwise may end an accidental short
  repeat or no repeat at all.
"""
from dataclasses import dataclass, field, replace

import numpy as np

KAPPA, W_DEF, D_DEF, TAU_DEF = 5, 10, 20, 0.4


@dataclass(frozen=True)
class Spec:
    name: str
    B: int
    n: tuple                 # (lo, hi): n_b ~ U{lo..hi}
    hid: int
    Hq: int
    Hkv: int
    d: int
    V: int
    dtype: str               # "f32" or "bf16"
    zipf: float
    structure: str           # "planted3" | "spans" | "tiers" | "boilerplate"
    seed: int
    coverage: float = 0.0    # fraction of positions inside planted copies
    span: tuple = (5, 200)   # planted span lengths
    copies: tuple = (3, 10)  # boilerplate: occurrences per block
    short_frac: float = 0.0  # accidental 2..4-token repeats, fraction of positions
    anchor: str = "full"     # "full" | "natural"
    lm_std: float = 0.02     # LM-head weight std
    q_scale: float = 1.0     # query scale (4.0 concentrates the softmax)
    kappa: int = KAPPA
    W: int = W_DEF
    D: int = D_DEF
    tau: float = TAU_DEF
    tiers: tuple = ()        # ((prob, coverage), ...) per-sequence copy tiers


CONFIGS = {
    # tiny single sequence, fp32, three planted repeats ending at the query
    "tiny": Spec("tiny", 1, (512, 512), 64, 1, 1, 64, 1000, "f32", 1.1, "planted3", 1001),
    # Llama-3.1-8B-shaped verify, batch 1, context 4096, 10.6 % of positions copied
    "llama8b_b1": Spec("llama8b_b1", 1, (4096, 4096), 4096, 32, 8, 128, 128256, "bf16", 1.1,
                       "spans", 1002, coverage=0.106),
    # same shape, batch 32 ragged contexts, heavy/medium/light copy tiers + short repeats
    "llama8b_b32": Spec("llama8b_b32", 32, (1024, 8192), 4096, 32, 8, 128, 128256, "bf16", 1.1,
                        "tiers", 1003, short_frac=0.05,
                        tiers=((0.106, 0.40), (0.117, 0.15), (0.777, 0.02))),
    # Qwen3-8B-shaped verify, batch 8, context 16384, boilerplate blocks repeated 3..10x
    "qwen3_8b_b8": Spec("qwen3_8b_b8", 8, (16384, 16384), 4096, 32, 8, 128, 151936, "bf16", 1.05,
                        "boilerplate", 1004, coverage=0.25, span=(5, 500), anchor="natural"),
    # Llama-3.3-70B-shaped single-layer share, batch 4, context 32768, 8.9 % copied
    "llama70b_b4": Spec("llama70b_b4", 4, (32768, 32768), 8192, 64, 8, 128, 128256, "bf16", 1.1,
                        "spans", 1005, coverage=0.089),
    # small parity shapes: several tiles and ragged tails, oracle finishes in seconds
    "small_bf16": Spec("small_bf16", 3, (300, 1100), 512, 4, 2, 128, 3001, "bf16", 1.1,
                       "spans", 2001, coverage=0.15),
    "small_f32": Spec("small_f32", 2, (200, 700), 128, 2, 1, 64, 1537, "f32", 1.1,
                      "spans", 2002, coverage=0.15),
}


def spec(name, **overrides):
    s = CONFIGS[name]
    return replace(s, **overrides) if overrides else s


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _rng(seed, *tags):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tags])))


_TAGS = {"ids": 1, "n": 2, "h": 3, "w": 4, "q": 5, "kp": 6, "vp": 7, "kc": 8, "vc": 9,
         "lm": 10, "tier": 11}


def _normal(seed, tag, shape, std, dtype, sub=0, chunk=1 << 26):
    """N(0, std^2) tensor in float32 (or bf16 bits), drawn in fixed chunks."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.float32 if dtype == "f32" else np.uint16)
    rng = _rng(seed, _TAGS[tag], sub)
    for s0 in range(0, total, chunk):
        e = min(total, s0 + chunk)
        x = rng.standard_normal(e - s0, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s0:e] = x if dtype == "f32" else f32_to_bf16_bits(x)
    return out.reshape(shape)


class _Ctx:
    """Token-id canvas of one sequence with a non-overlap mask for destinations."""

    def __init__(self, rng, n, V, zipf):
        self.rng, self.n = rng, n
        ranks = np.arange(1, V + 1, dtype=np.float64)
        cdf = np.cumsum(ranks ** (-zipf))
        cdf /= cdf[-1]
        u = rng.random(n)
        self.x = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int32)
        self.busy = np.zeros(n, dtype=bool)     # destinations and protected sources
        self.copy = np.zeros(n, dtype=bool)     # copy-position labels (>= 5-token copies)
        self.V = V

    def place(self, dst, src, length, label=True):
        self.x[dst:dst + length] = self.x[src:src + length]
        self.busy[dst:dst + length] = True
        if label:
            self.copy[dst:dst + length] = True

    def free(self, a, length):
        return a >= 0 and a + length <= self.n and not self.busy[a:a + length].any()

    def random_spans(self, lo, hi, target, end_limit, label=True, tries=20000):
        """Plant copies of random earlier spans until `target` positions are covered."""
        covered = 0
        rng = self.rng
        for _ in range(tries):
            if covered >= target:
                break
            L = int(rng.integers(lo, hi + 1))
            if end_limit - L <= L:
                continue
            dst = int(rng.integers(L, end_limit - L + 1))
            if not self.free(dst, L):
                continue
            src = int(rng.integers(0, dst - L + 1))
            self.place(dst, src, L, label)
            covered += L
        return covered


def _full_anchor(ctx, W, D, kappa, ls_cap=40):
    """End the sequence in a copy of a block that occurs W+1 times earlier."""
    n, rng = ctx.n, ctx.rng
    ls_max = max(kappa + 4, min(ls_cap, n // (2 * (W + 3))))
    ls_min = min(kappa + 8, ls_max)
    Ls = int(rng.integers(ls_min, ls_max + 1))
    m = int(rng.integers(kappa + 2, Ls)) if Ls > kappa + 2 else Ls   # anchor copies S[0..m)
    end_limit = n - m
    # source block S
    for _ in range(1000):
        s0 = int(rng.integers(0, max(1, end_limit // (W + 2))))
        if ctx.free(s0, Ls):
            break
    ctx.busy[s0:s0 + Ls] = True
    placed = 0
    for _ in range(20000):
        if placed == W:
            break
        dst = int(rng.integers(s0 + Ls, end_limit - Ls + 1))
        if ctx.free(dst, Ls):
            ctx.place(dst, s0, Ls)
            placed += 1
    ctx.place(n - m, s0, m)
    return m


def _natural_anchor(ctx, p_copy, kappa, lo, hi):
    """Anchor inside a repeat with probability p_copy, else maybe a short repeat."""
    n, rng = ctx.n, ctx.rng
    u = rng.random()
    if u < p_copy:
        L = int(rng.integers(max(lo, kappa + 1), max(lo, kappa + 1) + 40))
        L = min(L, n // 4)
        src = int(rng.integers(0, n - 2 * L))
        ctx.place(n - L, src, L)
    elif u < p_copy + 0.05:
        L = int(rng.integers(2, 5))
        src = int(rng.integers(0, n - 2 * L))
        ctx.place(n - L, src, L, label=False)
        return
    ctx.busy[n - 1] = True


@dataclass
class Workload:
    spec: Spec
    ids: np.ndarray          # [sum n] int32
    cu_len: np.ndarray       # [B+1] int32
    copy_pos: np.ndarray     # [sum n] bool, planted copy destinations
    h: np.ndarray            # [B, hid] float32 or bf16 bits
    w: np.ndarray            # [hid] float32
    q: np.ndarray            # [B, R, Hq, d]
    k_pre: np.ndarray        # [sum n, Hkv, d]
    v_pre: np.ndarray
    k_cand: np.ndarray       # [B, W*D, Hkv, d]
    v_cand: np.ndarray
    lm_head: np.ndarray      # [V, hid]
    extra: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.spec.B

    @property
    def R(self):
        return 1 + self.spec.W * self.spec.D

    @property
    def max_n(self):
        return int(np.max(np.diff(self.cu_len)))

    @property
    def scale(self):
        return float(1.0 / np.sqrt(self.spec.d))


def _sequence_ids(s, b, n):
    rng = _rng(s.seed, _TAGS["ids"], b)
    ctx = _Ctx(rng, n, s.V, s.zipf)
    W, D, kappa = s.W, s.D, s.kappa
    if s.structure == "planted3":
        Ls = int(rng.integers(8, 31))
        s0 = int(rng.integers(0, n // 8))
        ctx.busy[s0:s0 + Ls] = True
        ctx.place(n - Ls, s0, Ls)
        placed = 0
        while placed < 2:
            dst = int(rng.integers(s0 + Ls, n - 2 * Ls))
            if ctx.free(dst, Ls):
                ctx.place(dst, s0, Ls)
                placed += 1
        return ctx
    if s.structure == "spans":
        if s.anchor == "full":
            _full_anchor(ctx, W, D, kappa)
        else:
            _natural_anchor(ctx, s.coverage, kappa, *s.span)
        have = int(ctx.copy.sum())
        ctx.random_spans(s.span[0], s.span[1], int(s.coverage * n) - have, n - 1)
        return ctx
    if s.structure == "tiers":
        u = _rng(s.seed, _TAGS["tier"], b).random()
        acc = 0.0
        cov = s.tiers[-1][1]
        for p, c in s.tiers:
            acc += p
            if u < acc:
                cov = c
                break
        if s.anchor == "full":
            _full_anchor(ctx, W, D, kappa)
        else:
            _natural_anchor(ctx, cov, kappa, *s.span)
        have = int(ctx.copy.sum())
        ctx.random_spans(s.span[0], s.span[1], int(cov * n) - have, n - 1)
        ctx.random_spans(2, 4, int(s.short_frac * n), n - 1, label=False)
        return ctx
    if s.structure == "boilerplate":
        # the anchor ends inside the last occurrence of a repeated block
        Lb = int(rng.integers(max(s.span[0], kappa + 3), min(s.span[1], n // 40) + 1))
        k = int(rng.integers(s.copies[0], s.copies[1] + 1))
        t = int(rng.integers(kappa, Lb))            # anchor offset inside the last copy
        s0 = int(rng.integers(0, n // (2 * k)))
        ctx.busy[s0:s0 + Lb] = True
        placed = 1
        for _ in range(20000):
            if placed == k - 1:
                break
            dst = int(rng.integers(s0 + Lb, n - t - Lb))
            if ctx.free(dst, Lb):
                ctx.place(dst, s0, Lb)
                placed += 1
        ctx.place(n - t, s0, t)
        covered = int(ctx.copy.sum())
        target = int(s.coverage * n)
        for _ in range(20000):
            if covered >= target:
                break
            L = int(rng.integers(s.span[0], s.span[1] + 1))
            reps = int(rng.integers(s.copies[0], s.copies[1] + 1))
            src = int(rng.integers(0, n - 2 * L))
            if not ctx.free(src, L):
                continue
            ctx.busy[src:src + L] = True
            for _ in range(reps - 1):
                for _ in range(50):
                    dst = int(rng.integers(src + L, max(src + L + 1, n - 1 - L)))
                    if ctx.free(dst, L):
                        ctx.place(dst, src, L)
                        covered += L
                        break
        return ctx
    raise ValueError(s.structure)


def generate(name_or_spec, with_tensors=True, **overrides):
    """Build the workload.  with_tensors=False draws ids/h/w only (integer-stage tests)."""
    s = name_or_spec if isinstance(name_or_spec, Spec) else spec(name_or_spec, **overrides)
    if isinstance(name_or_spec, Spec) and overrides:
        s = replace(s, **overrides)
    nrng = _rng(s.seed, _TAGS["n"])
    ns = [int(nrng.integers(s.n[0], s.n[1] + 1)) for _ in range(s.B)]
    ctxs = [_sequence_ids(s, b, ns[b]) for b in range(s.B)]
    ids = np.concatenate([c.x for c in ctxs]).astype(np.int32)
    copy_pos = np.concatenate([c.copy for c in ctxs])
    cu = np.zeros(s.B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ns)
    # probe vector w ~ N(0, 1/hid); anchor state h ~ N(0, I) + 3 w/|w| at copy positions
    w = _rng(s.seed, _TAGS["w"]).standard_normal(s.hid, dtype=np.float32) / np.float32(np.sqrt(s.hid))
    hs = []
    for b in range(s.B):
        hb = _rng(s.seed, _TAGS["h"], b).standard_normal(s.hid, dtype=np.float32)
        if ctxs[b].copy[-1]:
            hb = hb + np.float32(3.0) * w / np.float32(np.linalg.norm(w))
        hs.append(hb.astype(np.float32))
    h = np.stack(hs)
    if s.dtype == "bf16":
        h = f32_to_bf16_bits(h)
    R = 1 + s.W * s.D
    N = int(cu[-1])
    t = {}
    if with_tensors:
        t["q"] = _normal(s.seed, "q", (s.B, R, s.Hq, s.d), s.q_scale, s.dtype)
        t["k_pre"] = _normal(s.seed, "kp", (N, s.Hkv, s.d), 1.0, s.dtype)
        t["v_pre"] = _normal(s.seed, "vp", (N, s.Hkv, s.d), 1.0, s.dtype)
        t["k_cand"] = _normal(s.seed, "kc", (s.B, s.W * s.D, s.Hkv, s.d), 1.0, s.dtype)
        t["v_cand"] = _normal(s.seed, "vc", (s.B, s.W * s.D, s.Hkv, s.d), 1.0, s.dtype)
        t["lm_head"] = _normal(s.seed, "lm", (s.V, s.hid), s.lm_std, s.dtype)
    else:
        t = {k: None for k in ("q", "k_pre", "v_pre", "k_cand", "v_cand", "lm_head")}
    return Workload(s, ids, cu, copy_pos, h, w, **t)


def device_tensors(wl, device="cuda"):
    """The float tensors of workload `wl` (q, k_pre, v_pre, k_cand, v_cand, lm_head)
    drawn on `device` by torch's generator seeded with the workload's seed, with the
    laws `generate` uses: N(0, q_scale^2) queries, N(0, 1) keys and values,
    N(0, lm_std^2) LM-head weights, in float32 and rounded once to bfloat16 for bf16
    workloads.  Same shapes and laws as the host draws, not the same values: for
    timing runs whose host generation would take longer than the measurement."""
    import torch
    s = wl.spec
    g = torch.Generator(device=device)
    g.manual_seed(s.seed)
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    R, N = 1 + s.W * s.D, int(wl.cu_len[-1])

    def draw(shape, std):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        return x.to(dt)

    return {"q": draw((s.B, R, s.Hq, s.d), s.q_scale),
            "k_pre": draw((N, s.Hkv, s.d), 1.0), "v_pre": draw((N, s.Hkv, s.d), 1.0),
            "k_cand": draw((s.B, s.W * s.D, s.Hkv, s.d), 1.0),
            "v_cand": draw((s.B, s.W * s.D, s.Hkv, s.d), 1.0),
            "lm_head": draw((s.V, s.hid), s.lm_std)}


def to_torch(arr, device):
    """numpy -> torch on `device`; uint16 arrays are reinterpreted as bfloat16."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.bool_:
        return torch.from_numpy(a.astype(np.uint8)).to(device)
    return torch.from_numpy(a).to(device)


def generate_with_ids(s, id_lists, anchor_copy=None):
    """Workload whose contexts are given explicitly (edge cases); float tensors are
    drawn as in `generate`.  anchor_copy[b] marks the anchor as a copy position."""
    B = len(id_lists)
    s = replace(s, B=B)
    ns = [len(x) for x in id_lists]
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ns)
    ids = np.concatenate([np.asarray(x, dtype=np.int32) for x in id_lists])
    copy_pos = np.zeros(len(ids), dtype=bool)
    w = _rng(s.seed, _TAGS["w"]).standard_normal(s.hid, dtype=np.float32) / np.float32(np.sqrt(s.hid))
    hs = []
    for b in range(B):
        hb = _rng(s.seed, _TAGS["h"], b).standard_normal(s.hid, dtype=np.float32)
        if anchor_copy is None or anchor_copy[b]:
            hb = hb + np.float32(3.0) * w / np.float32(np.linalg.norm(w))
            copy_pos[cu[b + 1] - 1] = True
        hs.append(hb.astype(np.float32))
    h = np.stack(hs)
    if s.dtype == "bf16":
        h = f32_to_bf16_bits(h)
    R = 1 + s.W * s.D
    N = int(cu[-1])
    return Workload(s, ids, cu, copy_pos, h, w,
                    _normal(s.seed, "q", (B, R, s.Hq, s.d), s.q_scale, s.dtype),
                    _normal(s.seed, "kp", (N, s.Hkv, s.d), 1.0, s.dtype),
                    _normal(s.seed, "vp", (N, s.Hkv, s.d), 1.0, s.dtype),
                    _normal(s.seed, "kc", (B, s.W * s.D, s.Hkv, s.d), 1.0, s.dtype),
                    _normal(s.seed, "vc", (B, s.W * s.D, s.Hkv, s.d), 1.0, s.dtype),
                    _normal(s.seed, "lm", (s.V, s.hid), s.lm_std, s.dtype))


# ---------------------------------------------------------------- probe calibration
@dataclass(frozen=True)
class CalibSpec:
    name: str
    B: int                   # contexts
    n: tuple                 # (lo, hi): n_b ~ U{lo..hi}
    V: int
    zipf: float
    coverage: float          # fraction of positions inside planted copies (spans >= 5)
    span: tuple              # planted span lengths
    short_frac: float        # accidental 2..4-token repeats (not copies), fraction of positions
    L: int                   # layers
    hid: int
    dtype: str               # "f32" or "bf16"
    seed: int
    peak_layer: int          # layer where the planted copy signal is strongest
    sep_peak: float = 3.0    # planted shift along the layer's probe direction at the peak
    sep_floor: float = 0.3   # ... far from the peak
    width: float = 5.0       # layers over which the shift decays (Gaussian profile)


CALIB_CONFIGS = {
    # full-size: one Llama-3.1-8B-shaped context, 32 layers of 4096-wide states
    "calib_llama8b": CalibSpec("calib_llama8b", 1, (4096, 4096), 128256, 1.1, 0.106, (5, 200), 0.05,
                               32, 4096, "bf16", 3001, 14),
    # small parity shapes (ragged contexts, odd hidden size for the fp32 path)
    "calib_small_bf16": CalibSpec("calib_small_bf16", 3, (300, 900), 400, 1.1, 0.15, (5, 60), 0.05,
                                  6, 512, "bf16", 3002, 3),
    "calib_small_f32": CalibSpec("calib_small_f32", 2, (200, 700), 300, 1.1, 0.15, (5, 60), 0.05,
                                 5, 200, "f32", 3003, 2),
}


@dataclass
class CalibWorkload:
    spec: CalibSpec
    ids: np.ndarray          # [sum n] int32
    cu_len: np.ndarray       # [B+1] int32
    copy_pos: np.ndarray     # [sum n] bool: destinations of the planted copies
    H: np.ndarray            # [L, sum n, hid] float32 or bf16 bits: per-layer states
    w: np.ndarray            # [L, hid] float32: per-layer probe vectors


def generate_calibration(name, **overrides):
    """Contexts with planted verbatim copies (>= 5 tokens) and accidental short repeats, and
    per-layer states h = N(0, I) + sep_l * w_l / |w_l| at the planted copy positions, with
    sep_l peaking at peak_layer.  The copy signal comes from the planted positions, not
    from any labelling rule."""
    s = CALIB_CONFIGS[name]
    if overrides:
        s = replace(s, **overrides)
    nrng = _rng(s.seed, _TAGS["n"])
    ns = [int(nrng.integers(s.n[0], s.n[1] + 1)) for _ in range(s.B)]
    ids, copy = [], []
    for b in range(s.B):
        ctx = _Ctx(_rng(s.seed, _TAGS["ids"], b), ns[b], s.V, s.zipf)
        ctx.random_spans(s.span[0], s.span[1], int(s.coverage * ns[b]), ns[b])
        ctx.random_spans(2, 4, int(s.short_frac * ns[b]), ns[b], label=False)
        ids.append(ctx.x)
        copy.append(ctx.copy)
    ids = np.concatenate(ids).astype(np.int32)
    copy_pos = np.concatenate(copy)
    cu = np.zeros(s.B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ns)
    N = int(cu[-1])
    w = np.empty((s.L, s.hid), np.float32)
    H = np.empty((s.L, N, s.hid), np.float32 if s.dtype == "f32" else np.uint16)
    rows = np.nonzero(copy_pos)[0]
    for l in range(s.L):
        wl = _rng(s.seed, _TAGS["w"], l).standard_normal(s.hid, dtype=np.float32) / np.float32(np.sqrt(s.hid))
        w[l] = wl
        sep = s.sep_floor + (s.sep_peak - s.sep_floor) * float(np.exp(-((l - s.peak_layer) / s.width) ** 2))
        u = (wl / np.linalg.norm(wl)).astype(np.float32) * np.float32(sep)
        rng = _rng(s.seed, _TAGS["h"], l)
        step = max(1, (1 << 24) // s.hid)
        for r0 in range(0, N, step):
            r1 = min(N, r0 + step)
            x = rng.standard_normal((r1 - r0, s.hid), dtype=np.float32)
            sel = rows[(rows >= r0) & (rows < r1)] - r0
            x[sel] += u
            H[l, r0:r1] = x if s.dtype == "f32" else f32_to_bf16_bits(x)
    return CalibWorkload(s, ids, cu, copy_pos, H, w)


# ---------------------------------------------------------------- multi-layer forward
FWD_CONFIGS = {
    # parity shape: the small bf16 contexts, hid 512 (4 q heads, 2 kv heads of 128), 2 layers
    "fwd_small": ("small_bf16", {"V": 3001}, 1024, 2),
    # Llama-3.1-8B shape (hid 4096, 32 / 8 heads, MLP 14336, vocabulary 128256), batch 1
    "fwd_llama8b": ("llama8b_b1", {}, 14336, 2),
}


@dataclass
class FwdWorkload:
    spec: Spec
    inter: int
    ids: np.ndarray
    cu_len: np.ndarray
    embed: np.ndarray        # [V, hid] bf16 bits
    layers: list             # dicts of bf16-bit arrays: attn_norm, wqkv, wo, mlp_norm, w_gate,
                             # w_up, w_down, k_cache, v_cache
    final_norm: np.ndarray
    lm_head: np.ndarray


def generate_forward(name, n_layers=None, **overrides):
    """Contexts of the named copy-step workload and synthetic Llama-family weights:
    norms 1 + N(0, 0.1^2), projections N(0, 1/fan_in), embeddings N(0, 1), prefix
    caches N(0, 1), LM head N(0, 1/hid)."""
    base, over, inter, L = FWD_CONFIGS[name]
    over = dict(over)
    over.update(overrides)
    s = spec(base, **over)
    L = L if n_layers is None else n_layers
    wl = generate(s, with_tensors=False)
    hid, Hq, Hkv, d = s.hid, s.Hq, s.Hkv, s.d
    N = int(wl.cu_len[-1])
    seed = s.seed + 7000

    def norm_w(tag, sub):
        return f32_to_bf16_bits(1.0 + 0.1 * _rng(seed, 40 + tag, sub).standard_normal(hid, dtype=np.float32))

    layers = []
    for l in range(L):
        layers.append({
            "attn_norm": norm_w(1, l),
            "wqkv": _normal(seed, "q", ((Hq + 2 * Hkv) * d, hid), 1.0 / np.sqrt(hid), "bf16", sub=100 + l),
            "wo": _normal(seed, "kp", (hid, Hq * d), 1.0 / np.sqrt(Hq * d), "bf16", sub=100 + l),
            "mlp_norm": norm_w(2, l),
            "w_gate": _normal(seed, "vp", (inter, hid), 1.0 / np.sqrt(hid), "bf16", sub=100 + l),
            "w_up": _normal(seed, "kc", (inter, hid), 1.0 / np.sqrt(hid), "bf16", sub=100 + l),
            "w_down": _normal(seed, "vc", (hid, inter), 1.0 / np.sqrt(inter), "bf16", sub=100 + l),
            "k_cache": _normal(seed, "kp", (N, Hkv, d), 1.0, "bf16", sub=200 + l),
            "v_cache": _normal(seed, "vp", (N, Hkv, d), 1.0, "bf16", sub=200 + l),
        })
    return FwdWorkload(s, inter, wl.ids, wl.cu_len,
                       _normal(seed, "lm", (s.V, hid), 1.0, "bf16", sub=1),
                       layers, norm_w(3, 0),
                       _normal(seed, "lm", (s.V, hid), 1.0 / np.sqrt(hid), "bf16", sub=2))


# ---------------------------------------------------------------- large-array kappa-gram scan
# Many long contexts of Zipf ids, scanned whole: the retrieval step's throughput
# regime.  The contexts have no planted repeats, so the anchor's kappa-gram almost
# never occurs earlier and every scan reads its whole context (the case in which
# the probe fires but the dual gate closes).
SCAN_SIZES = (1 << 24, 1 << 26, 1 << 28)   # ids per launch
SCAN_N = 16384                             # ids per context
SCAN_V, SCAN_ZIPF, SCAN_SEED = 128256, 1.1, 4001


def _zipf_cdf(V, zipf):
    ranks = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-zipf))
    return cdf / cdf[-1]


def scan_ids_device(total, n=SCAN_N, V=SCAN_V, zipf=SCAN_ZIPF, seed=SCAN_SEED, device="cuda"):
    """`total` Zipf(zipf) ids over V ranks, drawn on `device` by torch's seeded
    generator (inverse CDF, as in the host generator), as total / n contexts of
    n ids.  Returns (ids int32 [total], cu_len int32 [total / n + 1])."""
    import torch
    assert total % n == 0
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    cdf = torch.from_numpy(_zipf_cdf(V, zipf).astype(np.float32)).to(device)
    ids = torch.empty(total, dtype=torch.int32, device=device)
    step = 1 << 26
    for s0 in range(0, total, step):
        e = min(total, s0 + step)
        u = torch.rand(e - s0, generator=g, device=device, dtype=torch.float32)
        ids[s0:e] = torch.searchsorted(cdf, u, right=True, out_int32=True).clamp_(max=V - 1)
    B = total // n
    cu = torch.arange(0, B + 1, dtype=torch.int32, device=device) * n
    return ids, cu


def scan_ids_planted(ns, kappa=KAPPA, V=SCAN_V, zipf=SCAN_ZIPF, seed=SCAN_SEED, max_occ=14,
                     boundary=8192):
    """Host contexts for scan parity: one context of Zipf ids per length in `ns`,
    in which the anchor's kappa-gram is copied to 0..max_occ earlier end
    positions, spread over the whole context, some placed right at or across
    multiples of `boundary` (powers of two are natural chunk boundaries for a
    scan).  Returns (ids int32 [sum(ns)], cu_len int32 [len(ns) + 1])."""
    cdf = _zipf_cdf(V, zipf)
    out = []
    for b, n in enumerate(ns):
        rng = _rng(seed, 13, b)
        x = np.minimum(np.searchsorted(cdf, rng.random(n), side="right"), V - 1).astype(np.int32)
        suffix = x[n - kappa:].copy()
        occ = int(rng.integers(0, max_occ + 1)) if n >= 2 * kappa + 2 else 0
        ends = set()
        for _ in range(occ):
            if rng.random() < 0.3:   # near a power-of-two boundary
                p = (int(rng.integers(1, max(2, n // boundary + 1))) * boundary
                     + int(rng.integers(-kappa, kappa + 1)))
            else:
                p = int(rng.integers(kappa - 1, n - 1))
            if kappa - 1 <= p <= n - 2 - kappa:   # keep the suffix itself intact
                ends.add(p)
        for p in sorted(ends):
            x[p - kappa + 1:p + 1] = suffix
        out.append(x)
    cu = np.zeros(len(ns) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ns)
    return np.concatenate(out), cu
