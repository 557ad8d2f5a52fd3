"""Seeded synthetic inputs for the HSTU attention hot path.

This module is shared by the tests, the benchmark and the oracle checks.  It
draws random numbers and lays them out; it holds none of the method's
arithmetic (no bucketing, masking, activation, normalisation or products).

Every workload mirrors one of the five configurations the path is measured
on (sizes, distributions, bucket counts, scale).  Draw order inside one
generator is fixed: lengths -> stochastic-length subsets -> timestamps ->
Q, K, V, U (or X, W1, W2) -> relative-bias tables -> score vector.

Values called bf16 are float32 arrays whose values are exactly representable
in bfloat16 (rounded to nearest even); ``bf16_bits`` gives their 16-bit
patterns for upload.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

__all__ = [
    "AttnInputs", "LayerInputs", "bf16_round", "bf16_bits", "bits_to_f32",
    "make_attn", "make_layer_stack", "config", "CONFIG_NAMES",
    "sl_subsample", "TS_EPOCH",
]

# Unix-seconds origin for synthetic timestamps: realistic int64 magnitudes.
TS_EPOCH = 1_700_000_000


# ----------------------------------------------------------------------------
# bfloat16 storage helpers (round-to-nearest-even), used only to *store* inputs
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bfloat16 bit patterns, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 value (kept as float32)."""
    return bits_to_f32(bf16_bits(x))


# ----------------------------------------------------------------------------
# Containers
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class AttnInputs:
    """One jagged batch for the attention core (and its LN*U epilogue).

    Layout: q/k/v/u are [T, H, d] float32 (bf16-representable when
    dtype == "bf16"); token t of sequence b lives at row offsets[b] + t.
    ``lengths`` (optional) allows padded layouts: rows
    offsets[b]+lengths[b] .. offsets[b+1]-1 are padding.
    ``num_candidates`` (optional) marks the last c_b rows of sequence b as
    ranking candidates (M-FALCON layout).
    """
    B: int
    H: int
    d: int
    offsets: np.ndarray            # int32 [B+1]
    q: np.ndarray                  # float32 [T, H, d]
    k: np.ndarray
    v: np.ndarray
    u: np.ndarray
    ts: np.ndarray                 # int64 [T]
    rab_pos: np.ndarray            # float32 [P] (or [H, P])
    rab_time: np.ndarray           # float32 [NT] (or [H, NT])
    alpha: float
    dtype: str                     # "f32" | "bf16"
    lengths: Optional[np.ndarray] = None         # int32 [B]
    num_candidates: Optional[np.ndarray] = None  # int32 [B]
    w: Optional[np.ndarray] = None               # float32 [H*d] score vector
    eps: float = 1e-5
    name: str = ""

    @property
    def T(self) -> int:
        return int(self.offsets[-1])

    @property
    def P(self) -> int:
        return int(self.rab_pos.shape[-1])

    @property
    def NT(self) -> int:
        return int(self.rab_time.shape[-1])

    def seq_lengths(self) -> np.ndarray:
        if self.lengths is not None:
            return self.lengths.astype(np.int64)
        return np.diff(self.offsets).astype(np.int64)


@dataclasses.dataclass
class LayerInputs:
    """Input of an HSTU layer stack (projection f1, attention, LN*U, f2)."""
    B: int
    H: int
    d: int
    D: int
    offsets: np.ndarray            # int32 [B+1]
    x: np.ndarray                  # float32 [T, D] (bf16-representable)
    w1: List[np.ndarray]           # per layer float32 [4*H*d, D]  (out x in)
    w2: List[np.ndarray]           # per layer float32 [D, H*d]    (out x in)
    ts: np.ndarray                 # int64 [T]
    rab_pos: List[np.ndarray]      # per layer float32 [P]
    rab_time: List[np.ndarray]     # per layer float32 [NT]
    alpha: float
    eps: float = 1e-5
    name: str = ""

    @property
    def T(self) -> int:
        return int(self.offsets[-1])

    @property
    def layers(self) -> int:
        return len(self.w1)


# ----------------------------------------------------------------------------
# Primitive draws
# ----------------------------------------------------------------------------
def _timestamps(rng: np.random.Generator, n: int, mean_gap: float) -> np.ndarray:
    """Strictly increasing int64 seconds; gaps max(1, round(Exp(mean_gap)))."""
    t0 = TS_EPOCH + int(rng.integers(0, 10_000_000))
    gaps = np.maximum(1, np.rint(rng.exponential(mean_gap, size=n))).astype(np.int64)
    gaps[0] = 0
    return t0 + np.cumsum(gaps)


def sl_subsample(rng: np.random.Generator, length: int, cap: int) -> np.ndarray:
    """Stochastic-length subset: keep everything when length <= cap, else a
    uniformly random, order-preserving subset of ``cap`` indices."""
    if length <= cap:
        return np.arange(length, dtype=np.int64)
    idx = rng.choice(length, size=cap, replace=False)
    idx.sort()
    return idx.astype(np.int64)


def _normal(rng, shape, std, bf16: bool) -> np.ndarray:
    x = rng.normal(0.0, std, size=shape).astype(np.float32)
    return bf16_round(x) if bf16 else x


def upstream_grad(seed: int, shape, std: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """Seeded upstream gradient (dLoss/dO, dLoss/dY, or a stand-in forward
    output) of the given shape, N(0, std) rounded to bf16 for dtype bf16."""
    return _normal(np.random.default_rng(seed), shape, std, dtype == "bf16")


def _offsets(lengths) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.int32)
    off[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return off


def make_attn(seed: int, lengths, H: int, d: int, P: int, NT: int, alpha: float,
              dtype: str, *, qkv_std: float = 0.5, rab_std: float = 0.1,
              mean_gap: float = 60.0, num_candidates=None, sl_cap: Optional[int] = None,
              raw_lengths=None, with_w: bool = False, name: str = "") -> AttnInputs:
    """Generic jagged attention batch.

    ``lengths``: per-sequence token counts (after stochastic length when
    ``raw_lengths``/``sl_cap`` are given: then the raw sequences are drawn
    with ``raw_lengths`` events and subsampled to at most ``sl_cap``).
    ``num_candidates``: per-sequence candidate counts (M-FALCON); candidate
    timestamps repeat the last history timestamp.
    """
    rng = np.random.default_rng(seed)
    bf = dtype == "bf16"
    if raw_lengths is not None:
        subsets = [sl_subsample(rng, int(L), int(sl_cap)) for L in raw_lengths]
        lengths = [len(s) for s in subsets]
    else:
        subsets = None
    lengths = [int(x) for x in lengths]
    B = len(lengths)
    off = _offsets(lengths)
    T = int(off[-1])
    ts = np.empty(T, dtype=np.int64)
    for b in range(B):
        L = lengths[b]
        c = int(num_candidates[b]) if num_candidates is not None else 0
        n = L - c
        if subsets is not None:
            raw = _timestamps(rng, int(raw_lengths[b]), mean_gap)
            seq = raw[subsets[b]]
        else:
            hist = _timestamps(rng, n, mean_gap) if n > 0 else np.zeros(0, np.int64)
            last = hist[-1] if n > 0 else TS_EPOCH
            seq = np.concatenate([hist, np.full(c, last, dtype=np.int64)])
        ts[off[b]:off[b + 1]] = seq
    q = _normal(rng, (T, H, d), qkv_std, bf)
    k = _normal(rng, (T, H, d), qkv_std, bf)
    v = _normal(rng, (T, H, d), qkv_std, bf)
    u = _normal(rng, (T, H, d), qkv_std, bf)
    rab_pos = rng.normal(0.0, rab_std, size=P).astype(np.float32)
    rab_time = rng.normal(0.0, rab_std, size=NT).astype(np.float32)
    w = None
    if with_w:
        w = rng.normal(0.0, 1.0 / math.sqrt(H * d), size=H * d).astype(np.float32)
    nc = None if num_candidates is None else np.asarray(num_candidates, dtype=np.int32)
    return AttnInputs(B=B, H=H, d=d, offsets=off, q=q, k=k, v=v, u=u, ts=ts,
                      rab_pos=rab_pos, rab_time=rab_time, alpha=float(alpha),
                      dtype=dtype, num_candidates=nc, w=w, name=name)


@dataclasses.dataclass
class CachedSplit:
    """An M-FALCON batch cut into a history KV cache and candidate rows.

    ``hist_rows`` / ``cand_rows`` index the combined [history | candidates]
    layout of the source batch; the cache holds each user's history keys and
    values back to back (``hist_offsets``), the candidates theirs
    (``cand_offsets``).  ``ts`` is the combined layout's timestamps after the
    candidates' were redrawn (so the two layouts agree row for row)."""
    hist_offsets: np.ndarray   # int32 [B+1]
    cand_offsets: np.ndarray   # int32 [B+1]
    hist_rows: np.ndarray      # int64 [history rows]
    cand_rows: np.ndarray      # int64 [candidate rows]
    ts: np.ndarray             # int64 [T]


def split_cached(x: AttnInputs, seed: int, max_gap: int = 0) -> CachedSplit:
    """Cut ``x`` (built with ``num_candidates``) into cache and candidates.
    With ``max_gap`` > 0 every candidate's timestamp is redrawn as the user's
    last history timestamp plus a uniform gap in [0, max_gap] seconds (the
    request time of each candidate need not be the last event's)."""
    rng = np.random.default_rng(seed)
    nc = np.asarray(x.num_candidates, dtype=np.int64)
    L = np.diff(x.offsets.astype(np.int64))
    n = L - nc
    hist_rows = np.concatenate([np.arange(x.offsets[b], x.offsets[b] + n[b]) for b in range(x.B)]
                               + [np.zeros(0, np.int64)]).astype(np.int64)
    cand_rows = np.concatenate([np.arange(x.offsets[b] + n[b], x.offsets[b + 1]) for b in range(x.B)]
                               + [np.zeros(0, np.int64)]).astype(np.int64)
    ts = x.ts.copy()
    if max_gap > 0:
        for b in range(x.B):
            c0, c1 = int(x.offsets[b] + n[b]), int(x.offsets[b + 1])
            last = ts[c0 - 1] if n[b] > 0 else TS_EPOCH
            ts[c0:c1] = last + rng.integers(0, max_gap + 1, size=c1 - c0)
    return CachedSplit(hist_offsets=_offsets(n), cand_offsets=_offsets(nc), hist_rows=hist_rows,
                       cand_rows=cand_rows, ts=ts)


def make_layer_stack(seed: int, lengths, H: int, d: int, D: int, layers: int, P: int,
                     NT: int, alpha: float, *, x_std: float = 0.5, rab_std: float = 0.1,
                     mean_gap: float = 60.0, name: str = "") -> LayerInputs:
    """Jagged input X plus Xavier-uniform f1/f2 weights for ``layers`` layers."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    B = len(lengths)
    off = _offsets(lengths)
    T = int(off[-1])
    ts = np.empty(T, dtype=np.int64)
    for b in range(B):
        ts[off[b]:off[b + 1]] = _timestamps(rng, lengths[b], mean_gap)
    x = _normal(rng, (T, D), x_std, True)
    w1, w2 = [], []
    for _ in range(layers):
        a1 = math.sqrt(6.0 / (D + 4 * H * d))
        a2 = math.sqrt(6.0 / (H * d + D))
        w1.append(bf16_round(rng.uniform(-a1, a1, size=(4 * H * d, D)).astype(np.float32)))
        w2.append(bf16_round(rng.uniform(-a2, a2, size=(D, H * d)).astype(np.float32)))
    rp = [rng.normal(0.0, rab_std, size=P).astype(np.float32) for _ in range(layers)]
    rt = [rng.normal(0.0, rab_std, size=NT).astype(np.float32) for _ in range(layers)]
    return LayerInputs(B=B, H=H, d=d, D=D, offsets=off, x=x, w1=w1, w2=w2, ts=ts,
                       rab_pos=rp, rab_time=rt, alpha=float(alpha), name=name)


# ----------------------------------------------------------------------------
# The five measured workloads
# ----------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "hstu_attn_f32_b4_h2_d32",
    2: "hstu_attn_bf16_b64_l256-1024_h4_d128",
    3: "hstu_attn_bf16_longseq_b16_sl0.85_h8_d128",
    4: "mfalcon_bf16_b8_n2048_bm512_h4_d128",
    5: "hstu_stack_bf16_4layer_b32_l512-4096_D512_h4_d128",
}

# Stochastic-length cap of the long-sequence workload: floor(N ** 0.85) with
# N = 8192, the workload's maximum raw length (the scale 1/N uses the same N).
SL_EXPONENT = 0.85
SL_MAX_RAW = 8192
SL_CAP = int(math.floor(SL_MAX_RAW ** SL_EXPONENT))


def _lognormal_lengths(rng, B, median, sigma, lo, hi):
    raw = np.rint(rng.lognormal(math.log(median), sigma, size=B)).astype(np.int64)
    return np.clip(raw, lo, hi)


def longseq_raw_lengths(batch: int = 16, seed: int = 3) -> np.ndarray:
    """Raw (before stochastic length) lengths of the long-sequence workload:
    the same draws ``config(3)`` makes."""
    rng = np.random.default_rng(1000 + seed)
    return _lognormal_lengths(rng, batch, 3000, 0.5, 1024, SL_MAX_RAW)


def config(n: int, *, batch: Optional[int] = None, max_len: Optional[int] = None,
           seed: Optional[int] = None):
    """Inputs of workload ``n`` (1..5), seeded with ``n`` unless ``seed`` is given.

    ``batch``/``max_len`` shrink the workload for parity tests at sizes the
    oracle finishes in seconds; every other parameter is unchanged.
    """
    s = n if seed is None else seed
    rng = np.random.default_rng(1000 + s)   # length draws only
    if n == 1:
        B = batch or 4
        hi = max_len or 64
        lengths = rng.integers(8, hi + 1, size=B)
        return make_attn(s, lengths, H=2, d=32, P=128, NT=32, alpha=1.0 / 64,
                         dtype="f32", name=CONFIG_NAMES[1])
    if n == 2:
        B = batch or 64
        hi = max_len or 1024
        lo = min(256, hi)
        lengths = rng.integers(lo, hi + 1, size=B)
        return make_attn(s, lengths, H=4, d=128, P=1024, NT=32, alpha=1.0 / 1024,
                         dtype="bf16", name=CONFIG_NAMES[2])
    if n == 3:
        B = batch or 16
        hi = max_len or SL_MAX_RAW
        raw = _lognormal_lengths(rng, B, 3000, 0.5, min(1024, hi), hi)
        cap = SL_CAP if max_len is None else int(math.floor(hi ** SL_EXPONENT))
        return make_attn(s, None, H=8, d=128, P=1024, NT=32, alpha=1.0 / SL_MAX_RAW,
                         dtype="bf16", raw_lengths=raw, sl_cap=cap, name=CONFIG_NAMES[3])
    if n == 4:
        B = batch or 8
        nh = max_len or 2048
        bm = 512 if max_len is None else max(1, nh // 4)
        lengths = [nh + bm] * B
        return make_attn(s, lengths, H=4, d=128, P=1024, NT=32, alpha=1.0 / (2048 + 512),
                         dtype="bf16", num_candidates=[bm] * B, with_w=True,
                         name=CONFIG_NAMES[4])
    if n == 5:
        B = batch or 32
        hi = max_len or 4096
        lo = min(512, hi)
        lengths = rng.integers(lo, hi + 1, size=B)
        return make_layer_stack(s, lengths, H=4, d=128, D=512, layers=4, P=1024, NT=32,
                                alpha=1.0 / 4096, name=CONFIG_NAMES[5])
    raise ValueError(f"unknown workload {n}")
