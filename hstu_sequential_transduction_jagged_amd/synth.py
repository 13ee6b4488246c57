"""Seeded synthetic inputs for the HSTU workloads.

This module holds only input generation (random draws, rounding of the drawn
values to the storage dtype, jagged offsets).  It contains none of the layer's
arithmetic, so both the HIP path's tests/benchmark and the CPU oracle can take
their inputs from it.

Workloads (each a function below):
  attn_small   fp32 attention: B=4, n ~ U{16..128}, H=2, d=32, alpha=1/128
  layer_small  bf16 layer: D=256, H=4, d=64, B=32, n = clip(Zipf(1.5), 8, 1024)
  attn_long    bf16 attention: B=16, n = clip(rint(LogNormal(ln 2048, 1)), 256, 8192),
               H=8, d=64, alpha=1/8192, 256 position / 32 time buckets
  genrank      bf16 layer with ALiBi, tokens = item_emb + action_emb: B=64,
               n ~ U{512..4096}, D=512, H=8, d=64, item ids Zipf(1.1) over 1e6
  stack8       bf16 8-layer stack: D=512, H=8, d=64, B=128,
               n0 = clip(Zipf(1.2), 1, 4096), stochastic length to 1024 w.p. 0.5
  mfalcon      bf16 candidate scoring: attn_long's users and histories, 1024 candidates
               per user at the request time (last history event + Exp(mean 3600 s))

Value recipe: Q, K, V, X ~ N(0, 1); weights Xavier-uniform; bias tables
~ N(0, 0.02); timestamps = per-user base + floor(cumsum(Exp(mean 3600 s)));
embedding rows ~ N(0, 1/2) so that item + action ~ N(0, 1).
Draw order per workload: lengths, timestamps, activations, weights, tables.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BIAS_NONE, BIAS_RAB_PT, BIAS_ALIBI = 0, 1, 2


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 values that are exactly representable in bfloat16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty_like(a)
    u = a.reshape(-1).view(np.uint32)
    o = out.reshape(-1).view(np.uint32)
    step = 1 << 22
    for s in range(0, u.size, step):
        x = u[s:s + step]
        # add 0x7FFF plus the lowest kept bit, then clear the low half: nearest, ties to even.
        # In uint32 this wraps only for bit patterns of negative NaNs, which are reset below.
        r = (x >> 16) & 1
        r += 0x7FFF
        r += x
        r &= 0xFFFF0000
        o[s:s + step] = r
    out[np.isnan(a)] = np.nan
    return out


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else np.ascontiguousarray(a)


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off.astype(np.int32)


def _timestamps(rng, lengths, mean_gap=3600.0) -> np.ndarray:
    out = []
    for n in lengths:
        base = 1_600_000_000 + int(rng.integers(0, 100_000_000))
        gaps = rng.exponential(mean_gap, size=int(n))
        out.append(base + np.floor(np.cumsum(gaps)).astype(np.int64))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def _xavier(rng, fan_out, fan_in):
    a = math.sqrt(6.0 / (fan_in + fan_out))
    return rng.uniform(-a, a, size=(fan_out, fan_in)).astype(np.float32)


@dataclass
class BiasSpec:
    kind: int = BIAS_NONE
    w_pos: Optional[np.ndarray] = None    # fp32 [P] or [H, P]
    w_time: Optional[np.ndarray] = None   # fp32 [NT] or [H, NT]
    slopes: Optional[np.ndarray] = None   # fp32 [H] (ALiBi); None = library default


@dataclass
class AttnInputs:
    name: str
    seed: int
    dtype: str                 # "f32" or "bf16"
    B: int
    H: int
    dqk: int
    dv: int
    offsets: np.ndarray        # int32 [B+1]
    max_seqlen: int
    ts: Optional[np.ndarray]   # int64 [T]
    q: np.ndarray              # float32 [T, H, dqk] (exact in dtype)
    k: np.ndarray
    v: np.ndarray              # float32 [T, H, dv]
    bias: BiasSpec
    alpha: float
    out_scale: float = 1.0

    @property
    def T(self):
        return int(self.offsets[-1])


@dataclass
class LayerParams:
    w1: np.ndarray      # [2H(dqk+dv), D] (exact in dtype)
    b1: np.ndarray      # fp32 [2H(dqk+dv)]
    gamma: np.ndarray   # fp32 [H dv]
    beta: np.ndarray    # fp32 [H dv]
    w2: np.ndarray      # [D, H dv]
    b2: np.ndarray      # fp32 [D]
    bias: BiasSpec


@dataclass
class LayerInputs:
    name: str
    seed: int
    dtype: str
    B: int
    D: int
    H: int
    dqk: int
    dv: int
    offsets: np.ndarray
    max_seqlen: int
    ts: Optional[np.ndarray]
    x: np.ndarray                 # [T, D] (exact in dtype)
    layers: List[LayerParams]
    alpha: float
    residual: bool
    ln_eps: float = 1e-5
    # GenRank token construction (x = item_table[item_ids] + action_table[action_ids])
    item_ids: Optional[np.ndarray] = None
    action_ids: Optional[np.ndarray] = None
    item_table: Optional[np.ndarray] = None
    action_table: Optional[np.ndarray] = None

    @property
    def T(self):
        return int(self.offsets[-1])


def _tables(rng, P, NT, std, H=None):
    shape_p = (P,) if H is None else (H, P)
    shape_t = (NT,) if H is None else (H, NT)
    wp = (rng.standard_normal(shape_p) * std).astype(np.float32)
    wt = (rng.standard_normal(shape_t) * std).astype(np.float32)
    return wp, wt


def make_attn(name, seed, dtype, lengths, H, d, alpha, bias_kind=BIAS_RAB_PT, P=128, NT=32,
              table_std=0.02, per_head_tables=False, rng=None, max_seqlen=None, out_scale=1.0,
              qkv_std=1.0):
    """Attention-only inputs for given lengths (drawn values follow the recipe)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    offs = offsets_from_lengths(lengths)
    T = int(offs[-1])
    ts = _timestamps(rng, lengths)
    q = _store(rng.standard_normal((T, H, d), dtype=np.float32) * qkv_std, dtype)
    k = _store(rng.standard_normal((T, H, d), dtype=np.float32) * qkv_std, dtype)
    v = _store(rng.standard_normal((T, H, d), dtype=np.float32) * qkv_std, dtype)
    bias = BiasSpec(kind=bias_kind)
    if bias_kind == BIAS_RAB_PT:
        bias.w_pos, bias.w_time = _tables(rng, P, NT, table_std, H if per_head_tables else None)
    ms = int(lengths.max()) if max_seqlen is None and len(lengths) else int(max_seqlen or 0)
    return AttnInputs(name, seed, dtype, len(lengths), H, d, d, offs, ms, ts, q, k, v, bias,
                      float(alpha), out_scale)


def attn_small(seed=1000, B=4, **kw):
    """fp32 attention, B=4 users, n ~ U{16..128}, H=2, d=32, alpha=1/128."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(16, 129, size=B)
    return make_attn("attn_small", seed, "f32", lengths, H=2, d=32, alpha=1.0 / 128, P=128,
                     NT=32, rng=rng, **kw)


def lognormal_lengths(rng, B, median=2048, sigma=1.0, lo=256, hi=8192):
    return np.clip(np.rint(rng.lognormal(math.log(median), sigma, size=B)), lo, hi).astype(np.int64)


def attn_long(seed=1002, B=16, lo=256, hi=8192, **kw):
    """bf16 attention, B=16 users, lognormal lengths (median 2048) clipped to
    [256, 8192], H=8, d=64, alpha=1/8192, 256 position and 32 time buckets."""
    rng = np.random.default_rng(seed)
    lengths = lognormal_lengths(rng, B, lo=lo, hi=hi)
    kw.setdefault("alpha", 1.0 / 8192)
    return make_attn("attn_long", seed, "bf16", lengths, H=8, d=64, P=256, NT=32, rng=rng, **kw)


def _layer_params(rng, dtype, D, H, dqk, dv, bias_kind, P, NT, table_std, randomize_affine):
    N1 = 2 * H * (dqk + dv)
    HV = H * dv
    w1 = _store(_xavier(rng, N1, D), dtype)
    w2 = _store(_xavier(rng, D, HV), dtype)
    if randomize_affine:
        b1 = (rng.standard_normal(N1) * 0.1).astype(np.float32)
        b2 = (rng.standard_normal(D) * 0.1).astype(np.float32)
        gamma = (1.0 + rng.standard_normal(HV) * 0.1).astype(np.float32)
        beta = (rng.standard_normal(HV) * 0.1).astype(np.float32)
    else:
        b1 = np.zeros(N1, np.float32)
        b2 = np.zeros(D, np.float32)
        gamma = np.ones(HV, np.float32)
        beta = np.zeros(HV, np.float32)
    bias = BiasSpec(kind=bias_kind)
    if bias_kind == BIAS_RAB_PT:
        bias.w_pos, bias.w_time = _tables(rng, P, NT, table_std)
    return LayerParams(w1, b1, gamma, beta, w2, b2, bias)


def make_layer(name, seed, lengths, D, H, d, alpha, n_layers=1, residual=False,
               bias_kind=BIAS_RAB_PT, P=128, NT=32, table_std=0.02, randomize_affine=False,
               rng=None, ts=None, dtype="bf16", x_std=1.0):
    rng = rng if rng is not None else np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    offs = offsets_from_lengths(lengths)
    T = int(offs[-1])
    if ts is None:
        ts = _timestamps(rng, lengths)
    x = _store(rng.standard_normal((T, D), dtype=np.float32) * x_std, dtype)
    layers = [_layer_params(rng, dtype, D, H, d, d, bias_kind, P, NT, table_std, randomize_affine)
              for _ in range(n_layers)]
    ms = int(lengths.max()) if len(lengths) else 0
    return LayerInputs(name, seed, dtype, len(lengths), D, H, d, d, offs, ms, ts, x, layers,
                       float(alpha), residual)


def zipf_lengths(rng, B, a, lo, hi):
    return np.clip(rng.zipf(a, size=B), lo, hi).astype(np.int64)


def layer_small(seed=1001, B=32, randomize_affine=False, **kw):
    """Full layer, bf16: D=256, H=4, d=64, B=32, n = clip(Zipf(1.5), 8, 1024),
    alpha = 1/1024, 128 position / 32 time buckets, no residual."""
    rng = np.random.default_rng(seed)
    lengths = zipf_lengths(rng, B, 1.5, 8, 1024)
    return make_layer("layer_small", seed, lengths, D=256, H=4, d=64, alpha=1.0 / 1024, P=128,
                      NT=32, rng=rng, randomize_affine=randomize_affine, **kw)


def truncated_zipf(rng, size, a, n_items):
    """Ranks 1..n_items with P(r) proportional to r^-a, by inverse CDF; returns 0-based ids."""
    w = np.arange(1, n_items + 1, dtype=np.float64) ** (-a)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(size)
    return np.minimum(np.searchsorted(cdf, u, side="right"), n_items - 1).astype(np.int32)


def genrank(seed=1003, B=64, lo=512, hi=4096, n_items=1_000_000, emb_dim=512, n_actions=4,
            randomize_affine=False, **kw):
    """GenRank action-oriented layer, bf16: ALiBi bias, tokens = item_emb + action_emb,
    B=64, n ~ U{512..4096}, D=512, H=8, d=64, alpha = 1/4096."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, size=B)
    offs = offsets_from_lengths(lengths)
    T = int(offs[-1])
    ts = _timestamps(rng, lengths)
    item_ids = truncated_zipf(rng, T, 1.1, n_items)
    action_ids = rng.integers(0, n_actions, size=T).astype(np.int32)
    item_table = round_bf16(rng.standard_normal((n_items, emb_dim), dtype=np.float32)
                            * np.float32(math.sqrt(0.5)))
    action_table = round_bf16(rng.standard_normal((n_actions, emb_dim), dtype=np.float32)
                              * np.float32(math.sqrt(0.5)))
    H, d = 8, 64
    layers = [_layer_params(rng, "bf16", emb_dim, H, d, d, BIAS_ALIBI, 0, 0, 0.0,
                            randomize_affine)]
    ms = int(lengths.max()) if B else 0
    inp = LayerInputs("genrank", seed, "bf16", B, emb_dim, H, d, d, offs, ms, ts, None, layers,
                      kw.pop("alpha", 1.0 / 4096), False, item_ids=item_ids,
                      action_ids=action_ids, item_table=item_table, action_table=action_table)
    return inp


def stochastic_length(rng, lengths, ts_list, cap=1024, p=0.5):
    """Simplified Stochastic Length: a sequence longer than `cap` is replaced,
    with probability p, by `cap` of its events drawn uniformly without
    replacement and kept in time order; otherwise it is kept whole."""
    out_len, out_ts = [], []
    for n, t in zip(lengths, ts_list):
        if n > cap and rng.random() < p:
            keep = np.sort(rng.choice(int(n), size=cap, replace=False))
            out_len.append(cap)
            out_ts.append(t[keep])
        else:
            out_len.append(int(n))
            out_ts.append(t)
    return np.asarray(out_len, np.int64), out_ts


def stack8(seed=1004, B=128, n_layers=8, hi=4096, cap=1024, randomize_affine=False, **kw):
    """8-layer stack, bf16: D=512, H=8, d=64, 256 position / 32 time buckets,
    B=128, n0 = clip(Zipf(1.2), 1, 4096), then stochastic length (cap 1024, p=0.5),
    residual connections, alpha = 1/4096."""
    rng = np.random.default_rng(seed)
    n0 = zipf_lengths(rng, B, 1.2, 1, hi)
    ts0 = [_timestamps(rng, [n]) for n in n0]
    lengths, ts_list = stochastic_length(rng, n0, ts0, cap=cap)
    ts = np.concatenate(ts_list) if len(ts_list) else np.zeros(0, np.int64)
    return make_layer("stack8", seed, lengths, D=512, H=8, d=64, alpha=kw.pop("alpha", 1.0 / 4096),
                      n_layers=n_layers, residual=True, P=256, NT=32, rng=rng, ts=ts,
                      randomize_affine=randomize_affine, **kw)


@dataclass
class CandInputs:
    """Candidate scoring over a cached history: user b's history rows
    [hist_offsets[b], hist_offsets[b+1]) of kh, vh, ts_h; its candidates' rows
    [cand_offsets[b], cand_offsets[b+1]) of qc, kc, vc, ts_c."""
    name: str
    seed: int
    dtype: str
    B: int
    H: int
    d: int
    hist_offsets: np.ndarray   # int32 [B+1]
    cand_offsets: np.ndarray   # int32 [B+1]
    max_hist: int
    max_cand: int
    ts_h: np.ndarray           # int64 [Th]
    ts_c: np.ndarray           # int64 [Tc]
    qc: np.ndarray             # float32 [Tc, H, d] (exact in dtype)
    kc: np.ndarray
    vc: np.ndarray
    kh: np.ndarray             # float32 [Th, H, d]
    vh: np.ndarray
    bias: BiasSpec
    alpha: float
    out_scale: float = 1.0

    @property
    def Th(self):
        return int(self.hist_offsets[-1])

    @property
    def Tc(self):
        return int(self.cand_offsets[-1])


def make_candidates(name, seed, dtype, hist_lengths, cand_counts, H, d, alpha,
                    bias_kind=BIAS_RAB_PT, P=256, NT=32, table_std=0.02, per_head_tables=False,
                    rng=None, jitter=0, out_scale=1.0):
    """Histories as in make_attn; each user's candidates carry the request time (last
    history event + Exp(mean 3600 s)) plus U{0..jitter} seconds each."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    hist_lengths = np.asarray(hist_lengths, dtype=np.int64)
    cand_counts = np.asarray(cand_counts, dtype=np.int64)
    ho = offsets_from_lengths(hist_lengths)
    co = offsets_from_lengths(cand_counts)
    Th, Tc = int(ho[-1]), int(co[-1])
    ts_h = _timestamps(rng, hist_lengths)
    ts_c = np.zeros(Tc, np.int64)
    for b in range(len(hist_lengths)):
        last = int(ts_h[ho[b + 1] - 1]) if hist_lengths[b] else 1_600_000_000
        req = last + int(rng.exponential(3600.0))
        ts_c[co[b]:co[b + 1]] = req + rng.integers(0, jitter + 1, size=int(cand_counts[b]))
    kh = _store(rng.standard_normal((Th, H, d), dtype=np.float32), dtype)
    vh = _store(rng.standard_normal((Th, H, d), dtype=np.float32), dtype)
    qc = _store(rng.standard_normal((Tc, H, d), dtype=np.float32), dtype)
    kc = _store(rng.standard_normal((Tc, H, d), dtype=np.float32), dtype)
    vc = _store(rng.standard_normal((Tc, H, d), dtype=np.float32), dtype)
    bias = BiasSpec(kind=bias_kind)
    if bias_kind == BIAS_RAB_PT:
        bias.w_pos, bias.w_time = _tables(rng, P, NT, table_std, H if per_head_tables else None)
    mh = int(hist_lengths.max()) if len(hist_lengths) else 0
    mc = int(cand_counts.max()) if len(cand_counts) else 0
    return CandInputs(name, seed, dtype, len(hist_lengths), H, d, ho, co, mh, mc, ts_h, ts_c,
                      qc, kc, vc, kh, vh, bias, float(alpha), out_scale)


def mfalcon(seed=1005, B=16, n_cand=1024, lo=256, hi=8192, **kw):
    """bf16 candidate scoring: B=16 users with attn_long's history lengths (lognormal,
    median 2048, clipped to [256, 8192]), 1024 candidates each, H=8, d=64,
    alpha = 1/8192, 256 position / 32 time buckets."""
    rng = np.random.default_rng(seed)
    lengths = lognormal_lengths(rng, B, lo=lo, hi=hi)
    kw.setdefault("alpha", 1.0 / 8192)
    return make_candidates("mfalcon", seed, "bf16", lengths, np.full(B, n_cand), H=8, d=64,
                           P=256, NT=32, rng=rng, **kw)


WORKLOADS = {
    "attn_small": attn_small,
    "layer_small": layer_small,
    "attn_long": attn_long,
    "genrank": genrank,
    "stack8": stack8,
    "mfalcon": mfalcon,
}
