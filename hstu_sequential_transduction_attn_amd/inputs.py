"""Seeded synthetic inputs for the HSTU layer forward.

This module is shared by the tests, the benchmark and the CPU oracle's callers.  It holds
no arithmetic of the method itself: it only draws random numbers, rounds them to the
storage precision and lays them out.  Everything it returns is a plain numpy array, so
the oracle (float64, CPU) and the HIP library (device memory) both start from the very
same values.

Workload shapes follow the pages' regime: per-user event timelines with timestamps and
skewed item popularity ("DLRMv4：MLPerfの推薦システム訓練ベンチマークがシーケンス化時代へ",
sections "1つの訓練サンプルがHSTUでどのように処理されるか" and "データ分布がなぜ重要なのか"),
and sequence length 8192 for the attention speed regime ("Actions Speak Louder than Words:
Trillion-Parameter Sequential Transducers for Generative Recommendations", abstract).

bf16 tensors are carried as two arrays: ``bits`` (uint16 bit patterns, round-to-nearest-even
from the float32 draw) and ``values`` (float32 holding exactly those bf16 values).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

SEED_ROOT = 240217152
CAUSAL = 0
CAUSAL_CANDIDATES = 1


# --------------------------------------------------------------------------- rounding helpers
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A host tensor in its storage dtype: 'f32' or 'bf16' (values are float32 either way)."""
    values: np.ndarray            # float32, exact storage values
    dtype: str                    # 'f32' | 'bf16'
    bits: Optional[np.ndarray] = None  # uint16 when dtype == 'bf16'

    @staticmethod
    def make(x: np.ndarray, dtype: str) -> "Tensor":
        x = np.ascontiguousarray(x, dtype=np.float32)
        if dtype == "f32":
            return Tensor(values=x, dtype="f32")
        if dtype == "bf16":
            b = bf16_bits(x)
            return Tensor(values=bf16_values(b), dtype="bf16", bits=b)
        raise ValueError(dtype)

    @property
    def shape(self):
        return self.values.shape


# --------------------------------------------------------------------------- random draws
def rng_for(config_id: int, stream: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, config_id, stream])))


def xavier_uniform(rng: np.random.Generator, fan_out: int, fan_in: int) -> np.ndarray:
    bound = math.sqrt(6.0 / (fan_in + fan_out))
    return rng.uniform(-bound, bound, size=(fan_out, fan_in)).astype(np.float32)


def timestamps_for(rng: np.random.Generator, lengths: List[int], mean_gap: float = 3600.0) -> np.ndarray:
    """Per-user strictly increasing int64 seconds: start 1.7e9 + U{0..3.15e7-1}, gaps max(1, ceil(Exp(mean)))."""
    out = []
    for n in lengths:
        start = 1_700_000_000 + int(rng.integers(0, 31_500_000))
        gaps = np.maximum(1, np.ceil(rng.exponential(mean_gap, size=max(n - 1, 0)))).astype(np.int64)
        t = np.empty(n, dtype=np.int64)
        if n:
            t[0] = start
            t[1:] = start + np.cumsum(gaps)
        out.append(t)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def bounded_zipf(rng: np.random.Generator, a: float, n_items: int, size: int) -> np.ndarray:
    """Ranks 1..n_items with P(r) proportional to r**-a (inverse CDF), returned as ids rank-1 (int64)."""
    ranks = np.arange(1, n_items + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-a))
    cdf /= cdf[-1]
    u = rng.random(size)
    return np.minimum(np.searchsorted(cdf, u, side="left"), n_items - 1).astype(np.int64)


def offsets_of(lengths: List[int]) -> np.ndarray:
    o = np.zeros(len(lengths) + 1, dtype=np.int32)
    o[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return o


# --------------------------------------------------------------------------- containers
@dataclasses.dataclass
class Jagged:
    seq_offsets: np.ndarray                 # int32 [B+1]
    timestamps: np.ndarray                  # int64 [T]
    num_candidates: Optional[np.ndarray]    # int32 [B] or None
    attn_scale: Optional[np.ndarray]        # float32 [B] or None (=> 1/n_b)
    mask: int = CAUSAL

    @property
    def num_seqs(self) -> int:
        return len(self.seq_offsets) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.seq_offsets[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.seq_offsets.astype(np.int64))

    @property
    def max_seq_len(self) -> int:
        return int(self.lengths.max()) if self.num_seqs else 0


@dataclasses.dataclass
class Rab:
    pos_bias: np.ndarray    # float32 [R, P]
    time_bias: np.ndarray   # float32 [R, Tb]


@dataclasses.dataclass
class LayerWeights:
    w_uvqk: Tensor          # [4*H*Dh, D]
    b_uvqk: Optional[Tensor]
    w_out: Tensor           # [D, H*Dh]
    b_out: Optional[Tensor]
    rab: Rab
    ln_eps: float = 1e-6


@dataclasses.dataclass
class AttnCase:
    """Inputs of the attention-only call: Q, K, V as [T, H, Dh]."""
    name: str
    jagged: Jagged
    rab: Rab
    q: Tensor
    k: Tensor
    v: Tensor
    u: Optional[Tensor]
    num_heads: int
    head_dim: int
    dtype: str

    def flops(self) -> int:
        """Algorithmic FLOP: only allowed (unmasked, non-padded) pairs, 2*Dh for QK plus 2*Dh for AV."""
        return allowed_pairs(self.jagged) * self.num_heads * 4 * self.head_dim


@dataclasses.dataclass
class LayerCase:
    name: str
    jagged: Jagged
    x: Tensor                       # [T, D]
    layers: List[LayerWeights]
    num_heads: int
    head_dim: int
    d_model: int
    dtype: str
    ids: Optional[np.ndarray] = None         # int64 [T] (embedding-gather cases)
    table_rows: int = 0
    table_touched: Optional[np.ndarray] = None   # sorted unique ids
    table_values: Optional[Tensor] = None        # [len(touched), D]


def allowed_pairs(j: Jagged) -> int:
    """Number of (i, j) pairs that the mask lets through, summed over sequences (host-side count)."""
    n = j.lengths
    if j.mask == CAUSAL or j.num_candidates is None:
        return int(np.sum(n * (n + 1) // 2))
    m = j.num_candidates.astype(np.int64)
    nh = n - m
    return int(np.sum(nh * (nh + 1) // 2 + m * (nh + 1)))


# --------------------------------------------------------------------------- generic builders
def make_rab(rng: np.random.Generator, rows: int, P: int, Tb: int, std: float = 0.02) -> Rab:
    return Rab(pos_bias=rng.normal(0.0, std, size=(rows, P)).astype(np.float32),
               time_bias=rng.normal(0.0, std, size=(rows, Tb)).astype(np.float32))


def make_layer_weights(rng: np.random.Generator, D: int, H: int, Dh: int, P: int, Tb: int,
                       dtype: str, bias_std: float = 0.0, eps: float = 1e-6) -> LayerWeights:
    w1 = xavier_uniform(rng, 4 * H * Dh, D)
    w2 = xavier_uniform(rng, D, H * Dh)
    b1 = rng.normal(0.0, bias_std, size=4 * H * Dh).astype(np.float32) if bias_std else None
    b2 = rng.normal(0.0, bias_std, size=D).astype(np.float32) if bias_std else None
    rab = make_rab(rng, 1, P, Tb)
    return LayerWeights(w_uvqk=Tensor.make(w1, dtype), b_uvqk=None if b1 is None else Tensor.make(b1, dtype),
                        w_out=Tensor.make(w2, dtype), b_out=None if b2 is None else Tensor.make(b2, dtype),
                        rab=rab, ln_eps=eps)


def jagged_layer_case(name: str, config_id: int, lengths: List[int], D: int, H: int, Dh: int,
                      P: int, Tb: int, dtype: str, num_layers: int = 1, bias_std: float = 0.0,
                      stream: int = 0) -> LayerCase:
    """X ~ N(0,1) [T, D], Xavier weights, N(0, 0.02) rab tables, exponential-gap timestamps, causal."""
    rng = rng_for(config_id, stream)
    T = int(sum(lengths))
    x = rng.standard_normal(size=(T, D)).astype(np.float32)
    tau = timestamps_for(rng, lengths)
    layers = [make_layer_weights(rng, D, H, Dh, P, Tb, dtype, bias_std) for _ in range(num_layers)]
    jag = Jagged(seq_offsets=offsets_of(lengths), timestamps=tau, num_candidates=None, attn_scale=None)
    return LayerCase(name=name, jagged=jag, x=Tensor.make(x, dtype), layers=layers, num_heads=H,
                     head_dim=Dh, d_model=D, dtype=dtype)


def attn_case(name: str, config_id: int, lengths: List[int], H: int, Dh: int, P: int, Tb: int,
              dtype: str, stream: int = 0, with_u: bool = True, num_candidates: Optional[List[int]] = None,
              rab_rows: int = 1) -> AttnCase:
    """Q, K, V (and U) ~ N(0,1) [T, H, Dh]; rab tables N(0, 0.02); exponential-gap timestamps."""
    rng = rng_for(config_id, stream)
    T = int(sum(lengths))
    tau = timestamps_for(rng, lengths)
    rab = make_rab(rng, rab_rows, P, Tb)
    q = rng.standard_normal(size=(T, H, Dh)).astype(np.float32)
    k = rng.standard_normal(size=(T, H, Dh)).astype(np.float32)
    v = rng.standard_normal(size=(T, H, Dh)).astype(np.float32)
    u = rng.standard_normal(size=(T, H, Dh)).astype(np.float32) if with_u else None
    mask = CAUSAL if num_candidates is None else CAUSAL_CANDIDATES
    nc = None if num_candidates is None else np.asarray(num_candidates, dtype=np.int32)
    jag = Jagged(seq_offsets=offsets_of(lengths), timestamps=tau, num_candidates=nc, attn_scale=None, mask=mask)
    return AttnCase(name=name, jagged=jag, rab=rab, q=Tensor.make(q, dtype), k=Tensor.make(k, dtype),
                    v=Tensor.make(v, dtype), u=None if u is None else Tensor.make(u, dtype),
                    num_heads=H, head_dim=Dh, dtype=dtype)


# --------------------------------------------------------------------------- cached-history scoring
@dataclasses.dataclass
class CachedCase:
    """A candidate batch split from a one-pass candidate case: each user's history rows (the cache) and
    the candidate rows, plus where the candidates sit in the one-pass layout."""
    name: str
    hist_offsets: np.ndarray        # int32 [B+1]
    hist_timestamps: np.ndarray     # int64 [T_h]
    cand_offsets: np.ndarray        # int32 [B+1]
    cand_timestamps: np.ndarray     # int64 [T_c]
    k_hist: Tensor                  # [T_h, H, Dh]
    v_hist: Tensor
    q: Tensor                       # [T_c, H, Dh]
    k: Tensor
    v: Tensor
    rab: Rab
    num_heads: int
    head_dim: int
    dtype: str
    cand_rows: np.ndarray           # int64 [T_c]: row of each candidate in the one-pass batch
    one_pass_lengths: np.ndarray    # int64 [B]: n_h + m_b

    @property
    def max_candidates(self) -> int:
        d = np.diff(self.cand_offsets.astype(np.int64))
        return int(d.max()) if len(d) else 0


def _take(t: Tensor, idx: np.ndarray) -> Tensor:
    return Tensor(values=t.values[idx], dtype=t.dtype, bits=None if t.bits is None else t.bits[idx])


def split_candidates(case: AttnCase) -> CachedCase:
    """Slices a candidate-mask case (num_candidates set) into history and candidate parts per user."""
    offs = case.jagged.seq_offsets.astype(np.int64)
    m = case.jagged.num_candidates.astype(np.int64)
    B = len(offs) - 1
    hist_idx = [np.arange(offs[b], offs[b + 1] - m[b]) for b in range(B)]
    cand_idx = [np.arange(offs[b + 1] - m[b], offs[b + 1]) for b in range(B)]
    hi = np.concatenate(hist_idx) if B else np.zeros(0, np.int64)
    ci = np.concatenate(cand_idx) if B else np.zeros(0, np.int64)
    tau = case.jagged.timestamps
    return CachedCase(name=case.name + "_cached", hist_offsets=offsets_of([len(x) for x in hist_idx]),
                      hist_timestamps=tau[hi], cand_offsets=offsets_of([len(x) for x in cand_idx]),
                      cand_timestamps=tau[ci], k_hist=_take(case.k, hi), v_hist=_take(case.v, hi),
                      q=_take(case.q, ci), k=_take(case.k, ci), v=_take(case.v, ci), rab=case.rab,
                      num_heads=case.num_heads, head_dim=case.head_dim, dtype=case.dtype, cand_rows=ci,
                      one_pass_lengths=np.diff(offs))
