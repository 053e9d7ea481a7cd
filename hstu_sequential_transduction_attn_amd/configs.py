"""The five workloads (seeded, synthetic) that the tests and the benchmark run.

1. ``tiny_layer_f32``   - one layer, fp32: 4 sequences of length U{8..128}, D=64, H=2, Dh=32, P=Tb=32.
2. ``layer_bf16``       - one layer, bf16: 32 sequences, length clip(Zipf(1.2), 16, 1024), D=512, H=4x128,
                          P=Tb=128.
3. ``attn_L8192``       - attention only, bf16: 8 sequences of length 8192, H=4x128, P=Tb=256; Q, K, V, U
                          ~ N(0,1).  The sequence length of the pages' speed claim ("Actions Speak Louder
                          than Words ...", abstract).
4. ``stack8_bf16``      - 8-layer stack, bf16: 64 sequences of length U{512..4096}, D=1024, H=8x128,
                          X0 gathered from a 1M x 1024 table, ids bounded-Zipf(1.1); post-layer LayerNorm
                          between layers.
5. ``mfalcon_bf16``     - ranking forward with appended candidates, bf16: 16 users, history U{1024..8192}
                          plus 1024 candidates each, D=512, H=4x128, 3 layers, 10M x 512 table.
                          Candidates attend to the history and to themselves only.

The recipe of each draw is in ``inputs.py``; nothing here computes any part of the method.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from . import inputs as I


def _lengths_uniform(rng: np.random.Generator, lo: int, hi: int, n: int) -> List[int]:
    return [int(v) for v in rng.integers(lo, hi + 1, size=n)]


def tiny_layer_f32(num_seqs: int = 4) -> I.LayerCase:
    rng = I.rng_for(1, 100)
    lengths = _lengths_uniform(rng, 8, 128, num_seqs)
    return I.jagged_layer_case("tiny_layer_f32", 1, lengths, D=64, H=2, Dh=32, P=32, Tb=32, dtype="f32")


def layer_bf16(num_seqs: int = 32) -> I.LayerCase:
    rng = I.rng_for(2, 100)
    lengths = [int(v) for v in np.clip(rng.zipf(1.2, size=num_seqs), 16, 1024)]
    return I.jagged_layer_case("layer_bf16", 2, lengths, D=512, H=4, Dh=128, P=128, Tb=128, dtype="bf16")


def attn_L8192(num_seqs: int = 8, seq_len: int = 8192) -> I.AttnCase:
    return I.attn_case("attn_L8192", 3, [seq_len] * num_seqs, H=4, Dh=128, P=256, Tb=256, dtype="bf16")


def _gathered_case(name: str, config_id: int, lengths: List[int], ids: np.ndarray, table_rows: int,
                   D: int, H: int, Dh: int, P: int, Tb: int, num_layers: int,
                   timestamps: Optional[np.ndarray] = None, num_candidates: Optional[List[int]] = None) -> I.LayerCase:
    rng = I.rng_for(config_id, 1)
    touched = np.unique(ids)
    table = I.Tensor.make(rng.standard_normal(size=(len(touched), D)).astype(np.float32), "bf16")
    pos = np.searchsorted(touched, ids)
    x = I.Tensor(values=table.values[pos], dtype="bf16", bits=table.bits[pos])
    tau = timestamps if timestamps is not None else I.timestamps_for(rng, lengths)
    layers = [I.make_layer_weights(rng, D, H, Dh, P, Tb, "bf16") for _ in range(num_layers)]
    mask = I.CAUSAL if num_candidates is None else I.CAUSAL_CANDIDATES
    nc = None if num_candidates is None else np.asarray(num_candidates, dtype=np.int32)
    jag = I.Jagged(seq_offsets=I.offsets_of(lengths), timestamps=tau, num_candidates=nc, attn_scale=None, mask=mask)
    return I.LayerCase(name=name, jagged=jag, x=x, layers=layers, num_heads=H, head_dim=Dh, d_model=D,
                       dtype="bf16", ids=ids, table_rows=table_rows, table_touched=touched, table_values=table)


def stack8_bf16(num_seqs: int = 64, num_layers: int = 8) -> I.LayerCase:
    rng = I.rng_for(4, 0)
    lengths = _lengths_uniform(rng, 512, 4096, num_seqs)
    ids = I.bounded_zipf(rng, 1.1, 1_000_000, int(sum(lengths)))
    return _gathered_case("stack8_bf16", 4, lengths, ids, 1_000_000, D=1024, H=8, Dh=128, P=128, Tb=128,
                          num_layers=num_layers)


def mfalcon_bf16(num_users: int = 16, num_candidates: int = 1024, num_layers: int = 3,
                 hist_lo: int = 1024, hist_hi: int = 8192) -> I.LayerCase:
    rng = I.rng_for(5, 0)
    hist = _lengths_uniform(rng, hist_lo, hist_hi, num_users)
    lengths = [h + num_candidates for h in hist]
    vocab = 10_000_000
    ids, taus = [], []
    for h in hist:
        ids.append(I.bounded_zipf(rng, 1.1, vocab, h))
        ids.append(rng.integers(0, vocab, size=num_candidates).astype(np.int64))
        t_hist = I.timestamps_for(rng, [h])
        request = t_hist[-1] + max(1, int(np.ceil(rng.exponential(3600.0))))
        taus.append(t_hist)
        taus.append(np.full(num_candidates, request, dtype=np.int64))
    return _gathered_case("mfalcon_bf16", 5, lengths, np.concatenate(ids), vocab, D=512, H=4, Dh=128, P=128,
                          Tb=128, num_layers=num_layers, timestamps=np.concatenate(taus),
                          num_candidates=[num_candidates] * num_users)


ALL = {
    1: tiny_layer_f32,
    2: layer_bf16,
    3: attn_L8192,
    4: stack8_bf16,
    5: mfalcon_bf16,
}
