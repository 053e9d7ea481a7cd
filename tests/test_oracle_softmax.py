"""Pins of the oracle's causal softmax attention (the comparison kernel's reference): the scalar-loop
restatement, the closed forms of a one- and two-token sequence, rows of weights summing to one,
uniform weights giving the causal running mean, causality and jagged independence."""
import math

import numpy as np

from oracle import hstu_loops as LP
from oracle import hstu_oracle as O


def _rand(T, H, Dh, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, Dh)) for _ in range(3)]


def test_matches_scalar_loops():
    offs = np.array([0, 1, 6, 6, 13])
    q, k, v = _rand(13, 2, 4, 1)
    want = np.array(LP.softmax_attn_loops(offs, q.tolist(), k.tolist(), v.tolist()))
    got = O.softmax_attn_fwd(dict(seq_offsets=offs), q, k, v)
    assert np.abs(got - want).max() < 1e-12


def test_one_and_two_token_closed_forms():
    q, k, v = _rand(2, 1, 8, 2)
    got = O.softmax_attn_fwd(dict(seq_offsets=np.array([0, 2])), q, k, v)
    assert np.array_equal(got[0], v[0])                      # one allowed key: weight 1
    s0 = float(q[1, 0] @ k[0, 0]) / math.sqrt(8)
    s1 = float(q[1, 0] @ k[1, 0]) / math.sqrt(8)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.abs(got[1, 0] - (w0 * v[0, 0] + (1 - w0) * v[1, 0])).max() < 1e-14


def test_weights_sum_to_one_and_uniform_weights_average():
    q, k, v = _rand(40, 3, 16, 3)
    jag = dict(seq_offsets=np.array([0, 17, 40]))
    ones = O.softmax_attn_fwd(jag, q, k, np.ones_like(v))
    assert np.abs(ones - 1.0).max() < 1e-13
    # q = 0: every allowed key gets the same weight, so row i is the mean of v_0..v_i of its sequence
    avg = O.softmax_attn_fwd(jag, np.zeros_like(q), k, v)
    for o0, o1 in ((0, 17), (17, 40)):
        want = np.cumsum(v[o0:o1], axis=0) / np.arange(1, o1 - o0 + 1)[:, None, None]
        assert np.abs(avg[o0:o1] - want).max() < 1e-13


def test_causality_and_jagged_independence():
    q, k, v = _rand(30, 2, 8, 4)
    jag = dict(seq_offsets=np.array([0, 12, 30]))
    base = O.softmax_attn_fwd(jag, q, k, v)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[20:] += 5.0; k2[20:] -= 3.0; v2[20:] *= 7.0           # tokens 20.. of the second sequence
    got = O.softmax_attn_fwd(jag, q2, k2, v2)
    assert np.array_equal(got[:20], base[:20])
    rows = O.softmax_attn_fwd(jag, q, k, v, row_sample={1: np.array([0, 5, 17])})
    assert np.array_equal(rows[(1, 1)], base[[12, 17, 29], 1])
