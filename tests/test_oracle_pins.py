"""Pins of the float64 oracle against facts that do not come from its own code.

Closed forms derived by hand, Python-integer brute force read back through probe inputs,
library routines for special cases, and a scalar-loop restatement of the whole layer.
"""
import math

import numpy as np
import pytest

from oracle import hstu_oracle as O
from oracle import hstu_loops as Lp


def _jag(lengths, taus, mask=O.CAUSAL, num_candidates=None, attn_scale=None):
    offs = np.zeros(len(lengths) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lengths)
    return dict(seq_offsets=offs, timestamps=np.asarray(taus, np.int64), mask=mask,
                num_candidates=None if num_candidates is None else np.asarray(num_candidates),
                attn_scale=None if attn_scale is None else np.asarray(attn_scale, np.float64))


def _rand_taus(rng, lengths, spread=10_000):
    out = []
    for n in lengths:
        t0 = int(rng.integers(0, 1 << 40))
        out.append(t0 + np.cumsum(rng.integers(0, spread, size=n)))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


# --------------------------------------------------------------------------- SiLU and buckets
def test_silu_closed_forms():
    L = math.log(3.0)
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert O.silu(np.array(L)) == pytest.approx(0.75 * L, rel=1e-15)
    assert O.silu(np.array(-L)) == pytest.approx(-0.25 * L, rel=1e-15)
    assert O.silu(np.array(0.0)) == 0.0
    x = np.linspace(-30, 30, 101)
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-12)   # SiLU(x) - SiLU(-x) = x
    assert O.silu(np.array(-1e4)) == 0.0 and O.silu(np.array(1e4)) == 1e4


def test_time_bucket_brute_force_python_ints():
    rng = np.random.default_rng(7)
    edge = [0, 1, 2, 3, 4, 7, 8, 3600, (1 << 31) - 1, 1 << 31, (1 << 32) + 5, (1 << 62), (1 << 63) - 1,
            -1, -(1 << 63), -(1 << 62), -3600]
    a = np.array(edge + list(rng.integers(-(1 << 62), 1 << 62, size=200)), dtype=np.int64)
    b = np.array(list(reversed(edge)) + list(rng.integers(-(1 << 40), 1 << 40, size=200)), dtype=np.int64)
    for Tb in (1, 2, 32, 65, 256):
        got = O.time_bucket(a, b, Tb)
        want = [min(abs(int(x) - int(y)).bit_length(), Tb - 1) for x, y in zip(a, b)]
        assert got.tolist() == want
    # hand-stated values: |dt| = 0 -> 0; 1 -> 1; 2,3 -> 2; 4..7 -> 3; 3600 -> 12; 2**64-1 -> 64
    t = np.array([0, 1, 2, 3, 4, 7, 3600], dtype=np.int64)
    assert O.time_bucket(t, np.zeros_like(t), 256).tolist() == [0, 1, 2, 2, 3, 3, 12]
    assert int(O.time_bucket(np.array([(1 << 63) - 1]), np.array([-(1 << 63)]), 256)[0]) == 64


def test_position_bucket_brute_force():
    i = np.arange(0, 300)[:, None]
    j = np.arange(0, 300)[None, :]
    for P in (1, 2, 32, 256):
        got = O.position_bucket(i, j, P)
        want = np.array([[min(abs(a - b), P - 1) for b in range(300)] for a in range(300)])
        assert (got == want).all()


# --------------------------------------------------------------------------- closed forms
def test_single_token_closed_form():
    rng = np.random.default_rng(3)
    Dh = 8
    q, k, v = rng.standard_normal((3, 1, 1, Dh))
    wp = rng.standard_normal((1, 4))
    wt = rng.standard_normal((1, 5))
    jag = _jag([1], [123456789])
    out = O.attn_fwd(jag, q, k, v, wp, wt)
    s = float(np.dot(q[0, 0], k[0, 0])) + wp[0, 0] + wt[0, 0]
    want = (s / (1.0 + math.exp(-s))) * v[0, 0]          # c = 1/n = 1
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-14)


def test_two_token_hand_example():
    # Dh = 1, H = 1; q = [1, 2], k = [0.5, -1], v = [3, 5]; tau = [100, 103]; P = 2, Tb = 4
    # wp = [0, L], wt = [0, 0, L, 0], L = ln 3.
    # s00 = 1*0.5 + wp[0] + wt[bitlen 0 = 0]           = 0.5
    # s10 = 2*0.5 + wp[min(1,1)=1] + wt[bitlen(3) = 2]   = 1 + 2L
    # s11 = 2*(-1) + wp[0] + wt[0]                       = -2
    # O0 = (1/2) SiLU(0.5) * 3 ;  O1 = (1/2) (SiLU(1 + 2L) * 3 + SiLU(-2) * 5)
    L = math.log(3.0)
    silu = lambda z: z / (1.0 + math.exp(-z))
    q = np.array([[[1.0]], [[2.0]]]); k = np.array([[[0.5]], [[-1.0]]]); v = np.array([[[3.0]], [[5.0]]])
    jag = _jag([2], [100, 103])
    out = O.attn_fwd(jag, q, k, v, np.array([[0.0, L]]), np.array([[0.0, 0.0, L, 0.0]]))
    want0 = 0.5 * silu(0.5) * 3.0
    want1 = 0.5 * (silu(1.0 + 2.0 * L) * 3.0 + silu(-2.0) * 5.0)
    np.testing.assert_allclose(out[:, 0, 0], [want0, want1], rtol=1e-14)
    # exp(-(1 + 2 ln 3)) = e^-1 / 9  ->  SiLU(1 + 2L) = (1 + 2L) / (1 + 1/(9e))
    np.testing.assert_allclose(silu(1.0 + 2.0 * L), (1.0 + 2.0 * L) / (1.0 + 1.0 / (9.0 * math.e)), rtol=1e-15)


def test_constant_score_reduces_to_cumsum():
    # Q = 0 and constant tables: every allowed a_ij = SiLU(alpha + beta), so O_i = c SiLU(a+b) sum_{j<=i} v_j
    rng = np.random.default_rng(5)
    lengths = [7, 1, 13]
    T = sum(lengths)
    H, Dh = 2, 4
    q = np.zeros((T, H, Dh)); k = rng.standard_normal((T, H, Dh)); v = rng.standard_normal((T, H, Dh))
    alpha, beta = 0.3, -1.1
    jag = _jag(lengths, _rand_taus(rng, lengths))
    out = O.attn_fwd(jag, q, k, v, np.full((1, 16), alpha), np.full((1, 64), beta))
    a = (alpha + beta) / (1.0 + math.exp(-(alpha + beta)))
    offs = jag["seq_offsets"]
    for b, n in enumerate(lengths):
        seg = v[offs[b]:offs[b + 1]]
        np.testing.assert_allclose(out[offs[b]:offs[b + 1]], (a / n) * np.cumsum(seg, axis=0), rtol=1e-13,
                                   atol=1e-15)


# --------------------------------------------------------------------------- probes read back buckets
def _indicator_probe(n, P, Tb, which, idx, taus, mask=O.CAUSAL, m=0):
    """Q = 0, V = I (Dh = n), one-hot table -> O[i, j] * n / SiLU(1) = [bucket(i,j) == idx and allowed]."""
    q = np.zeros((n, 1, n)); k = np.zeros((n, 1, n)); v = np.eye(n)[:, None, :]
    wp = np.zeros((1, P)); wt = np.zeros((1, Tb))
    (wp if which == "pos" else wt)[0, idx] = 1.0
    jag = _jag([n], taus, mask=mask, num_candidates=[m] if mask == O.CAUSAL_CANDIDATES else None)
    out = O.attn_fwd(jag, q, k, v, wp, wt)[:, 0, :]
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    return out * n / s1


def _allowed_py(i, j, n_hist, mask):
    if mask == O.CAUSAL or i < n_hist:
        return j <= i
    return j < n_hist or j == i


@pytest.mark.parametrize("mask,m", [(O.CAUSAL, 0), (O.CAUSAL_CANDIDATES, 3)])
def test_position_probe_matches_python(mask, m):
    n, P = 20, 6
    rng = np.random.default_rng(11)
    taus = np.cumsum(rng.integers(0, 50, size=n))
    n_hist = n - m
    pos = [i if mask == O.CAUSAL else min(i, n_hist) for i in range(n)]
    for idx in range(P):
        got = _indicator_probe(n, P, 8, "pos", idx, taus, mask, m)
        want = np.array([[1.0 if (_allowed_py(i, j, n_hist, mask) and min(abs(pos[i] - pos[j]), P - 1) == idx)
                          else 0.0 for j in range(n)] for i in range(n)])
        np.testing.assert_allclose(got, want, atol=1e-12)


def test_time_probe_matches_python():
    n, Tb = 24, 12
    rng = np.random.default_rng(12)
    # non-monotone timestamps with duplicates and a giant gap
    taus = rng.integers(0, 3000, size=n).astype(np.int64)
    taus[5] = taus[4]
    taus[10] = taus[9] + (1 << 33)
    for idx in range(Tb):
        got = _indicator_probe(n, 4, Tb, "time", idx, taus)
        want = np.array([[1.0 if (j <= i and min(abs(int(taus[i]) - int(taus[j])).bit_length(), Tb - 1) == idx)
                          else 0.0 for j in range(n)] for i in range(n)])
        np.testing.assert_allclose(got, want, atol=1e-12)


@pytest.mark.parametrize("m", [0, 1, 5, 9])
def test_candidate_mask_probe(m):
    # constant scores: O[i, j] is proportional to the allowed pattern itself
    n = 9
    q = np.zeros((n, 1, n)); k = np.zeros((n, 1, n)); v = np.eye(n)[:, None, :]
    jag = _jag([n], np.arange(n) * 10, mask=O.CAUSAL_CANDIDATES, num_candidates=[m], attn_scale=[1.0])
    out = O.attn_fwd(jag, q, k, v, np.full((1, 4), 0.5), np.full((1, 4), 0.5))[:, 0, :]
    s = 1.0 / (1.0 + math.exp(-1.0))
    want = np.array([[s if _allowed_py(i, j, n - m, O.CAUSAL_CANDIDATES) else 0.0 for j in range(n)]
                     for i in range(n)])
    np.testing.assert_allclose(out, want, atol=1e-15)


# --------------------------------------------------------------------------- projection layout
def test_projection_split_layout():
    # D = H*Dh; W1 = [a I; b I; c I; d I]: U = SiLU(a x), V = SiLU(b x), Q = SiLU(c x), K = SiLU(d x),
    # each reshaped head-major [T, H, Dh]
    rng = np.random.default_rng(2)
    H, Dh, T = 3, 4, 5
    D = H * Dh
    x = rng.standard_normal((T, D))
    coef = [0.5, -1.5, 2.0, 0.25]
    w = np.concatenate([c * np.eye(D) for c in coef], axis=0)
    u, v, q, k = O.projection(x, w, None, H, Dh)
    silu = lambda z: z / (1.0 + np.exp(-z))
    for got, c in zip((u, v, q, k), coef):
        np.testing.assert_allclose(got, silu(c * x).reshape(T, H, Dh), rtol=1e-15)
    # bias lands on the right column
    b = np.zeros(4 * D); b[2 * D + 1 * Dh + 2] = 3.0           # Q, head 1, dim 2
    _, _, q2, _ = O.projection(np.zeros((1, D)), np.zeros((4 * D, D)), b, H, Dh)
    assert q2[0, 1, 2] == pytest.approx(3.0 / (1.0 + math.exp(-3.0))) and np.count_nonzero(q2) == 1


def test_layer_norm_moments():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 33)) * 5 + 2
    y = O.layer_norm(x, 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-14)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1, rtol=1e-13)
    # eps enters as var + eps
    y2 = O.layer_norm(np.array([[1.0, -1.0]]), 3.0)     # var = 1 -> /sqrt(4)
    np.testing.assert_allclose(y2, [[0.5, -0.5]], rtol=1e-15)


def test_gather_rows_matches_python_indexing():
    table = np.arange(40.0).reshape(10, 4)
    ids = [3, 3, 0, 9, 5]
    np.testing.assert_array_equal(O.gather_rows(table, ids), np.array([table[i] for i in ids]))


# --------------------------------------------------------------------------- scalar loops vs vectorised
def _tiny_layer(rng, lengths, D, H, Dh, P, Tb, mask, m_list, R=1, bias=True):
    T = sum(lengths)
    x = rng.standard_normal((T, D))
    w1 = rng.standard_normal((4 * H * Dh, D)) * 0.4
    w2 = rng.standard_normal((D, H * Dh)) * 0.4
    b1 = rng.standard_normal(4 * H * Dh) * 0.2 if bias else None
    b2 = rng.standard_normal(D) * 0.2 if bias else None
    wp = rng.standard_normal((R, P)) * 0.5
    wt = rng.standard_normal((R, Tb)) * 0.5
    taus = _rand_taus(rng, lengths, spread=5000)
    jag = _jag(lengths, taus, mask, m_list)
    return x, w1, b1, w2, b2, wp, wt, jag


@pytest.mark.parametrize("seed,lengths,mask,m_list,R", [
    (0, [3, 0, 5], O.CAUSAL, None, 1),
    (1, [1, 6, 2], O.CAUSAL, None, 2),
    (2, [6, 4], O.CAUSAL_CANDIDATES, [2, 0], 1),
    (3, [7, 1, 5], O.CAUSAL_CANDIDATES, [3, 1, 5], 2),
])
def test_attention_matches_scalar_loops(seed, lengths, mask, m_list, R):
    rng = np.random.default_rng(seed)
    H, Dh, P, Tb = 2, 3, 4, 6
    T = sum(lengths)
    q, k, v = rng.standard_normal((3, T, H, Dh))
    wp = rng.standard_normal((R, P)); wt = rng.standard_normal((R, Tb))
    taus = _rand_taus(rng, lengths, spread=40)
    jag = _jag(lengths, taus, mask, m_list)
    got = O.attn_fwd(jag, q, k, v, wp, wt)
    want = Lp.attn_fwd_loops(jag["seq_offsets"].tolist(), taus.tolist(), q.tolist(), k.tolist(), v.tolist(),
                             wp.tolist(), wt.tolist(), mask, m_list, None)
    np.testing.assert_allclose(got, np.array(want).reshape(T, H, Dh) if T else got, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed,mask,ln_output", [(0, O.CAUSAL, 0), (1, O.CAUSAL, 1), (2, O.CAUSAL_CANDIDATES, 1)])
def test_layer_matches_scalar_loops(seed, mask, ln_output):
    rng = np.random.default_rng(100 + seed)
    lengths = [4, 1, 6]
    m_list = [1, 0, 2] if mask == O.CAUSAL_CANDIDATES else None
    D, H, Dh, P, Tb = 6, 2, 3, 5, 7
    x, w1, b1, w2, b2, wp, wt, jag = _tiny_layer(rng, lengths, D, H, Dh, P, Tb, mask, m_list)
    eps = 1e-3
    got = O.layer_fwd(x, jag, w1, b1, w2, b2, wp, wt, H, Dh, eps, ln_output)
    want = Lp.layer_fwd_loops(x.tolist(), jag["seq_offsets"].tolist(), jag["timestamps"].tolist(), w1.tolist(),
                              b1.tolist(), w2.tolist(), b2.tolist(), wp.tolist(), wt.tolist(), H, Dh, eps,
                              ln_output, mask, m_list, None)
    np.testing.assert_allclose(got, np.array(want), rtol=1e-11, atol=1e-12)


def test_stack_is_layers_in_sequence():
    rng = np.random.default_rng(9)
    lengths = [5, 3]
    D, H, Dh = 4, 2, 2
    layers = []
    x, *_ , jag = _tiny_layer(rng, lengths, D, H, Dh, 4, 4, O.CAUSAL, None)
    for _ in range(3):
        _, w1, b1, w2, b2, wp, wt, _ = _tiny_layer(rng, lengths, D, H, Dh, 4, 4, O.CAUSAL, None)
        layers.append(dict(w_uvqk=w1, b_uvqk=b1, w_out=w2, b_out=b2, pos_bias=wp, time_bias=wt, ln_eps=1e-5))
    got = O.stack_fwd(x, jag, layers, H, Dh)
    y = x.tolist()
    for li, L in enumerate(layers):
        y = Lp.layer_fwd_loops(y, jag["seq_offsets"].tolist(), jag["timestamps"].tolist(), L["w_uvqk"].tolist(),
                               L["b_uvqk"].tolist(), L["w_out"].tolist(), L["b_out"].tolist(),
                               L["pos_bias"].tolist(), L["time_bias"].tolist(), H, Dh, 1e-5, li < 2)
    np.testing.assert_allclose(got, np.array(y), rtol=1e-11, atol=1e-12)
