"""Invariants that the layer's definition implies, checked on the float64 oracle.

Causality and one causal block per sequence, candidates that see the history but not each
other (DLRMv4 page, "1つの訓練サンプルがHSTUでどのように処理されるか"); a bias from position and
time distance only (DLRMv4 page, "モデルアーキテクチャ"); no softmax (linearity in V).
"""
import numpy as np
import pytest

from oracle import hstu_oracle as O


def _jag(lengths, taus, mask=O.CAUSAL, num_candidates=None, attn_scale=None):
    offs = np.zeros(len(lengths) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lengths)
    return dict(seq_offsets=offs, timestamps=np.asarray(taus, np.int64), mask=mask,
                num_candidates=None if num_candidates is None else np.asarray(num_candidates),
                attn_scale=None if attn_scale is None else np.asarray(attn_scale, np.float64))


def _taus(rng, lengths):
    out = []
    for n in lengths:
        gaps = np.maximum(1, np.ceil(rng.exponential(3600.0, size=n))).astype(np.int64)
        out.append(1_700_000_000 + np.cumsum(gaps))
    return np.concatenate(out)


def _attn_inputs(seed, lengths, H=2, Dh=8, P=16, Tb=32, R=1):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    q, k, v = rng.standard_normal((3, T, H, Dh))
    wp = rng.normal(0, 0.5, (R, P)); wt = rng.normal(0, 0.5, (R, Tb))
    return rng, q, k, v, wp, wt, _taus(rng, lengths)


def _layer_inputs(seed, lengths, D=16, H=2, Dh=8, P=16, Tb=32):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    x = rng.standard_normal((T, D))
    w1 = rng.uniform(-1, 1, (4 * H * Dh, D)) * np.sqrt(6 / (D + 4 * H * Dh))
    w2 = rng.uniform(-1, 1, (D, H * Dh)) * np.sqrt(6 / (D + H * Dh))
    b1 = rng.normal(0, 0.1, 4 * H * Dh); b2 = rng.normal(0, 0.1, D)
    wp = rng.normal(0, 0.3, (1, P)); wt = rng.normal(0, 0.3, (1, Tb))
    return rng, x, w1, b1, w2, b2, wp, wt, _taus(rng, lengths)


def test_causality_attention_bitwise():
    lengths = [40]
    rng, q, k, v, wp, wt, taus = _attn_inputs(1, lengths)
    jag = _jag(lengths, taus)
    base = O.attn_fwd(jag, q, k, v, wp, wt)
    for cut in (0, 17, 39):
        q2, k2, v2, t2 = q.copy(), k.copy(), v.copy(), taus.copy()
        q2[cut + 1:] += 3.0; k2[cut + 1:] -= 2.0; v2[cut + 1:] *= -5.0; t2[cut + 1:] += 10 ** 7
        out = O.attn_fwd(_jag(lengths, t2), q2, k2, v2, wp, wt)
        # c_b = 1/n depends on n only, so rows <= cut are bitwise unchanged
        assert np.array_equal(out[:cut + 1], base[:cut + 1])
        if cut + 1 < lengths[0]:
            assert not np.allclose(out[cut + 1:], base[cut + 1:])


def test_causality_layer():
    lengths = [30]
    rng, x, w1, b1, w2, b2, wp, wt, taus = _layer_inputs(2, lengths)
    base = O.layer_fwd(x, _jag(lengths, taus), w1, b1, w2, b2, wp, wt, 2, 8, 1e-6, 1)
    x2 = x.copy(); x2[20:] = rng.standard_normal(x2[20:].shape)
    out = O.layer_fwd(x2, _jag(lengths, taus), w1, b1, w2, b2, wp, wt, 2, 8, 1e-6, 1)
    np.testing.assert_allclose(out[:20], base[:20], rtol=0, atol=1e-12)


def test_jagged_independence_and_permutation():
    lengths = [9, 0, 25, 1, 14]
    rng, q, k, v, wp, wt, taus = _attn_inputs(3, lengths)
    jag = _jag(lengths, taus)
    full = O.attn_fwd(jag, q, k, v, wp, wt)
    offs = jag["seq_offsets"]
    for b, n in enumerate(lengths):
        sl = slice(offs[b], offs[b + 1])
        alone = O.attn_fwd(_jag([n], taus[sl]), q[sl], k[sl], v[sl], wp, wt)
        assert np.array_equal(alone, full[sl])
    perm = [4, 2, 0, 3, 1]
    idx = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in perm])
    out = O.attn_fwd(_jag([lengths[b] for b in perm], taus[idx]), q[idx], k[idx], v[idx], wp, wt)
    assert np.array_equal(out, full[idx])


def test_jagged_independence_layer():
    lengths = [12, 5, 20]
    rng, x, w1, b1, w2, b2, wp, wt, taus = _layer_inputs(4, lengths)
    full = O.layer_fwd(x, _jag(lengths, taus), w1, b1, w2, b2, wp, wt, 2, 8, 1e-6, 0)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    for b, n in enumerate(lengths):
        sl = slice(offs[b], offs[b + 1])
        alone = O.layer_fwd(x[sl], _jag([n], taus[sl]), w1, b1, w2, b2, wp, wt, 2, 8, 1e-6, 0)
        np.testing.assert_allclose(alone, full[sl], rtol=0, atol=1e-12)


def test_time_translation_invariance():
    lengths = [33, 7]
    rng, q, k, v, wp, wt, taus = _attn_inputs(5, lengths)
    a = O.attn_fwd(_jag(lengths, taus), q, k, v, wp, wt)
    b = O.attn_fwd(_jag(lengths, taus + (1 << 40)), q, k, v, wp, wt)
    c = O.attn_fwd(_jag(lengths, taus - (1 << 50)), q, k, v, wp, wt)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_rab_split_shift():
    # w_p + c together with w_t - c leaves every score, hence the output, unchanged
    lengths = [21, 11]
    rng, q, k, v, wp, wt, taus = _attn_inputs(6, lengths)
    a = O.attn_fwd(_jag(lengths, taus), q, k, v, wp, wt)
    b = O.attn_fwd(_jag(lengths, taus), q, k, v, wp + 0.7, wt - 0.7)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    # while shifting only one of them does change it
    c = O.attn_fwd(_jag(lengths, taus), q, k, v, wp + 0.7, wt)
    assert not np.allclose(a, c)


def test_linearity_in_v():
    lengths = [17, 4]
    rng, q, k, v, wp, wt, taus = _attn_inputs(7, lengths)
    v2 = rng.standard_normal(v.shape)
    jag = _jag(lengths, taus)
    lhs = O.attn_fwd(jag, q, k, v + 2.5 * v2, wp, wt)
    rhs = O.attn_fwd(jag, q, k, v, wp, wt) + 2.5 * O.attn_fwd(jag, q, k, v2, wp, wt)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)


def test_attn_scale_override():
    lengths = [10, 3]
    rng, q, k, v, wp, wt, taus = _attn_inputs(8, lengths)
    a = O.attn_fwd(_jag(lengths, taus), q, k, v, wp, wt)
    b = O.attn_fwd(_jag(lengths, taus, attn_scale=[2.0, -1.0]), q, k, v, wp, wt)
    np.testing.assert_allclose(b[:10], a[:10] * 2.0 * 10, rtol=1e-13)
    np.testing.assert_allclose(b[10:], a[10:] * -1.0 * 3, rtol=1e-13)


def test_zero_u_and_zero_b2_gives_identity():
    lengths = [9, 4]
    rng, x, w1, b1, w2, b2, wp, wt, taus = _layer_inputs(9, lengths)
    HD = 2 * 8
    w1 = w1.copy(); b1 = b1.copy()
    w1[:HD] = 0.0; b1[:HD] = 0.0          # z_U = 0 -> U = SiLU(0) = 0 -> gate is 0
    y = O.layer_fwd(x, _jag(lengths, taus), w1, b1, w2, np.zeros_like(b2), wp, wt, 2, 8, 1e-6, 0)
    assert np.array_equal(y, x)


def test_layernorm_scale_invariance_eps0():
    # with eps = 0, scaling V (or c_b) scales O, and the norm removes it
    lengths = [15]
    rng, x, w1, b1, w2, b2, wp, wt, taus = _layer_inputs(10, lengths)
    jag = _jag(lengths, taus)
    u, v, q, k = O.projection(x, w1, b1, 2, 8)
    o = O.attn_fwd(jag, q, k, v, wp, wt)
    o2 = O.attn_fwd(_jag(lengths, taus, attn_scale=[0.013]), q, k, 4.0 * v, wp, wt)
    np.testing.assert_allclose(O.norm_gate(o, u, 0.0), O.norm_gate(o2, u, 0.0), rtol=1e-10, atol=1e-12)


def test_giant_gaps_and_duplicates():
    lengths = [6]
    rng, q, k, v, wp, wt, taus = _attn_inputs(11, lengths, Tb=64)
    taus = np.array([0, 0, 1 << 33, (1 << 33) + 1, (1 << 62), (1 << 62)], dtype=np.int64)
    out = O.attn_fwd(_jag(lengths, taus), q, k, v, wp, wt)
    # row 5 against row 0: gap 2**62 -> bucket 63; duplicates -> bucket 0
    assert O.time_bucket(np.array([taus[5]]), np.array([taus[0]]), 64)[0] == 63
    assert O.time_bucket(np.array([taus[1]]), np.array([taus[0]]), 64)[0] == 0
    assert np.isfinite(out).all()


# --------------------------------------------------------------------------- candidate-mask reductions
def _cand_setup(seed, n_hist, m, H=2, Dh=8, P=16, Tb=32):
    rng = np.random.default_rng(seed)
    n = n_hist + m
    q, k, v = rng.standard_normal((3, n, H, Dh))
    wp = rng.normal(0, 0.5, (1, P)); wt = rng.normal(0, 0.5, (1, Tb))
    t_hist = 1_000_000 + np.cumsum(rng.integers(1, 7200, size=n_hist))
    taus = np.concatenate([t_hist, np.full(m, t_hist[-1] + 999)])
    return q, k, v, wp, wt, taus


def test_candidates_history_rows_equal_plain_causal():
    n_hist, m = 25, 6
    q, k, v, wp, wt, taus = _cand_setup(12, n_hist, m)
    c = 1.0 / (n_hist + m)
    cand = O.attn_fwd(_jag([n_hist + m], taus, O.CAUSAL_CANDIDATES, [m]), q, k, v, wp, wt)
    hist = O.attn_fwd(_jag([n_hist], taus[:n_hist], attn_scale=[c]), q[:n_hist], k[:n_hist], v[:n_hist], wp, wt)
    assert np.array_equal(cand[:n_hist], hist)


def test_each_candidate_equals_history_plus_itself():
    n_hist, m = 19, 5
    q, k, v, wp, wt, taus = _cand_setup(13, n_hist, m)
    c = 1.0 / (n_hist + m)
    cand = O.attn_fwd(_jag([n_hist + m], taus, O.CAUSAL_CANDIDATES, [m]), q, k, v, wp, wt)
    for r in range(m):
        idx = np.concatenate([np.arange(n_hist), [n_hist + r]])
        one = O.attn_fwd(_jag([n_hist + 1], taus[idx], attn_scale=[c]), q[idx], k[idx], v[idx], wp, wt)
        np.testing.assert_allclose(cand[n_hist + r], one[-1], rtol=1e-13, atol=1e-15)


def test_candidates_do_not_see_each_other():
    n_hist, m = 14, 7
    q, k, v, wp, wt, taus = _cand_setup(14, n_hist, m)
    jag = _jag([n_hist + m], taus, O.CAUSAL_CANDIDATES, [m])
    base = O.attn_fwd(jag, q, k, v, wp, wt)
    # perturb candidate 3 only: every other row stays bitwise equal
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[n_hist + 3] += 1.0; k2[n_hist + 3] -= 1.0; v2[n_hist + 3] *= 3.0
    out = O.attn_fwd(jag, q2, k2, v2, wp, wt)
    keep = [i for i in range(n_hist + m) if i != n_hist + 3]
    assert np.array_equal(out[keep], base[keep])
    # permuting the candidates permutes their outputs
    perm = np.concatenate([np.arange(n_hist), n_hist + np.random.default_rng(0).permutation(m)])
    out_p = O.attn_fwd(jag, q[perm], k[perm], v[perm], wp, wt)
    np.testing.assert_allclose(out_p, base[perm], rtol=1e-13, atol=1e-15)


def test_no_candidates_equals_causal():
    lengths = [11, 6]
    rng, q, k, v, wp, wt, taus = _attn_inputs(15, lengths)
    a = O.attn_fwd(_jag(lengths, taus), q, k, v, wp, wt)
    b = O.attn_fwd(_jag(lengths, taus, O.CAUSAL_CANDIDATES, [0, 0]), q, k, v, wp, wt)
    assert np.array_equal(a, b)


def test_row_sample_matches_full():
    lengths = [50, 3]
    rng, q, k, v, wp, wt, taus = _attn_inputs(16, lengths)
    jag = _jag(lengths, taus)
    full = O.attn_fwd(jag, q, k, v, wp, wt)
    part = O.attn_fwd(jag, q, k, v, wp, wt, row_sample={0: np.array([0, 7, 49]), 1: np.array([2])})
    # same arithmetic; BLAS may block a 1-row product differently, so allow last-bit differences
    np.testing.assert_allclose(part[(0, 1)], full[[0, 7, 49], 1], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(part[(1, 0)], full[[52], 0], rtol=1e-14, atol=1e-15)
