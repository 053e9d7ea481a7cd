"""Pins of the float64 attention backward (oracle.attn_bwd).

The gradients are checked against central finite differences of the forward oracle, whose own pins
(scalar loops, closed forms, invariants) are elsewhere; the difference quotient knows nothing of the
backward formulas, so a dropped term, a wrong sign, a missing SiLU' factor, a transposed product or a
bucket sent to the wrong bin fails here.
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


def _inputs(seed, lengths, H=2, Dh=4, P=5, Tb=6, R=1):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    q, k, v, g = rng.standard_normal((4, T, H, Dh))
    wp, wt = rng.normal(0, 0.7, (R, P)), rng.normal(0, 0.7, (R, Tb))
    taus = []
    for n in lengths:
        taus.append(1_700_000_000 + np.cumsum(rng.integers(1, 40, size=n)))
    return q, k, v, g, wp, wt, np.concatenate(taus)


def _loss(jag, q, k, v, wp, wt, g):
    return float(np.sum(O.attn_fwd(jag, q, k, v, wp, wt) * g))


def _fd(f, x, eps=1e-6):
    """Central differences of the scalar f with respect to every entry of x (modified in place)."""
    out = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps; fp = f()
        x[i] = old - eps; fm = f()
        x[i] = old
        out[i] = (fp - fm) / (2 * eps)
    return out


@pytest.mark.parametrize("mask,lengths,m,R,scale", [
    (O.CAUSAL, [5, 1, 7], None, 1, None),
    (O.CAUSAL, [6, 4], None, 2, [0.5, -1.5]),
    (O.CAUSAL_CANDIDATES, [7, 5], [3, 2], 2, None),
])
def test_gradients_match_finite_differences(mask, lengths, m, R, scale):
    q, k, v, g, wp, wt, tau = _inputs(len(lengths) + (m or [0])[0] + R, lengths, R=R)
    jag = _jag(lengths, tau, mask, m, scale)
    dq, dk, dv, dwp, dwt = O.attn_bwd(jag, q, k, v, wp, wt, g)
    f = lambda: _loss(jag, q, k, v, wp, wt, g)
    for got, x, name in [(dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv"), (dwp, wp, "d_pos_bias"),
                         (dwt, wt, "d_time_bias")]:
        want = _fd(f, x)
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7, err_msg=name)


def test_bias_gradients_each_sum_to_the_total_score_gradient():
    """Every allowed pair lands in exactly one position bin and one time bin."""
    lengths = [9, 3, 12]
    q, k, v, g, wp, wt, tau = _inputs(5, lengths, H=3, P=4, Tb=3, R=3)
    jag = _jag(lengths, tau)
    dq, dk, dv, dwp, dwt = O.attn_bwd(jag, q, k, v, wp, wt, g)
    np.testing.assert_allclose(dwp.sum(axis=1), dwt.sum(axis=1), rtol=1e-12, atol=1e-12)
    # and the position-bin sum equals the gradient of a constant added to every score of head r
    eps = 1e-6
    for r in range(3):
        up, dn = wp.copy(), wp.copy()
        up[r] += eps; dn[r] -= eps
        fd = (_loss(jag, q, k, v, up, wt, g) - _loss(jag, q, k, v, dn, wt, g)) / (2 * eps)
        np.testing.assert_allclose(dwp[r].sum(), fd, rtol=1e-6, atol=1e-7)


def test_zero_upstream_gradient_gives_zero():
    lengths = [4, 6]
    q, k, v, g, wp, wt, tau = _inputs(9, lengths)
    jag = _jag(lengths, tau)
    for x in O.attn_bwd(jag, q, k, v, wp, wt, np.zeros_like(g)):
        assert not np.any(x)


def test_bin_sums_of_squares():
    """Every allowed pair adds its dS^2 to one position bin and one time bin (equal totals, each bin at
    least its sum squared over its pair count), and a one-token sequence has the single pair's dS^2."""
    lengths = [9, 3, 12]
    q, k, v, g, wp, wt, tau = _inputs(6, lengths, H=2, P=4, Tb=3, R=1)
    jag = _jag(lengths, tau)
    dq, dk, dv, dwp, dwt, sqp, sqt = O.attn_bwd(jag, q, k, v, wp, wt, g, return_sq=True)
    np.testing.assert_allclose(sqp.sum(), sqt.sum(), rtol=1e-12)
    assert np.all(sqp >= 0) and np.all(sqt >= 0)
    n_pairs = 2 * sum(n * (n + 1) // 2 for n in lengths)
    assert np.all(sqp * n_pairs >= dwp ** 2 - 1e-12)
    q1, k1, v1, g1, wp1, wt1, tau1 = _inputs(7, [1], H=1, P=4, Tb=3, R=1)
    jag1 = _jag([1], tau1)
    *_, sqp1, sqt1 = O.attn_bwd(jag1, q1, k1, v1, wp1, wt1, g1, return_sq=True)
    s = q1[0, 0] @ k1[0, 0] + wp1[0, 0] + wt1[0, 0]
    ds = (g1[0, 0] @ v1[0, 0]) * O.silu_grad(s)
    np.testing.assert_allclose(sqp1[0, 0], ds ** 2, rtol=1e-12)
    np.testing.assert_allclose(sqt1[0, 0], ds ** 2, rtol=1e-12)


@pytest.mark.parametrize("mask", [O.CAUSAL, O.CAUSAL_CANDIDATES])
def test_sampled_rows_and_columns_match_the_full_backward(mask):
    """attn_bwd_sampled restricts attn_bwd (pinned above to finite differences) to single query rows and
    key rows: equal to it on every sampled row, per-head tables, both masks."""
    lengths = [11, 1, 17]
    q, k, v, g, wp, wt, tau = _inputs(12, lengths, H=3, P=6, Tb=5, R=3)
    cands = [4, 1, 6] if mask == O.CAUSAL_CANDIDATES else None
    jag = _jag(lengths, tau, mask=mask, num_candidates=cands, attn_scale=[0.3, 1.0, -0.7])
    dq, dk, dv, _, _ = O.attn_bwd(jag, q, k, v, wp, wt, g)
    offs = jag["seq_offsets"]
    for b, rows, cols in [(0, [0, 3, 10], [0, 5, 10]), (1, [0], [0]), (2, [16, 2, 11, 12], [1, 12, 16])]:
        for h in range(3):
            sq, sk, sv = O.attn_bwd_sampled(jag, q, k, v, wp, wt, g, b, h, rows, cols)
            o0 = int(offs[b])
            np.testing.assert_allclose(sq, dq[o0 + np.asarray(rows), h], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(sk, dk[o0 + np.asarray(cols), h], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(sv, dv[o0 + np.asarray(cols), h], rtol=1e-12, atol=1e-13)
