"""Pins of the cached-history candidate scoring of the float64 oracle.

The scoring is defined to give exactly the candidate rows of the one-pass computation in which the
candidates are appended to the history (DLRMv4 page, "1つの訓練サンプルがHSTUでどのように処理されるか"),
with the same c_b; the one-pass attention is pinned separately (scalar loops, closed forms), so these
checks tie the cached path to it through code that shares no index or mask logic with it.
"""
import numpy as np
import pytest

from oracle import hstu_oracle as O


def _case(seed, hist_lens, cand_lens, H=2, Dh=8, P=16, Tb=32, R=1):
    rng = np.random.default_rng(seed)
    B = len(hist_lens)
    taus_h, taus_c = [], []
    for nh, m in zip(hist_lens, cand_lens):
        gaps = np.maximum(1, np.ceil(rng.exponential(3600.0, size=nh))).astype(np.int64)
        th = 1_700_000_000 + np.cumsum(gaps)
        taus_h.append(th)
        req = (th[-1] if nh else 1_700_000_000) + int(rng.integers(0, 5000))
        taus_c.append(np.full(m, req, dtype=np.int64))   # every candidate carries the request time
    Th, Tc = sum(hist_lens), sum(cand_lens)
    kh, vh = rng.standard_normal((2, Th, H, Dh))
    q, k, v = rng.standard_normal((3, Tc, H, Dh))
    qh = rng.standard_normal((Th, H, Dh))
    wp, wt = rng.normal(0, 0.5, (R, P)), rng.normal(0, 0.5, (R, Tb))
    ho = np.concatenate([[0], np.cumsum(hist_lens)]).astype(np.int64)
    co = np.concatenate([[0], np.cumsum(cand_lens)]).astype(np.int64)
    hist = dict(seq_offsets=ho, timestamps=np.concatenate(taus_h) if Th else np.zeros(0, np.int64))
    cand = dict(seq_offsets=co, timestamps=np.concatenate(taus_c) if Tc else np.zeros(0, np.int64))
    return hist, cand, qh, kh, vh, q, k, v, wp, wt


def _one_pass(hist, cand, qh, kh, vh, q, k, v, wp, wt):
    """The candidate-masked one-pass attention over [history | candidates] per user; returns the
    candidate rows in candidate order."""
    ho, co = hist["seq_offsets"], cand["seq_offsets"]
    B = len(ho) - 1
    parts_q, parts_k, parts_v, parts_t, lens, ms = [], [], [], [], [], []
    for b in range(B):
        h0, h1, c0, c1 = ho[b], ho[b + 1], co[b], co[b + 1]
        parts_q += [qh[h0:h1], q[c0:c1]]
        parts_k += [kh[h0:h1], k[c0:c1]]
        parts_v += [vh[h0:h1], v[c0:c1]]
        parts_t += [hist["timestamps"][h0:h1], cand["timestamps"][c0:c1]]
        lens.append((h1 - h0) + (c1 - c0))
        ms.append(c1 - c0)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    jag = dict(seq_offsets=offs, timestamps=np.concatenate(parts_t), mask=O.CAUSAL_CANDIDATES,
               num_candidates=np.asarray(ms), attn_scale=None)
    full = O.attn_fwd(jag, np.concatenate(parts_q), np.concatenate(parts_k), np.concatenate(parts_v), wp, wt)
    rows = np.concatenate([np.arange(offs[b + 1] - ms[b], offs[b + 1]) for b in range(B)]).astype(np.int64)
    scales = np.asarray([1.0 / n if n else 0.0 for n in lens])
    return full[rows], scales


@pytest.mark.parametrize("seed,hist_lens,cand_lens,R", [
    (0, [5, 0, 37, 1], [3, 4, 1, 6], 1),
    (1, [64, 130, 0, 9], [17, 1, 2, 33], 2),
    (2, [300, 2], [40, 0], 1),
])
def test_cached_equals_one_pass_candidate_rows(seed, hist_lens, cand_lens, R):
    hist, cand, qh, kh, vh, q, k, v, wp, wt = _case(seed, hist_lens, cand_lens, R=R)
    want, _ = _one_pass(hist, cand, qh, kh, vh, q, k, v, wp, wt)
    got = O.attn_cached(hist, cand, kh, vh, q, k, v, wp, wt)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_micro_batches_with_the_full_scale_reassemble_the_one_pass_rows():
    hist_lens, cand_lens = [50, 3, 120], [23, 9, 31]
    hist, cand, qh, kh, vh, q, k, v, wp, wt = _case(7, hist_lens, cand_lens, R=2)
    want, scales = _one_pass(hist, cand, qh, kh, vh, q, k, v, wp, wt)
    co = cand["seq_offsets"]
    rng = np.random.default_rng(8)
    got = np.zeros_like(want)
    # cut every user's candidates at random points; micro-batch t takes piece t of every user
    cuts = [np.sort(rng.choice(np.arange(1, m), size=2, replace=False)) for m in cand_lens]
    for t in range(3):
        sel = []
        for b, m in enumerate(cand_lens):
            edges = [0, *cuts[b], m]
            sel.append(np.arange(co[b] + edges[t], co[b] + edges[t + 1]))
        mb_offs = np.concatenate([[0], np.cumsum([len(x) for x in sel])]).astype(np.int64)
        idx = np.concatenate(sel)
        mb = dict(seq_offsets=mb_offs, timestamps=cand["timestamps"][idx])
        got[idx] = O.attn_cached(hist, mb, kh, vh, q[idx], k[idx], v[idx], wp, wt, attn_scale=scales)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_no_history_closed_form():
    hist, cand, qh, kh, vh, q, k, v, wp, wt = _case(11, [0, 0], [3, 1])
    got = O.attn_cached(hist, cand, kh, vh, q, k, v, wp, wt)
    co = cand["seq_offsets"]
    for b in range(2):
        m = co[b + 1] - co[b]
        for c in range(co[b], co[b + 1]):
            for h in range(q.shape[1]):
                s = float(q[c, h] @ k[c, h]) + wp[0, 0] + wt[0, 0]
                want = (1.0 / m) * (s / (1.0 + np.exp(-s))) * v[c, h]
                np.testing.assert_allclose(got[c, h], want, rtol=1e-13, atol=1e-14)
