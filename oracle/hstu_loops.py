"""Scalar, per-element Python loops of the HSTU layer forward -- TEST INFRASTRUCTURE ONLY.

A second, independently written statement of the same definition as ``hstu_oracle`` (which it
does not import): Python floats and Python integers, one multiply-add at a time.  It is far too slow
for anything but tiny inputs and exists to cross-check the vectorised float64 oracle.
Definition and sources: see the header of ``hstu_oracle`` (the HSTU abstract page and the DLRMv4
page, sections on the model architecture and on how one training sample is processed).
"""
from __future__ import annotations

import math

CAUSAL = 0
CAUSAL_CANDIDATES = 1


def _silu(z: float) -> float:
    # z * sigmoid(z), written through the logistic function on each side of 0 to avoid overflow
    if z >= 0:
        return z / (1.0 + math.exp(-z))
    e = math.exp(z)
    return z * e / (1.0 + e)


def _bucket_pos(pi: int, pj: int, P: int) -> int:
    return min(abs(pi - pj), P - 1)


def _bucket_time(ti: int, tj: int, Tb: int) -> int:
    return min(abs(int(ti) - int(tj)).bit_length(), Tb - 1)


def _allowed(i: int, j: int, n_hist: int, mask: int) -> bool:
    if mask == CAUSAL:
        return j <= i
    if i < n_hist:
        return j <= i
    return j < n_hist or j == i


def attn_fwd_loops(offsets, timestamps, q, k, v, pos_bias, time_bias, mask=CAUSAL, num_candidates=None,
                   attn_scale=None):
    """Nested lists in, nested lists out: q, k, v indexable as [t][h][d]; returns O [T][H][Dh]."""
    T = offsets[-1]
    H = len(q[0]) if T else 0
    Dh = len(q[0][0]) if T else 0
    R = len(pos_bias)
    P, Tb = len(pos_bias[0]), len(time_bias[0])
    out = [[[0.0] * Dh for _ in range(H)] for _ in range(T)]
    for b in range(len(offsets) - 1):
        o0, o1 = int(offsets[b]), int(offsets[b + 1])
        n = o1 - o0
        if n == 0:
            continue
        m = int(num_candidates[b]) if mask == CAUSAL_CANDIDATES else 0
        n_hist = n - m
        c = (1.0 / n) if attn_scale is None else float(attn_scale[b])
        for h in range(H):
            r = 0 if R == 1 else h
            for i in range(n):
                pi = i if mask == CAUSAL else min(i, n_hist)
                acc = [0.0] * Dh
                for j in range(n):
                    if not _allowed(i, j, n_hist, mask):
                        continue
                    pj = j if mask == CAUSAL else min(j, n_hist)
                    s = 0.0
                    for d in range(Dh):
                        s += float(q[o0 + i][h][d]) * float(k[o0 + j][h][d])
                    s += float(pos_bias[r][_bucket_pos(pi, pj, P)])
                    s += float(time_bias[r][_bucket_time(timestamps[o0 + i], timestamps[o0 + j], Tb)])
                    a = _silu(s)
                    for d in range(Dh):
                        acc[d] += a * float(v[o0 + j][h][d])
                for d in range(Dh):
                    out[o0 + i][h][d] = c * acc[d]
    return out


def _layer_norm_row(row, eps):
    n = len(row)
    mu = sum(row) / n
    var = sum((x - mu) * (x - mu) for x in row) / n
    inv = 1.0 / math.sqrt(var + eps)
    return [(x - mu) * inv for x in row]


def layer_fwd_loops(x, offsets, timestamps, w_uvqk, b_uvqk, w_out, b_out, pos_bias, time_bias, H, Dh,
                    eps, ln_output, mask=CAUSAL, num_candidates=None, attn_scale=None):
    """x: [T][D]; w_uvqk: [4*H*Dh][D]; w_out: [D][H*Dh]; returns y [T][D] (Python floats)."""
    T = len(x)
    D = len(x[0]) if T else 0
    HD = H * Dh
    z = []
    for t in range(T):
        zt = []
        for c in range(4 * HD):
            acc = 0.0 if b_uvqk is None else float(b_uvqk[c])
            for d in range(D):
                acc += float(w_uvqk[c][d]) * float(x[t][d])
            zt.append(_silu(acc))
        z.append(zt)
    # columns: U | V | Q | K, each head-major [h][d]
    def part(p):
        return [[[z[t][p * HD + h * Dh + d] for d in range(Dh)] for h in range(H)] for t in range(T)]
    u, v, q, k = part(0), part(1), part(2), part(3)
    o = attn_fwd_loops(offsets, timestamps, q, k, v, pos_bias, time_bias, mask, num_candidates, attn_scale)
    y = []
    for t in range(T):
        flat_o = [o[t][h][d] for h in range(H) for d in range(Dh)]
        flat_u = [u[t][h][d] for h in range(H) for d in range(Dh)]
        nrm = _layer_norm_row(flat_o, eps)
        g = [nrm[i] * flat_u[i] for i in range(HD)]
        yt = []
        for c in range(D):
            acc = float(x[t][c]) + (0.0 if b_out is None else float(b_out[c]))
            for i in range(HD):
                acc += float(w_out[c][i]) * g[i]
            yt.append(acc)
        if ln_output:
            yt = _layer_norm_row(yt, eps)
        y.append(yt)
    return y


def softmax_attn_loops(offsets, q, k, v):
    """Causal softmax attention, one score at a time: O_i = sum_{j<=i} w_ij v_j with
    w_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij), s_ij = q_i . k_j / sqrt(Dh)."""
    T, H, Dh = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * Dh for _ in range(H)] for _ in range(T)]
    for b in range(len(offsets) - 1):
        o0, o1 = int(offsets[b]), int(offsets[b + 1])
        for h in range(H):
            for i in range(o1 - o0):
                s = []
                for j in range(i + 1):
                    acc = 0.0
                    for d in range(Dh):
                        acc += float(q[o0 + i][h][d]) * float(k[o0 + j][h][d])
                    s.append(acc / math.sqrt(Dh))
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for d in range(Dh):
                    out[o0 + i][h][d] = sum(e[j] / z * float(v[o0 + j][h][d]) for j in range(i + 1))
    return out
