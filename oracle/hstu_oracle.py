"""Float64 CPU oracle of the HSTU layer (forward and its gradients) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may import this
module.  The HIP library never calls it, and it imports nothing from the library: it depends on
numpy alone.  Inputs are the exact storage values (bf16 or fp32) upcast to float64.

Sources (the pages):
  [HSTU]   "Actions Speak Louder than Words: Trillion-Parameter Sequential Transducers for
           Generative Recommendations" -- abstract: HSTU is an attention variant for
           high-cardinality, non-stationary streaming data; 8192-length sequences.
  [DLRMv4] "DLRMv4：MLPerfの推薦システム訓練ベンチマークがシーケンス化時代へ"
           - section "モデルアーキテクチャ：HSTUが従来の特徴インタラクションスタックに取って代わる"
             (Model architecture): inside a layer, one projection makes every internal
             representation; pointwise attention aggregates the sequence with a bias from the
             positional and the temporal distance of two events; a gated transformation lets the
             aggregated features interact and takes the place of cross network and feed-forward.
           - section "1つの訓練サンプルがHSTUでどのように処理されるか" (one training sample):
             a time-ordered per-user event stream, candidates appended at the end and scored in
             one forward pass, the whole sequence processed as one causal block.

The pages give the structure but no formulas.  The formulas below are the plainest reading of it
(each reading is listed with its alternatives in the design notes of this repository):
  1. z = W1 x + b1; SiLU on all of z; U | V | Q | K are the four consecutive H*Dh slices, head-major.
  2. s_ij = q_i . k_j + w_p[bp(i,j)] + w_t[bt(i,j)]   (no 1/sqrt(Dh) scale)
       bp = min(|pos(i) - pos(j)|, P-1);  bt = min(bitlen(|tau_i - tau_j|), Tb-1), exact integers,
       bitlen(0) = 0, bitlen(g) = floor(log2 g) + 1.
     a_ij = SiLU(s_ij) on allowed pairs, 0 elsewhere.  No softmax.
  3. O_i = c_b * sum_j a_ij v_j,  c_b = 1/n_b unless given per sequence.
  4. y = x + W2 (LN(concat_h O) * U) + b2; LN over H*Dh, biased variance, no affine, eps given;
     between stacked layers y <- LN(y).
Masks: CAUSAL allows j <= i.  CAUSAL_CANDIDATES (the last m_b tokens of a sequence are candidates,
n_h = n_b - m_b): a history row i < n_h allows j <= i; a candidate row allows every j < n_h and j = i;
every candidate has position n_h.

Functions whose result has no independent pin are marked "parity unpinned" in their docstring.
"""
from __future__ import annotations

import numpy as np

CAUSAL = 0
CAUSAL_CANDIDATES = 1

_ROW_BLOCK = 1024


# --------------------------------------------------------------------------- elementwise pieces
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), float64.  e^-z may overflow to inf for z << 0,
    which gives the correct limit -0."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def abs_diff_u64(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| for int64 a, b as exact uint64 (the true difference always fits in 64 unsigned bits;
    unsigned subtraction of the larger minus the smaller is exact modulo 2**64)."""
    a, b = np.broadcast_arrays(np.asarray(a, dtype=np.int64), np.asarray(b, dtype=np.int64))
    au, bu = a.view(np.uint64), b.view(np.uint64)
    return np.where(a >= b, au - bu, bu - au).astype(np.uint64)


def bitlen_u64(g: np.ndarray) -> np.ndarray:
    """Number of significant bits of unsigned 64-bit integers (0 -> 0), by binary lifting."""
    x = np.array(g, dtype=np.uint64, copy=True)
    n = np.zeros(x.shape, dtype=np.int64)
    for s in (32, 16, 8, 4, 2, 1):
        big = x >= np.uint64(1 << s)
        n[big] += s
        x[big] >>= np.uint64(s)
    return n + (x > 0)


def position_bucket(pos_i: np.ndarray, pos_j: np.ndarray, P: int) -> np.ndarray:
    """bp = min(|pos_i - pos_j|, P - 1) (position distance, [DLRMv4] Model architecture)."""
    return np.minimum(np.abs(np.asarray(pos_i, np.int64) - np.asarray(pos_j, np.int64)), P - 1)


def time_bucket(tau_i: np.ndarray, tau_j: np.ndarray, Tb: int) -> np.ndarray:
    """bt = min(bitlen(|tau_i - tau_j|), Tb - 1): log2 buckets of the time gap, exact in integers
    (temporal distance, [DLRMv4] Model architecture)."""
    return np.minimum(bitlen_u64(abs_diff_u64(tau_i, tau_j)), Tb - 1)


def positions(n: int, n_hist: int, mask: int) -> np.ndarray:
    """Token positions inside a sequence: i for CAUSAL; min(i, n_h) for CAUSAL_CANDIDATES."""
    i = np.arange(n, dtype=np.int64)
    return i if mask == CAUSAL else np.minimum(i, n_hist)


def allowed(rows: np.ndarray, n: int, n_hist: int, mask: int) -> np.ndarray:
    """Boolean [len(rows), n]: which (i, j) pairs contribute ([DLRMv4] one training sample: one causal
    block; candidates appended at the end see the full history)."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n, dtype=np.int64)[None, :]
    if mask == CAUSAL:
        return j <= i
    hist_row = (i < n_hist) & (j <= i)
    cand_row = (i >= n_hist) & ((j < n_hist) | (j == i))
    return hist_row | cand_row


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """Row LayerNorm over the last axis: (x - mean) / sqrt(biased var + eps), no affine."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


# --------------------------------------------------------------------------- attention
def attn_sequence_head(q, k, v, tau, wp, wt, mask, n_hist, scale, rows=None):
    """Pointwise attention for one sequence and one head.

    q, k, v: [n, Dh] float64; tau: int64 [n]; wp: [P]; wt: [Tb]; returns O[rows]: [len(rows), Dh].
    Steps 2 and 3 of the layer ([DLRMv4] Model architecture: pointwise attention with a
    position/time-distance bias; [HSTU] abstract: attention variant, no softmax normaliser here).
    """
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    P, Tb = len(wp), len(wt)
    pos = positions(n, n_hist, mask)
    out = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    for s in range(0, len(rows), _ROW_BLOCK):
        r = rows[s:s + _ROW_BLOCK]
        scores = q[r] @ k.T
        scores = scores + wp[position_bucket(pos[r][:, None], pos[None, :], P)]
        scores = scores + wt[time_bucket(tau[r][:, None], tau[None, :], Tb)]
        a = np.where(allowed(r, n, n_hist, mask), silu(scores), 0.0)
        out[s:s + _ROW_BLOCK] = scale * (a @ v)
    return out


def _seq_params(jag, b):
    o0, o1 = int(jag["seq_offsets"][b]), int(jag["seq_offsets"][b + 1])
    n = o1 - o0
    mask = int(jag.get("mask", CAUSAL))
    m = 0
    if mask == CAUSAL_CANDIDATES:
        m = int(jag["num_candidates"][b])
    n_hist = n - m
    sc = jag.get("attn_scale")
    scale = (1.0 / n if n else 0.0) if sc is None else float(sc[b])
    return o0, o1, n, n_hist, mask, scale


def attn_fwd(jag: dict, q, k, v, pos_bias, time_bias, row_sample=None):
    """O = attention output [T, H, Dh] in float64.

    jag: dict with seq_offsets int [B+1], timestamps int64 [T], mask, num_candidates [B] (candidates
    mask only), attn_scale [B] or None.  q, k, v: [T, H, Dh]; pos_bias [R, P]; time_bias [R, Tb]
    (R = 1 shared by all heads, or R = H, one row per head).
    row_sample: optional dict b -> local row indices; then only those rows are computed and the
    result is a dict (b, h) -> [rows, Dh].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    wp = np.asarray(pos_bias, np.float64)
    wt = np.asarray(time_bias, np.float64)
    tau = np.asarray(jag["timestamps"], np.int64)
    T, H, Dh = q.shape
    B = len(jag["seq_offsets"]) - 1
    R = wp.shape[0]
    out = {} if row_sample is not None else np.zeros((T, H, Dh), dtype=np.float64)
    for b in range(B):
        o0, o1, n, n_hist, mask, scale = _seq_params(jag, b)
        if n == 0:
            continue
        if row_sample is not None and b not in row_sample:
            continue
        for h in range(H):
            r = 0 if R == 1 else h
            rows = None if row_sample is None else row_sample[b]
            o = attn_sequence_head(q[o0:o1, h], k[o0:o1, h], v[o0:o1, h], tau[o0:o1], wp[r], wt[r],
                                   mask, n_hist, scale, rows)
            if row_sample is None:
                out[o0:o1, h] = o
            else:
                out[(b, h)] = o
    return out


# --------------------------------------------------------------------------- attention backward
def silu_grad(z: np.ndarray) -> np.ndarray:
    """d SiLU / dz = sigma(z) (1 + z (1 - sigma(z))), float64 (the derivative of z * sigma(z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-z))
    return sig * (1.0 + z * (1.0 - sig))


def attn_bwd(jag: dict, q, k, v, pos_bias, time_bias, d_out, return_sq=False):
    """Gradients of the pointwise attention (the forward of attn_fwd) for an upstream gradient d_out.

    Returns (dq, dk, dv, d_pos_bias, d_time_bias) in float64: [T, H, Dh] x 3, [R, P], [R, Tb]; with
    return_sq also the per-bin sums of squares of the summed terms, sum of dS_ij^2 ([R, P] and
    [R, Tb]): the scale of a bin's rounding noise when each term carries an independent error.
    With a_ij = SiLU(s_ij) on allowed pairs and O_i = c_b sum_j a_ij v_j:
        dv_j = c_b sum_i a_ij dO_i,   dA_ij = c_b dO_i . v_j,   dS_ij = dA_ij SiLU'(s_ij) (allowed pairs),
        dq_i = sum_j dS_ij k_j,   dk_j = sum_i dS_ij q_i,
        d w_p[r][p] = sum of dS_ij over the pairs with bp(i, j) = p (heads of table row r, all sequences),
        d w_t[r][t] likewise with bt(i, j) = t.
    c_b is a constant (no gradient).  No softmax, hence no normaliser term.
    """
    q, k, v, g = (np.asarray(a, np.float64) for a in (q, k, v, d_out))
    wp = np.asarray(pos_bias, np.float64)
    wt = np.asarray(time_bias, np.float64)
    tau = np.asarray(jag["timestamps"], np.int64)
    T, H, Dh = q.shape
    R, P, Tb = wp.shape[0], wp.shape[1], wt.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dwp, dwt = np.zeros_like(wp), np.zeros_like(wt)
    sqp, sqt = np.zeros_like(wp), np.zeros_like(wt)
    B = len(jag["seq_offsets"]) - 1
    for b in range(B):
        o0, o1, n, n_hist, mask, scale = _seq_params(jag, b)
        if n == 0:
            continue
        pos = positions(n, n_hist, mask)
        bp = position_bucket(pos[:, None], pos[None, :], P)
        bt = time_bucket(tau[o0:o1][:, None], tau[o0:o1][None, :], Tb)
        ok = allowed(np.arange(n), n, n_hist, mask)
        for h in range(H):
            r = 0 if R == 1 else h
            qh, kh, vh, gh = q[o0:o1, h], k[o0:o1, h], v[o0:o1, h], g[o0:o1, h]
            s = qh @ kh.T + wp[r][bp] + wt[r][bt]
            a = np.where(ok, silu(s), 0.0)
            dv[o0:o1, h] = scale * (a.T @ gh)
            ds = np.where(ok, scale * (gh @ vh.T) * silu_grad(s), 0.0)
            dq[o0:o1, h] = ds @ kh
            dk[o0:o1, h] = ds.T @ qh
            dwp[r] += np.bincount(bp[ok], weights=ds[ok], minlength=P)
            dwt[r] += np.bincount(bt[ok], weights=ds[ok], minlength=Tb)
            if return_sq:
                sqp[r] += np.bincount(bp[ok], weights=ds[ok] ** 2, minlength=P)
                sqt[r] += np.bincount(bt[ok], weights=ds[ok] ** 2, minlength=Tb)
    if return_sq:
        return dq, dk, dv, dwp, dwt, sqp, sqt
    return dq, dk, dv, dwp, dwt


def attn_bwd_sampled(jag: dict, q, k, v, pos_bias, time_bias, d_out, b, h, rows, cols):
    """dq for the query rows `rows` and dk, dv for the key rows `cols` of sequence b, head h, in float64:
    attn_bwd's definitions restricted to one row of S and dP per sampled query and one column per
    sampled key, so that single rows of a long sequence can be checked without the n x n products."""
    q, k, v, g = (np.asarray(a, np.float64) for a in (q, k, v, d_out))
    wp = np.asarray(pos_bias, np.float64)
    wt = np.asarray(time_bias, np.float64)
    tau = np.asarray(jag["timestamps"], np.int64)
    R, P, Tb = wp.shape[0], wp.shape[1], wt.shape[1]
    r = 0 if R == 1 else h
    o0, o1, n, n_hist, mask, scale = _seq_params(jag, b)
    pos = positions(n, n_hist, mask)
    tb = tau[o0:o1]
    qh, kh, vh, gh = q[o0:o1, h], k[o0:o1, h], v[o0:o1, h], g[o0:o1, h]
    ri = np.asarray(rows, dtype=np.int64)
    s = (qh[ri] @ kh.T + wp[r][position_bucket(pos[ri][:, None], pos[None, :], P)]
         + wt[r][time_bucket(tb[ri][:, None], tb[None, :], Tb)])
    ds = np.where(allowed(ri, n, n_hist, mask), scale * (gh[ri] @ vh.T) * silu_grad(s), 0.0)
    dq = ds @ kh
    cj = np.asarray(cols, dtype=np.int64)
    s2 = (qh @ kh[cj].T + wp[r][position_bucket(pos[:, None], pos[cj][None, :], P)]
          + wt[r][time_bucket(tb[:, None], tb[cj][None, :], Tb)])
    ok2 = allowed(np.arange(n), n, n_hist, mask)[:, cj]
    dv = scale * (np.where(ok2, silu(s2), 0.0).T @ gh)
    ds2 = np.where(ok2, scale * (gh @ vh[cj].T) * silu_grad(s2), 0.0)
    dk = ds2.T @ qh
    return dq, dk, dv


# --------------------------------------------------------------------------- cached-history scoring
def attn_cached(hist: dict, cand: dict, k_hist, v_hist, q, k, v, pos_bias, time_bias, attn_scale=None):
    """Candidates scored against a cached user history: O [T_c, H, Dh] in float64.

    Mini-batched candidate scoring ([HSTU] key contributions / technical approach: M-FALCON scores
    candidates in mini-batches), read as: each user's history keys, values and timestamps are
    computed once; a call scores some of that user's candidates, each against the whole history and
    itself only ([DLRMv4] one training sample: candidates appended to the history see all of it).
    hist: seq_offsets [B+1] into the history rows, timestamps [T_h]; cand: seq_offsets [B+1] into the
    candidate rows, timestamps [T_c].  k_hist, v_hist: [T_h, H, Dh]; q, k, v: [T_c, H, Dh].
    Candidate c of user b (n_h history tokens, m_b candidates in this call) has position n_h:
        s_cj = q_c . k_j + w_p[min(n_h - j, P - 1)] + w_t[bt(tau_c, tau_j)]   for history j < n_h
        s_cc = q_c . k_c + w_p[0] + w_t[0]                                     (itself: both distances 0)
        O_c  = c_b * (sum_j SiLU(s_cj) v_j + SiLU(s_cc) v_c),  c_b = attn_scale[b] or 1 / (n_h + m_b)
    """
    k_hist = np.asarray(k_hist, np.float64)
    v_hist = np.asarray(v_hist, np.float64)
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    wp = np.asarray(pos_bias, np.float64)
    wt = np.asarray(time_bias, np.float64)
    th = np.asarray(hist["timestamps"], np.int64)
    tc = np.asarray(cand["timestamps"], np.int64)
    ho = np.asarray(hist["seq_offsets"], np.int64)
    co = np.asarray(cand["seq_offsets"], np.int64)
    T_c, H, Dh = q.shape
    R, P, Tb = wp.shape[0], wp.shape[1], wt.shape[1]
    out = np.zeros((T_c, H, Dh), dtype=np.float64)
    for b in range(len(co) - 1):
        h0, h1, c0, c1 = int(ho[b]), int(ho[b + 1]), int(co[b]), int(co[b + 1])
        n_h, m = h1 - h0, c1 - c0
        if m == 0:
            continue
        scale = 1.0 / (n_h + m) if attn_scale is None else float(attn_scale[b])
        j = np.arange(n_h, dtype=np.int64)
        bp = np.minimum(n_h - j, P - 1)                                        # [n_h]
        bt = time_bucket(tc[c0:c1][:, None], th[h0:h1][None, :], Tb)          # [m, n_h]
        for h in range(H):
            r = 0 if R == 1 else h
            qh = q[c0:c1, h]
            s_hist = qh @ k_hist[h0:h1, h].T + wp[r][bp][None, :] + wt[r][bt]
            s_self = np.sum(qh * k[c0:c1, h], axis=1) + wp[r][0] + wt[r][0]
            out[c0:c1, h] = scale * (silu(s_hist) @ v_hist[h0:h1, h] + silu(s_self)[:, None] * v[c0:c1, h])
    return out


# --------------------------------------------------------------------------- layer, stack, gather
def projection(x, w_uvqk, b_uvqk, num_heads, head_dim):
    """Step 1 ([DLRMv4] Model architecture: a single projection makes all internal representations):
    SiLU(x W1^T + b1), split into U, V, Q, K, each [T, H, Dh]."""
    x = np.asarray(x, np.float64)
    z = x @ np.asarray(w_uvqk, np.float64).T
    if b_uvqk is not None:
        z = z + np.asarray(b_uvqk, np.float64)
    z = silu(z)
    T = x.shape[0]
    hd = num_heads * head_dim
    u, v, q, k = (z[:, c * hd:(c + 1) * hd].reshape(T, num_heads, head_dim) for c in range(4))
    return u, v, q, k


def norm_gate(o, u, eps):
    """Step 4a ([DLRMv4] Model architecture: gated transformation): LN(concat_h O) * U, [T, H*Dh]."""
    T = o.shape[0]
    return layer_norm(o.reshape(T, -1), eps) * np.asarray(u, np.float64).reshape(T, -1)


def layer_fwd(x, jag, w_uvqk, b_uvqk, w_out, b_out, pos_bias, time_bias, num_heads, head_dim,
              ln_eps, ln_output, return_parts=False):
    """One HSTU layer: projection, pointwise attention, norm-gate, output projection and residual
    (plus the post-layer LayerNorm when ln_output)."""
    x = np.asarray(x, np.float64)
    u, v, q, k = projection(x, w_uvqk, b_uvqk, num_heads, head_dim)
    o = attn_fwd(jag, q, k, v, pos_bias, time_bias)
    g = norm_gate(o, u, ln_eps)
    y = x + g @ np.asarray(w_out, np.float64).T
    if b_out is not None:
        y = y + np.asarray(b_out, np.float64)
    if ln_output:
        y = layer_norm(y, ln_eps)
    if return_parts:
        return y, dict(u=u, v=v, q=q, k=k, o=o, g=g)
    return y


def layer_norm_bwd(x, eps, dy):
    """Gradient of y = layer_norm(x, eps) over the last axis for an upstream gradient dy, float64.
    With x_hat = (x - mean) * rstd and rstd = 1/sqrt(var + eps):
        dx = rstd * (dy - mean(dy) - x_hat * mean(dy * x_hat)).
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xh = (x - mu) * rstd
    return rstd * (dy - dy.mean(axis=-1, keepdims=True) - xh * (dy * xh).mean(axis=-1, keepdims=True))


def round_bf16(a) -> np.ndarray:
    """Each value rounded to the nearest bfloat16 (8 significant bits, ties to even), returned as
    float64: the float32 value of the input keeps its top 16 bits after rounding."""
    f = np.asarray(a, np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def layer_bwd(x, jag, w_uvqk, b_uvqk, w_out, b_out, pos_bias, time_bias, num_heads, head_dim,
              ln_eps, ln_output, dy, return_sq=False, bf16_attention=False, attn_operands=None):
    """Gradients of layer_fwd for an upstream gradient dy of its output y (the layer is trained:
    [DLRMv4] describes a training benchmark).  Returns a dict of float64 arrays:
        dx [T, D], d_w_uvqk [4*H*Dh, D], d_b_uvqk [4*H*Dh], d_w_out [D, H*Dh], d_b_out [D],
        d_pos_bias [R, P], d_time_bias [R, Tb]
    (with return_sq also d_pos_bias_sq, d_time_bias_sq: attn_bwd's per-bin sums of squares).
    bf16_attention: the attention's operands q, k, v (forward and backward) and do (backward) are
    rounded to bf16 first, the precision in which a bf16 layer stores them; every other step stays
    float64.
    attn_operands: a function (name, array) -> array applied to the same four operands, named
    "q", "k", "v" and "do" (e.g. a perturbation of each element); bf16_attention is the case of
    round_bf16.  The same q, k, v serve the attention's forward and backward.
    The chain, from the output back (r = x + g W2^T + b2 is the pre-LayerNorm sum, g = LN(o) * U):
        dr = layer_norm_bwd(r, dy) if ln_output else dy
        d_b_out = sum_t dr;  d_w_out = dr^T g;  dg = dr W2
        dU = dg * LN(o);  do = layer_norm_bwd(o, dg * U)       (o = concat_h O, per token)
        dQ, dK, dV, d_pos_bias, d_time_bias = attn_bwd(..., do)
        dz = [dU | dV | dQ | dK] * SiLU'(z)                     (z = x W1^T + b1, before the SiLU)
        d_b_uvqk = sum_t dz;  d_w_uvqk = dz^T x;  dx = dr + dz W1
    """
    x = np.asarray(x, np.float64)
    w1 = np.asarray(w_uvqk, np.float64)
    w2 = np.asarray(w_out, np.float64)
    T = x.shape[0]
    hd = num_heads * head_dim
    z = x @ w1.T
    if b_uvqk is not None:
        z = z + np.asarray(b_uvqk, np.float64)
    s = silu(z)
    u, v, q, k = (s[:, c * hd:(c + 1) * hd].reshape(T, num_heads, head_dim) for c in range(4))
    if bf16_attention:
        if attn_operands is not None:
            raise ValueError("give bf16_attention or attn_operands, not both")
        attn_operands = lambda name, a: round_bf16(a)
    if attn_operands is not None:
        q, k, v = attn_operands("q", q), attn_operands("k", k), attn_operands("v", v)
    o = attn_fwd(jag, q, k, v, pos_bias, time_bias).reshape(T, hd)
    on = layer_norm(o, ln_eps)
    uf = u.reshape(T, hd)
    g = on * uf
    dy = np.asarray(dy, np.float64)
    if ln_output:
        r = x + g @ w2.T
        if b_out is not None:
            r = r + np.asarray(b_out, np.float64)
        dr = layer_norm_bwd(r, ln_eps, dy)
    else:
        dr = dy
    d_w_out = dr.T @ g
    d_b_out = dr.sum(axis=0)
    dg = dr @ w2
    du = dg * on
    do = layer_norm_bwd(o, ln_eps, dg * uf)
    if attn_operands is not None:
        do = attn_operands("do", do)
    res = attn_bwd(jag, q, k, v, pos_bias, time_bias, do.reshape(T, num_heads, head_dim), return_sq=return_sq)
    dq, dk, dv, dwp, dwt = res[:5]
    ds = np.concatenate([du, dv.reshape(T, hd), dq.reshape(T, hd), dk.reshape(T, hd)], axis=1)
    dz = ds * silu_grad(z)
    out = dict(dx=dr + dz @ w1, d_w_uvqk=dz.T @ x, d_b_uvqk=dz.sum(axis=0), d_w_out=d_w_out,
               d_b_out=d_b_out, d_pos_bias=dwp, d_time_bias=dwt)
    if return_sq:
        out.update(d_pos_bias_sq=res[5], d_time_bias_sq=res[6])
    return out


def stack_fwd(x, jag, layers, num_heads, head_dim):
    """A stack of layers; every layer but the last ends with the post-layer LayerNorm.
    layers: list of dicts with w_uvqk, b_uvqk, w_out, b_out, pos_bias, time_bias, ln_eps."""
    y = np.asarray(x, np.float64)
    for li, L in enumerate(layers):
        y = layer_fwd(y, jag, L["w_uvqk"], L.get("b_uvqk"), L["w_out"], L.get("b_out"), L["pos_bias"],
                      L["time_bias"], num_heads, head_dim, L["ln_eps"], ln_output=li < len(layers) - 1)
    return y


def gather_rows(table, ids):
    """X0[t] = E[id_t] (embedding lookup, [DLRMv4] Model architecture)."""
    return np.asarray(table)[np.asarray(ids, np.int64)]


# --------------------------------------------------------------------------- softmax attention (comparison)
def softmax_attn_fwd(jag: dict, q, k, v, row_sample=None):
    """Causal softmax attention over the same jagged batch, the comparison point of [HSTU] abstract
    (HSTU against FlashAttention2-based Transformers at sequence length 8192; the pages give no more
    about those models, so this is the textbook scaled dot-product attention):
        O_i = sum_{j <= i} softmax_j(q_i . k_j / sqrt(Dh)) v_j   per sequence and head, float64,
    written with the row maximum subtracted before the exponential.  Only the causal mask; no bias.
    q, k, v: [T, H, Dh]; returns [T, H, Dh], or with row_sample (dict b -> local rows) a dict
    (b, h) -> [rows, Dh]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    offs = np.asarray(jag["seq_offsets"], np.int64)
    T, H, Dh = q.shape
    scale = 1.0 / np.sqrt(Dh)
    out = {} if row_sample is not None else np.zeros((T, H, Dh), dtype=np.float64)
    for b in range(len(offs) - 1):
        o0, o1 = int(offs[b]), int(offs[b + 1])
        n = o1 - o0
        if n == 0 or (row_sample is not None and b not in row_sample):
            continue
        rows_all = np.arange(n) if row_sample is None else np.asarray(row_sample[b], np.int64)
        for h in range(H):
            res = np.zeros((len(rows_all), Dh), dtype=np.float64)
            for s in range(0, len(rows_all), _ROW_BLOCK):
                r = rows_all[s:s + _ROW_BLOCK]
                scores = (q[o0 + r, h] @ k[o0:o1, h].T) * scale
                scores = np.where(np.arange(n)[None, :] <= r[:, None], scores, -np.inf)
                w = np.exp(scores - scores.max(axis=1, keepdims=True))
                w = w / w.sum(axis=1, keepdims=True)
                res[s:s + _ROW_BLOCK] = w @ v[o0:o1, h]
            if row_sample is None:
                out[o0:o1, h] = res
            else:
                out[(b, h)] = res
    return out
