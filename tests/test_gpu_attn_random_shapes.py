"""Seeded random shapes for the attention forward and backward against the float64 oracle.

Each case draws the batch (including empty sequences and one longer sequence), heads, head_dim, bias
table sizes (P from 1, Tb from 1), shared or per-head tables, bf16 or fp32, the candidate mask and
explicit c_b, so that combinations the hand-written cases do not name are exercised too.
"""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import inputs as I
from oracle import hstu_oracle as O

from _util import dev, host, jag_dev, max_abs, oracle_jag, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.integers(0, 600, B)]
    if rng.random() < 0.3:
        lengths[0] = int(rng.integers(600, 1500))
    H = int(rng.integers(1, 4))
    Dh = int(rng.choice([32, 64, 128]))
    P, Tb = int(rng.integers(1, 300)), int(rng.integers(1, 70))
    R = 1 if rng.random() < 0.5 else H
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    cands = [int(rng.integers(0, n + 1)) for n in lengths] if rng.random() < 0.4 else None
    case = I.attn_case("rnd", seed, lengths, H=H, Dh=Dh, P=P, Tb=Tb, dtype=dtype, num_candidates=cands,
                       rab_rows=R, with_u=False)
    if rng.random() < 0.3:
        case.jagged.attn_scale = rng.normal(0, 0.5, B).astype(np.float32)
    g = I.Tensor.make(rng.standard_normal(case.q.shape).astype(np.float32), dtype)
    return case, g, f"B={B} lengths={lengths} H={H} Dh={Dh} P={P} Tb={Tb} R={R} {dtype} cands={cands}"


@pytest.mark.parametrize("seed", [9003, 9011, 9024, 9037, 9042, 9058, 9066, 9071])
def test_random_shapes_forward_and_backward(seed):
    from hstu_sequential_transduction_attn_amd import _lib as ops
    case, g, what = _case(seed)
    print(f"\n[case] seed={seed} {what}", flush=True)
    jd = jag_dev(case.jagged)
    common = dict(max_seq_len=jd["max_seq_len"], mask=jd["mask"], num_candidates=jd["num_candidates"],
                  attn_scale=jd["attn_scale"])
    got_b = [host(x) for x in ops.attn_bwd(jd["seq_offsets"], jd["timestamps"], dev(case.q), dev(case.k),
                                           dev(case.v), dev(g), dev(case.rab.pos_bias), dev(case.rab.time_bias),
                                           **common)]
    got_f = host(ops.attn_fwd(jd["seq_offsets"], jd["timestamps"], dev(case.q), dev(case.k), dev(case.v),
                              dev(case.rab.pos_bias), dev(case.rab.time_bias), out_dtype=torch.float32, **common))
    torch.cuda.synchronize()
    oj = oracle_jag(case.jagged)
    want = O.attn_bwd(oj, case.q.values, case.k.values, case.v.values, case.rab.pos_bias, case.rab.time_bias,
                      g.values, return_sq=True)
    want_f = O.attn_fwd(oj, case.q.values, case.k.values, case.v.values, case.rab.pos_bias, case.rab.time_bias)
    bf = case.dtype == "bf16"
    for x, y, name in zip(got_b + [got_f], list(want[:5]) + [want_f], ["dq", "dk", "dv", "dwp", "dwt", "O"]):
        if y.size == 0:
            continue
        r, m = rel_l2(x, y), max_abs(x, y)
        ymax = float(np.abs(y).max())
        if name in ("dwp", "dwt"):
            # each bin sums many dS terms with their own roundings: its error scale is sqrt(sum dS^2)
            sq = want[5] if name == "dwp" else want[6]
            unit = 2.0 ** -7 if bf else 1e-5
            tol = 4 * unit * np.sqrt(sq) + unit * np.abs(y) + 1e-6
            assert np.all(np.abs(x - y) <= tol), f"{name}: rel_l2={r:.3e} max_abs={m:.3e}"
        elif bf:
            assert r <= 5e-3 and m <= 2e-2 + 2.0 ** -7 * ymax, f"{name}: rel_l2={r:.3e} max_abs={m:.3e}"
        else:
            assert r <= 1e-5, f"{name}: rel_l2={r:.3e} max_abs={m:.3e}"
