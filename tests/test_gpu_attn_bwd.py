"""GPU parity of hstu_attn_bwd (the attention backward) against the float64 oracle gradients.

The oracle's gradients are pinned to finite differences of the forward oracle (test_oracle_backward).
Cases: ragged batches with empty and one-token sequences, every head_dim, bf16 and fp32, shared and
per-head bias tables, the candidate mask, tiles of every class, and bitwise determinism.
"""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import inputs as I
from oracle import hstu_oracle as O

from _util import assert_close, dev, host, jag_dev, max_abs, oracle_jag, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

RAGGED = [1, 7, 0, 64, 65, 127, 128, 129, 300, 33]


def _grad_out(case, seed):
    rng = np.random.default_rng(seed)
    return I.Tensor.make(rng.standard_normal(case.q.shape).astype(np.float32), case.dtype)


def _gpu(case, g):
    from hstu_sequential_transduction_attn_amd import _lib as ops
    jd = jag_dev(case.jagged)
    return [host(x) for x in ops.attn_bwd(jd["seq_offsets"], jd["timestamps"], dev(case.q), dev(case.k), dev(case.v),
                                          dev(g), dev(case.rab.pos_bias), dev(case.rab.time_bias),
                                          max_seq_len=jd["max_seq_len"], mask=jd["mask"],
                                          num_candidates=jd["num_candidates"], attn_scale=jd["attn_scale"])]


def _oracle(case, g):
    return O.attn_bwd(oracle_jag(case.jagged), case.q.values, case.k.values, case.v.values, case.rab.pos_bias,
                      case.rab.time_bias, g.values)


NAMES = ["dq", "dk", "dv", "d_pos_bias", "d_time_bias"]


def _check(got, want, dtype, what):
    """Gradients are sums of many terms with cancellation, so the bar is norm-wise: rel-L2 as for the
    forward (bf16 5e-3, fp32 1e-5) and, for bf16, max-abs within 2e-2 + 2^-7 max|want| (each term
    carries the bf16 rounding of dS or SiLU(s), 2^-9 relative)."""
    for x, y, name in zip(got, want, NAMES):
        assert np.all(np.isfinite(x)), f"{what} {name}: non-finite"
        r, m = rel_l2(x, y), max_abs(x, y)
        if dtype == "bf16":
            bound = 2e-2 + 2.0 ** -7 * float(np.abs(y).max() if y.size else 0.0)
            assert r <= 5e-3 and m <= bound, f"{what} {name}: rel_l2={r:.3e} max_abs={m:.3e} (bound {bound:.3e})"
        else:
            assert r <= 1e-5, f"{what} {name}: rel_l2={r:.3e} max_abs={m:.3e}"


@pytest.mark.parametrize("Dh,R", [(32, 1), (64, 3), (128, 1), (128, 3)])
def test_bf16_bwd_ragged_causal(Dh, R):
    print(f"\n[case] bwd bf16 ragged causal Dh={Dh} R={R}", flush=True)
    case = I.attn_case("bwd", 1100 + Dh + R, RAGGED, H=3, Dh=Dh, P=40, Tb=24, dtype="bf16", rab_rows=R, with_u=False)
    g = _grad_out(case, 1100 + Dh)
    _check(_gpu(case, g), _oracle(case, g), "bf16", f"Dh={Dh} R={R}")


@pytest.mark.parametrize("Dh", [32, 128])
def test_f32_bwd_ragged_causal(Dh):
    print(f"\n[case] bwd f32 ragged causal Dh={Dh}", flush=True)
    case = I.attn_case("bwd32", 1110 + Dh, RAGGED, H=2, Dh=Dh, P=32, Tb=32, dtype="f32", with_u=False)
    g = _grad_out(case, 1110 + Dh)
    _check(_gpu(case, g), _oracle(case, g), "f32", f"f32 Dh={Dh}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_candidates_and_scale(dtype):
    print(f"\n[case] bwd candidates {dtype}", flush=True)
    lengths = [300, 40, 129, 1, 64, 200]
    cands = [44, 40, 0, 1, 63, 130]
    case = I.attn_case("bwdc", 1120, lengths, H=2, Dh=64, P=64, Tb=32, dtype=dtype, num_candidates=cands,
                       rab_rows=2, with_u=False)
    case.jagged.attn_scale = np.array([0.5, -2.0, 1.0 / 7.0, 1.0, 0.01, 0.2], dtype=np.float32)
    g = _grad_out(case, 1120)
    _check(_gpu(case, g), _oracle(case, g), dtype, f"candidates {dtype}")


def test_bwd_long_sequences_uniform_tiles():
    """Sequences long enough that most tiles take the one-bias class, P = Tb = 256 as in the L = 8192
    workload."""
    print("\n[case] bwd 2 x 2048 + 777, P=Tb=256", flush=True)
    case = I.attn_case("bwdl", 1130, [2048, 777, 2048], H=2, Dh=128, P=256, Tb=256, dtype="bf16", with_u=False)
    g = _grad_out(case, 1130)
    _check(_gpu(case, g), _oracle(case, g), "bf16", "long")


@pytest.mark.parametrize("P,Tb", [(1, 1), (2, 3), (33, 1)])
def test_bwd_tiny_bias_tables(P, Tb):
    """Degenerate tables: with P = 1 every pair's position bucket is the clamped one, with P = 2 only the
    diagonal is unclamped, and Tb = 1 gives one time bucket.  Sequences long enough for near-diagonal
    tiles both with and without clamped pairs; also the candidate mask (its candidate waves sum the
    position buckets score by score)."""
    print(f"\n[case] bwd tiny tables P={P} Tb={Tb}", flush=True)
    case = I.attn_case("bwdt", 1150 + P + Tb, [700, 1, 130, 64], H=2, Dh=64, P=P, Tb=Tb, dtype="bf16",
                       with_u=False)
    g = _grad_out(case, 1150)
    _check(_gpu(case, g), _oracle(case, g), "bf16", f"P={P} Tb={Tb}")
    cc = I.attn_case("bwdtc", 1160 + P + Tb, [400, 90], H=2, Dh=64, P=P, Tb=Tb, dtype="bf16",
                     num_candidates=[70, 30], with_u=False)
    gc = _grad_out(cc, 1160)
    _check(_gpu(cc, gc), _oracle(cc, gc), "bf16", f"candidates P={P} Tb={Tb}")


def test_bwd_deterministic_and_bins_consistent():
    print("\n[case] bwd determinism", flush=True)
    case = I.attn_case("bwdd", 1140, [1500, 900, 3], H=2, Dh=64, P=300, Tb=40, dtype="bf16", with_u=False)
    g = _grad_out(case, 1140)
    a, b = _gpu(case, g), _gpu(case, g)
    for x, y, name in zip(a, b, NAMES):
        assert np.array_equal(x, y), f"{name} differs between runs"
    # every allowed pair lands in one position bin and one time bin
    np.testing.assert_allclose(a[3].sum(axis=1), a[4].sum(axis=1), rtol=1e-4, atol=1e-5)


def test_bwd_xcd_grouped_work_order():
    """A batch whose (sequence, head) pairs take the XCD-local work order with all three segments:
    256 sequences x 2 heads = 512 pairs (64 per XCD), at most 8 query blocks per pair, so each XCD runs
    its first 16 pairs together, the next 32 one at a time and its last 16 together (csrc/work_order.hpp).
    Both passes run in that order, and the dQ pass stores each workgroup's bias-gradient bins at its
    query-block-major row: every gradient, the bias tables' included, against the whole oracle, the
    forward as well, and two runs bitwise equal."""
    print("\n[case] bwd and fwd in the XCD-grouped work order (256 x 2 pairs)", flush=True)
    rng = np.random.default_rng(1180)
    lengths = [int(v) for v in rng.integers(1, 80, size=256)]
    for i in rng.choice(256, size=10, replace=False):
        lengths[int(i)] = int(rng.integers(900, 1025))
    lengths[int(rng.integers(0, 256))] = 1024            # the longest: 8 query blocks per pair
    case = I.attn_case("bwdx", 1180, lengths, H=2, Dh=32, P=64, Tb=32, dtype="bf16", with_u=False)
    g = _grad_out(case, 1181)
    got = _gpu(case, g)
    _check(got, _oracle(case, g), "bf16", "grouped order")
    again = _gpu(case, g)
    for x, y, name in zip(got, again, NAMES):
        assert np.array_equal(x, y), f"{name} differs between runs"
    from hstu_sequential_transduction_attn_amd import _lib as ops
    jd = jag_dev(case.jagged)
    o = host(ops.attn_fwd(jd["seq_offsets"], jd["timestamps"], dev(case.q), dev(case.k), dev(case.v),
                          dev(case.rab.pos_bias), dev(case.rab.time_bias), max_seq_len=jd["max_seq_len"]))
    want = O.attn_fwd(oracle_jag(case.jagged), case.q.values, case.k.values, case.v.values, case.rab.pos_bias,
                      case.rab.time_bias)
    # an ad-hoc batch: sequences of 1 to 80 tokens have c_b up to 1 and outputs up to about 20, so the
    # elementwise bar grows with the value (two bf16 roundings, 2^-7 |want|)
    assert_close(o, want, "bf16", "forward, grouped order", magnitude_aware=True)


def test_bwd_empty_batch_zeroes_the_bias_gradients():
    from hstu_sequential_transduction_attn_amd import _lib as ops
    print("\n[case] bwd empty batch", flush=True)
    offs = torch.zeros(3, dtype=torch.int32, device="cuda")
    tau = torch.zeros(0, dtype=torch.int64, device="cuda")
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    wp = torch.randn(1, 16, device="cuda")
    wt = torch.randn(1, 8, device="cuda")
    dq, dk, dv, d_pos, d_time = ops.attn_bwd(offs, tau, q, q, q, q, wp, wt, max_seq_len=0)
    assert dq.shape[0] == 0
    assert not torch.any(d_pos).item() and not torch.any(d_time).item()


def test_bwd_L8192_sampled_rows_against_oracle():
    """The attention backward at its benchmark shape (8 x 8192, H = 4 x 128, P = Tb = 256), launched as
    for the full batch: dq of sampled query rows and dk, dv of sampled key rows of two (sequence, head)
    pairs against the oracle's row- and column-restricted backward (tile edges, the first and last rows,
    and random rows)."""
    from hstu_sequential_transduction_attn_amd import configs as C
    print("\n[case] attn_L8192 backward, sampled rows", flush=True)
    case = C.attn_L8192()
    g = _grad_out(case, 1170)
    got = _gpu(case, g)
    rng = np.random.default_rng(1171)
    picks = [0, 1, 31, 32, 63, 64, 127, 128, 4095, 4096, 8190, 8191] + [int(x) for x in rng.integers(0, 8192, 4)]
    jag = oracle_jag(case.jagged)
    offs = case.jagged.seq_offsets
    for b, h in [(0, 0), (7, 3)]:
        want = O.attn_bwd_sampled(jag, case.q.values, case.k.values, case.v.values, case.rab.pos_bias,
                                  case.rab.time_bias, g.values, b, h, picks, picks)
        idx = int(offs[b]) + np.asarray(picks)
        for x, y, name in zip((got[0][idx, h], got[1][idx, h], got[2][idx, h]), want, NAMES):
            r, m = rel_l2(x, y), max_abs(x, y)
            print(f"  b={b} h={h} {name}: rel_l2={r:.3e} max_abs={m:.3e}")
            bound = 2e-2 + 2.0 ** -7 * float(np.abs(y).max())
            assert r <= 5e-3 and m <= bound, f"b={b} h={h} {name}: rel_l2={r:.3e} max_abs={m:.3e}"
