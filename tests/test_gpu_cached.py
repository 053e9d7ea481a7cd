"""GPU parity of hstu_attn_fwd_cached (candidates against a cached history) through the C ABI.

Against the float64 oracle element by element, and against the one-pass candidate-masked kernel:
candidate micro-batches scored with the one-pass c_b must reassemble its candidate rows.
"""
import dataclasses

import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import inputs as I
from oracle import hstu_oracle as O

from _util import assert_close, dev, gpu_attn, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

HIST = [300, 40, 0, 1, 64, 200, 700, 129]
CAND = [44, 40, 5, 1, 63, 130, 0, 33]


def _case(seed, hist, cand, H=3, Dh=128, P=64, Tb=32, dtype="bf16", R=1):
    full = I.attn_case("cached", seed, [h + c for h, c in zip(hist, cand)], H=H, Dh=Dh, P=P, Tb=Tb, dtype=dtype,
                       num_candidates=cand, rab_rows=R, with_u=False)
    return full, I.split_candidates(full)


def _subset(cc, picks):
    """Candidates picks[b] (user-local indices) of every user, as a CachedCase of its own."""
    co = cc.cand_offsets.astype(np.int64)
    idx = np.concatenate([co[b] + np.asarray(p, np.int64) for b, p in enumerate(picks)])
    take = lambda t: I.Tensor(values=t.values[idx], dtype=t.dtype, bits=None if t.bits is None else t.bits[idx])
    return dataclasses.replace(cc, cand_offsets=I.offsets_of([len(p) for p in picks]),
                               cand_timestamps=cc.cand_timestamps[idx], q=take(cc.q), k=take(cc.k), v=take(cc.v),
                               cand_rows=cc.cand_rows[idx]), idx


def _oracle(cc, attn_scale=None):
    hist = dict(seq_offsets=cc.hist_offsets.astype(np.int64), timestamps=cc.hist_timestamps)
    cand = dict(seq_offsets=cc.cand_offsets.astype(np.int64), timestamps=cc.cand_timestamps)
    return O.attn_cached(hist, cand, cc.k_hist.values, cc.v_hist.values, cc.q.values, cc.k.values, cc.v.values,
                         cc.rab.pos_bias, cc.rab.time_bias, attn_scale)


def _gpu(cc, attn_scale=None, out_dtype=None, max_history=None):
    from hstu_sequential_transduction_attn_amd import _lib as ops
    if max_history is None:
        d = np.diff(cc.hist_offsets.astype(np.int64))
        max_history = int(d.max()) if len(d) else 0
    return ops.attn_fwd_cached(dev(cc.hist_offsets.astype(np.int32)), dev(cc.hist_timestamps.astype(np.int64)),
                               dev(cc.k_hist), dev(cc.v_hist), dev(cc.cand_offsets.astype(np.int32)),
                               dev(cc.cand_timestamps.astype(np.int64)), dev(cc.q), dev(cc.k), dev(cc.v),
                               dev(cc.rab.pos_bias), dev(cc.rab.time_bias), max_candidates=cc.max_candidates,
                               max_history=max_history,
                               attn_scale=None if attn_scale is None else dev(np.asarray(attn_scale, np.float32)),
                               out_dtype=out_dtype)


@pytest.mark.parametrize("Dh,out,R", [(32, "bf16", 1), (64, "f32", 3), (128, "bf16", 1), (128, "f32", 3)])
def test_bf16_cached_matches_oracle(Dh, out, R):
    print(f"\n[case] cached bf16 Dh={Dh} out={out} R={R}", flush=True)
    _, cc = _case(1000 + Dh + R, HIST, CAND, Dh=Dh, R=R)
    got = host(_gpu(cc, out_dtype=torch.bfloat16 if out == "bf16" else torch.float32))
    assert_close(got, _oracle(cc), "bf16", f"cached Dh={Dh}", magnitude_aware=True)


@pytest.mark.parametrize("Dh", [32, 128])
def test_f32_cached_matches_oracle(Dh):
    print(f"\n[case] cached f32 Dh={Dh}", flush=True)
    _, cc = _case(1010 + Dh, HIST, CAND, H=2, Dh=Dh, P=16, Tb=40, dtype="f32")
    assert_close(host(_gpu(cc)), _oracle(cc), "f32", f"cached f32 Dh={Dh}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_micro_batches_reassemble_the_one_pass_candidate_rows(dtype):
    print(f"\n[case] cached micro-batches vs one-pass {dtype}", flush=True)
    full, cc = _case(1020, HIST, CAND, H=2, Dh=64, P=48, Tb=32, dtype=dtype)
    scale = (1.0 / cc.one_pass_lengths).astype(np.float32)
    rng = np.random.default_rng(1020)
    parts = [[], [], []]
    for m in CAND:   # three micro-batches: random cut points of each user's candidates
        cuts = np.sort(rng.integers(0, m + 1, size=2))
        edges = [0, int(cuts[0]), int(cuts[1]), m]
        for t in range(3):
            parts[t].append(np.arange(edges[t], edges[t + 1]))
    got = np.zeros(cc.q.shape, np.float64)
    for t in range(3):
        sub, idx = _subset(cc, parts[t])
        got[idx] = host(_gpu(sub, attn_scale=scale, out_dtype=torch.float32))
    want_oracle = _oracle(cc)   # default c_b = 1 / (n_h + m_b) with every candidate present
    one_pass = host(gpu_attn(full, out_dtype=torch.float32))[cc.cand_rows]
    assert_close(got, want_oracle, dtype, "micro-batches vs oracle", magnitude_aware=True)
    assert_close(got, one_pass, dtype, "micro-batches vs one-pass kernel", magnitude_aware=True)


def test_giant_gaps_and_large_tables():
    print("\n[case] cached P=Tb=4096, giant timestamps", flush=True)
    full, _ = _case(1030, [257, 100, 0], [20, 9, 4], H=2, Dh=64, P=4096, Tb=4096, dtype="f32")
    rng = np.random.default_rng(1030)
    t = full.jagged.timestamps.copy()
    t[5] = t[4]
    t[100:140] = rng.integers(-(1 << 62), 1 << 62, size=40)
    t[260] = np.iinfo(np.int64).min
    t[380] = np.iinfo(np.int64).max
    full.jagged.timestamps = t
    full.rab.pos_bias[:] = rng.normal(0, 0.5, full.rab.pos_bias.shape)
    full.rab.time_bias[:] = rng.normal(0, 0.5, full.rab.time_bias.shape)
    cc = I.split_candidates(full)
    assert_close(host(_gpu(cc)), _oracle(cc), "f32", "cached giant gaps")


def test_no_candidates_and_no_history():
    print("\n[case] cached: users without candidates, users without history", flush=True)
    _, cc = _case(1040, [0, 50, 0], [3, 0, 1], H=1, Dh=32)
    assert_close(host(_gpu(cc, out_dtype=torch.float32)), _oracle(cc), "bf16", "empty parts", magnitude_aware=True)
    _, cc0 = _case(1041, [10, 20], [0, 0], H=1, Dh=32)
    assert _gpu(cc0).shape[0] == 0


def test_mfalcon_size_micro_batch_sampled_users():
    """16 users with histories U{1024..8192} and 1024 candidates; one micro-batch of 256 candidates per
    user scored against the full history, checked on three users."""
    print("\n[case] cached mfalcon size, 256-candidate micro-batch", flush=True)
    rng = I.rng_for(5, 7)
    hist = [int(x) for x in rng.integers(1024, 8193, size=16)]
    full, cc = _case(1050, hist, [1024] * 16, H=4, Dh=128, P=128, Tb=128)
    sub, _ = _subset(cc, [np.arange(256 * (b % 4), 256 * (b % 4 + 1)) for b in range(16)])
    scale = (1.0 / sub.one_pass_lengths).astype(np.float32)
    got = host(_gpu(sub, attn_scale=scale))
    users = [0, 7, int(np.argmax(hist))]
    so = sub.cand_offsets.astype(np.int64)
    for b in users:
        one, idx = _subset(sub, [np.arange(so[u + 1] - so[u]) if u == b else np.zeros(0, np.int64)
                                 for u in range(16)])
        rows = np.arange(so[b], so[b + 1])
        want = _oracle(one, attn_scale=scale)
        assert_close(got[rows], want, "bf16", f"user {b}")


@pytest.mark.parametrize("max_history", [None, 0, 1500, 100000])
def test_history_split_over_workgroups(max_history):
    """Few candidates and long histories: the history is split over several workgroups whose partial
    sums are reduced in order.  max_history only sets the split; any value gives the same result
    (an underestimate leaves the rest to the last split; 100000 > T_h is clamped to T_h by the caller)."""
    print(f"\n[case] cached key splits max_history={max_history}", flush=True)
    _, cc = _case(1060, [4000, 2500, 37, 0, 3100], [3, 70, 5, 2, 129], H=2, Dh=128, P=200, Tb=40)
    T_h = int(cc.hist_offsets[-1])
    mh = None if max_history is None else min(max_history, T_h)
    got = host(_gpu(cc, out_dtype=torch.float32, max_history=mh))
    assert_close(got, _oracle(cc), "bf16", f"key splits {max_history}", magnitude_aware=True)
    again = host(_gpu(cc, out_dtype=torch.float32, max_history=mh))
    assert np.array_equal(got, again), "not deterministic"
