"""GPU parity of hstu_softmax_attn_fwd (the causal softmax attention the pointwise attention is compared
with) against the oracle's float64 softmax attention, through the C ABI."""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import configs as C
from hstu_sequential_transduction_attn_amd import inputs as I
from oracle import hstu_oracle as O

from _util import assert_close, dev, host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _gpu(case, out_dtype=None):
    from hstu_sequential_transduction_attn_amd import _lib as ops
    j = case.jagged
    return ops.softmax_attn_fwd(dev(j.seq_offsets.astype(np.int32)), dev(case.q), dev(case.k), dev(case.v),
                                max_seq_len=j.max_seq_len, out_dtype=out_dtype)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_softmax_ragged(out):
    print(f"\n[case] softmax ragged out={out}", flush=True)
    case = I.attn_case("smx", 3301, [1, 7, 0, 64, 65, 127, 128, 129, 300, 33, 1000], H=3, Dh=128, P=8, Tb=8,
                       dtype="bf16")
    got = host(_gpu(case, torch.bfloat16 if out == "bf16" else torch.float32))
    want = O.softmax_attn_fwd(dict(seq_offsets=case.jagged.seq_offsets), case.q.values, case.k.values,
                              case.v.values)
    r, m = assert_close(got, want, "bf16", f"softmax ragged {out}")
    print(f"  rel_l2={r:.3e} max_abs={m:.3e}")


def test_softmax_L8192_every_query_block():
    """The L=8192 shapes (8 x 8192, H = 4 x 128): first, last and one random row of every 128-row query
    block of every (sequence, head) against the oracle."""
    print("\n[case] softmax attn_L8192 every query block", flush=True)
    case = C.attn_L8192()
    got = host(_gpu(case))
    rng = np.random.default_rng(5)
    rows = {b: np.unique(np.concatenate([np.arange(0, 8192, 128), np.arange(127, 8192, 128),
                                         np.arange(0, 8192, 128) + rng.integers(1, 127, size=64)]))
            for b in range(8)}
    want = O.softmax_attn_fwd(dict(seq_offsets=case.jagged.seq_offsets), case.q.values, case.k.values,
                              case.v.values, row_sample=rows)
    offs = case.jagged.seq_offsets
    g = np.concatenate([got[offs[b] + rows[b], h] for b in range(8) for h in range(4)])
    w = np.concatenate([want[(b, h)] for b in range(8) for h in range(4)])
    r, m = assert_close(g, w, "bf16", "softmax L8192")
    print(f"  rel_l2={r:.3e} max_abs={m:.3e}")
