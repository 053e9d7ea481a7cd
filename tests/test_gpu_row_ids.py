"""Out-of-range row ids on the GPU: the gathers clamp each id into [0, table_rows) (the nearest row is
read, never memory past the table) and count the clamped reads in the device's id-error word, which
hstu_id_errors reads back.  Checked for hstu_gather_rows and for the fused stack, whose layer-0 GEMMs
gather their operand and residual rows themselves: the output equals, bit for bit, the output of the
same call with the ids clamped on the host, and the word is nonzero after it and zero after a call
whose ids are all in range."""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import inputs as I

from _util import dev, host, jag_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BAD = [-1, -(1 << 40), 10**12]


def _ids(rng, rows, T, n_bad):
    ids = rng.integers(0, rows, T).astype(np.int64)
    where = rng.choice(T, n_bad, replace=False)
    ids[where] = np.resize(np.array(BAD + [rows, rows + 1], np.int64), n_bad)
    return ids, np.clip(ids, 0, rows - 1)


def test_gather_clamps_and_counts_out_of_range_ids():
    from hstu_sequential_transduction_attn_amd import _lib as ops
    print("\n[case] gather with out-of-range ids", flush=True)
    rng = np.random.default_rng(1500)
    rows, D, T = 1000, 128, 3000
    table = torch.from_numpy(rng.standard_normal((rows, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    ids, clamped = _ids(rng, rows, T, 5)
    ops.id_errors(reset=True)
    want = ops.gather_rows(table, dev(clamped))
    assert ops.id_errors() == 0
    got = ops.gather_rows(table, dev(ids))
    n = ops.id_errors(reset=False)
    assert n >= 5, n
    assert ops.id_errors(reset=True) == n            # read without reset keeps the count
    assert ops.id_errors() == 0                       # reset cleared it
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_fused_stack_clamps_and_counts_out_of_range_ids():
    from hstu_sequential_transduction_attn_amd import _lib as ops
    print("\n[case] fused stack with out-of-range ids", flush=True)
    rng = np.random.default_rng(1510)
    lengths = [int(v) for v in rng.integers(1, 1025, size=40)]
    T, rows = sum(lengths), 30_000
    case = I.jagged_layer_case("stk_bad", 1510, lengths, D=256, H=2, Dh=128, P=64, Tb=64, dtype="bf16",
                               num_layers=2, bias_std=0.1)
    table = dev(I.Tensor.make(rng.standard_normal((rows, 256)).astype(np.float32), "bf16"))
    ids, clamped = _ids(rng, rows, T, 7)
    jd = jag_dev(case.jagged)
    layers = [dict(w_uvqk=dev(L.w_uvqk), w_out=dev(L.w_out), pos_bias=dev(L.rab.pos_bias),
                   time_bias=dev(L.rab.time_bias), b_uvqk=dev(L.b_uvqk), b_out=dev(L.b_out), ln_eps=L.ln_eps)
              for L in case.layers]

    def run(i):
        return ops.stack_fwd(table, dev(i), jd["seq_offsets"], jd["timestamps"], layers, 2, 128,
                             max_seq_len=jd["max_seq_len"], y_dtype=torch.float32)
    ops.id_errors(reset=True)
    want = run(clamped)
    assert ops.id_errors() == 0
    got = run(ids)
    assert ops.id_errors() > 0
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert np.all(np.isfinite(host(got)))
