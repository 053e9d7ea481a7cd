"""GPU parity of hstu_stack_fwd (a layer stack over embedding-table rows) against the float64 oracle.

The oracle is the composition of its own pinned pieces: gather_rows, then stack_fwd (post-layer
LayerNorm between layers).  Cases: a small stack that takes the unfused path (gather, then one layer
call at a time), ragged batches large enough for the fused path (gather inside layer 0's GEMMs,
LayerNorm applied inside the next layer's GEMMs), identity rows (no ids), split activations, the
candidate mask, and the 8-layer and candidate workloads at full size (shortest and longest sequences).
"""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import configs as C
from hstu_sequential_transduction_attn_amd import inputs as I
from oracle import hstu_oracle as O

from _util import (assert_close, dev, host, jag_dev, oracle_jag, oracle_layers, oracle_stack_sequence,
                   sub_jagged, workload_case, workload_sequences)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _table_case(name, seed, lengths, D, H, Dh, P, Tb, num_layers, table_rows, mask_candidates=None, bias_std=0.0):
    """A layer case whose input rows come from a seeded bf16 table through Zipf-distributed ids."""
    case = I.jagged_layer_case(name, seed, lengths, D=D, H=H, Dh=Dh, P=P, Tb=Tb, dtype="bf16",
                               num_layers=num_layers, bias_std=bias_std)
    rng = np.random.default_rng(seed + 7)
    table = I.Tensor.make(rng.standard_normal((table_rows, D)).astype(np.float32), "bf16")
    ids = I.bounded_zipf(rng, 1.1, table_rows, case.jagged.total_tokens)
    if mask_candidates is not None:
        case.jagged.mask = I.CAUSAL_CANDIDATES
        case.jagged.num_candidates = np.asarray(mask_candidates, np.int32)
    return case, table, ids


def _fused(T, D, HD):
    """The shapes the fused path takes (bf16): every GEMM fits the large-tile kernels (K a multiple of
    32; at least 256 tiles of 128 x 256 for the projection and of 64 x 256 for the gated output GEMM)."""
    tiles = lambda M, N, BM: -(-M // BM) * -(-N // 256)
    return D % 32 == 0 and HD % 32 == 0 and tiles(T, 4 * HD, 128) >= 256 and tiles(T, D, 64) >= 256


def _layers_dev(case):
    return [dict(w_uvqk=dev(L.w_uvqk), w_out=dev(L.w_out), pos_bias=dev(L.rab.pos_bias),
                 time_bias=dev(L.rab.time_bias), b_uvqk=None if L.b_uvqk is None else dev(L.b_uvqk),
                 b_out=None if L.b_out is None else dev(L.b_out), ln_eps=L.ln_eps) for L in case.layers]


def _gpu(case, table, ids, act_split=False, y_dtype=None):
    from hstu_sequential_transduction_attn_amd import _lib as ops
    jd = jag_dev(case.jagged)
    y = ops.stack_fwd(dev(table), None if ids is None else dev(ids.astype(np.int64)), jd["seq_offsets"],
                      jd["timestamps"], _layers_dev(case), case.num_heads, case.head_dim,
                      max_seq_len=jd["max_seq_len"], mask=jd["mask"], num_candidates=jd["num_candidates"],
                      act_split=act_split, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return host(y)


def _oracle(case, table, ids, seqs=None):
    x = O.gather_rows(table.values, ids) if ids is not None else table.values
    jag = case.jagged
    if seqs is not None:
        jag, idx = sub_jagged(jag, seqs)
        x = x[idx]
    return O.stack_fwd(x, oracle_jag(jag), oracle_layers(case), case.num_heads, case.head_dim)


def test_stack_small_unfused_path():
    """Too small for the large-tile GEMMs: gather, then layer by layer."""
    print("\n[case] stack small (unfused path)", flush=True)
    case, table, ids = _table_case("stk_s", 1400, [5, 1, 0, 70, 128, 33, 200], D=64, H=2, Dh=32, P=32, Tb=32,
                                   num_layers=3, table_rows=300, bias_std=0.2)
    assert not _fused(case.jagged.total_tokens, 64, 64)
    got = _gpu(case, table, ids, y_dtype=torch.float32)
    assert_close(got, _oracle(case, table, ids), "bf16", "stack small", magnitude_aware=True)


@pytest.mark.parametrize("act_split", [False, True])
def test_stack_fused_gather_ragged(act_split):
    """About 20k ragged tokens, D = 256, H*Dh = 256: the fused path (every GEMM large-tile)."""
    print(f"\n[case] stack fused gather act_split={act_split}", flush=True)
    rng = np.random.default_rng(1410)
    lengths = [int(v) for v in rng.integers(1, 1025, size=40)]
    case, table, ids = _table_case("stk_f", 1410, lengths, D=256, H=2, Dh=128, P=64, Tb=64, num_layers=3,
                                   table_rows=40_000, bias_std=0.1)
    print(f"  T={sum(lengths)}", flush=True)
    assert _fused(sum(lengths), 256, 256)
    got = _gpu(case, table, ids, act_split=act_split, y_dtype=torch.float32)
    assert_close(got, _oracle(case, table, ids), "bf16", "stack fused gather", magnitude_aware=True)


def test_stack_fused_identity_rows_bf16_out():
    """No ids (x_0 = the table's first T rows), bf16 output."""
    print("\n[case] stack fused identity rows", flush=True)
    rng = np.random.default_rng(1420)
    lengths = [int(v) for v in rng.integers(300, 1025, size=32)]
    case, table, _ = _table_case("stk_i", 1420, lengths, D=256, H=2, Dh=128, P=64, Tb=64, num_layers=2,
                                 table_rows=sum(lengths) + 5)
    print(f"  T={sum(lengths)}", flush=True)
    assert _fused(sum(lengths), 256, 256)
    got = _gpu(case, table, None)
    want = _oracle(case, I.Tensor.make(table.values[:sum(lengths)], "bf16"), None)
    assert_close(got, want, "bf16", "stack fused identity", magnitude_aware=True)


def test_stack_fused_candidates():
    print("\n[case] stack fused candidates", flush=True)
    rng = np.random.default_rng(1430)
    hist = [int(v) for v in rng.integers(600, 2000, size=14)]
    m = [int(v) for v in rng.integers(1, 300, size=14)]
    lengths = [h + c for h, c in zip(hist, m)]
    case, table, ids = _table_case("stk_c", 1430, lengths, D=256, H=2, Dh=128, P=64, Tb=64, num_layers=2,
                                   table_rows=20_000, mask_candidates=m)
    print(f"  T={sum(lengths)}", flush=True)
    assert _fused(sum(lengths), 256, 256)
    got = _gpu(case, table, ids, y_dtype=torch.float32)
    assert_close(got, _oracle(case, table, ids), "bf16", "stack fused candidates", magnitude_aware=True)


def _workload_table(case):
    """The workload's table restricted to the rows its ids touch (values as generated), with the ids
    renumbered into it, so that table[ids] equals the workload's x_0."""
    pos = np.searchsorted(case.table_touched, case.ids)
    return case.table_values, pos.astype(np.int64)


def _check_sequences(name, case, y, what):
    offs = case.jagged.seq_offsets
    for seq in workload_sequences(case):
        print(f"  {what}: sequence {seq} (n = {int(case.jagged.lengths[seq])})", flush=True)
        got = y[int(offs[seq]):int(offs[seq + 1])]
        r, m = assert_close(got, oracle_stack_sequence(name, case, seq), "bf16", f"{what} sequence {seq}")
        print(f"    rel_l2={r:.3e} max_abs={m:.3e}", flush=True)


def test_stack8_fused_full_size_shortest_and_longest_sequences():
    """The 8-layer stack workload (T = 145,051, D = 1024, H = 8 x 128) through hstu_stack_fwd with split
    activations and an fp32 output; the two shortest sequences and the longest vs the oracle."""
    print("\n[case] stack8_bf16 fused, full batch", flush=True)
    case = workload_case("stack8_bf16")
    table, ids = _workload_table(case)
    y = _gpu(case, table, ids, act_split=True, y_dtype=torch.float32)
    _check_sequences("stack8_bf16", case, y, "stack8 fused")


def test_mfalcon_fused_full_size_shortest_and_longest_users():
    """The candidate-masked 3-layer workload through hstu_stack_fwd; the two shortest users and the
    longest vs the oracle."""
    print("\n[case] mfalcon_bf16 fused, full batch", flush=True)
    case = workload_case("mfalcon_bf16")
    table, ids = _workload_table(case)
    y = _gpu(case, table, ids, y_dtype=torch.float32)
    _check_sequences("mfalcon_bf16", case, y, "mfalcon fused")


def test_stack_fused_partial_statistics_tile():
    """D = 352: each row's LayerNorm statistics merge a 256-column tile and a 96-column tile (unequal
    counts), and the gathered residual rows span both column tiles."""
    print("\n[case] stack fused D=352", flush=True)
    rng = np.random.default_rng(1440)
    lengths = [int(v) for v in rng.integers(1, 900, size=22)]
    case, table, ids = _table_case("stk_p", 1440, lengths, D=352, H=2, Dh=128, P=64, Tb=64, num_layers=3,
                                   table_rows=5_000, bias_std=0.1)
    print(f"  T={sum(lengths)}", flush=True)
    assert _fused(sum(lengths), 352, 256)
    got = _gpu(case, table, ids, act_split=True, y_dtype=torch.float32)
    assert_close(got, _oracle(case, table, ids), "bf16", "stack fused D=352", magnitude_aware=True)
