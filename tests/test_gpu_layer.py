"""GPU parity of hstu_layer_fwd (and the gather followed by layer-by-layer stacks) against the float64 oracle."""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import configs as C
from hstu_sequential_transduction_attn_amd import inputs as I
from oracle import hstu_oracle as O

from _util import (assert_close, gpu_layer_stack, gather_input, host, dev, oracle_jag, oracle_layers,
                   oracle_stack_sequence, sub_jagged, workload_case, workload_sequences)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _oracle_stack(case, seqs=None):
    jag = case.jagged
    x = case.x.values
    if seqs is not None:
        jag, idx = sub_jagged(jag, seqs)
        x = x[idx]
    return O.stack_fwd(x, oracle_jag(jag), oracle_layers(case), case.num_heads, case.head_dim)


def test_tiny_layer_f32_full():
    print("\n[case] tiny_layer_f32 (config 1)", flush=True)
    case = C.tiny_layer_f32()
    got = host(gpu_layer_stack(case))
    r, m = assert_close(got, _oracle_stack(case), "f32", "tiny layer f32")
    print(f"  rel_l2={r:.3e} max_abs={m:.3e}")


def test_layer_bf16_full():
    print("\n[case] layer_bf16 (config 2)", flush=True)
    case = C.layer_bf16()
    got = host(gpu_layer_stack(case))
    r, m = assert_close(got, _oracle_stack(case), "bf16", "layer bf16")
    print(f"  rel_l2={r:.3e} max_abs={m:.3e}")


@pytest.mark.parametrize("dtype,ln_output", [("f32", True), ("bf16", True), ("bf16", False)])
def test_layer_biases_ragged(dtype, ln_output):
    """Nonzero biases, post-layer LayerNorm, odd sizes (D = 72, H = 3, ragged lengths incl. empty)."""
    print(f"\n[case] layer with biases {dtype} ln_output={ln_output}", flush=True)
    case = I.jagged_layer_case("bias", 960, [1, 0, 129, 64, 200, 31], D=72, H=3, Dh=64, P=50, Tb=30, dtype=dtype,
                               num_layers=2 if ln_output else 1, bias_std=0.3)
    got = host(gpu_layer_stack(case))
    assert_close(got, _oracle_stack(case), dtype, "layer with biases", magnitude_aware=True)


@pytest.mark.parametrize("act_split", [False, True])
def test_layer_f32_residual_stream(act_split):
    """bf16 weights with an fp32 residual stream (x, y fp32), with and without split activations."""
    print(f"\n[case] fp32 residual stream act_split={act_split}", flush=True)
    case = I.jagged_layer_case("res32", 965, [70, 1, 300, 129], D=256, H=2, Dh=128, P=64, Tb=64, dtype="bf16",
                               num_layers=3, bias_std=0.2)
    got = host(gpu_layer_stack(case, residual_f32=True, act_split=act_split))
    assert_close(got, _oracle_stack(case), "bf16", "fp32 residual stream", magnitude_aware=True)


@pytest.mark.parametrize("residual_f32,act_split", [(False, False), (True, False), (True, True)])
def test_layer_large_tiles_ragged_tails(residual_f32, act_split):
    """Enough rows for the large-tile GEMMs, with ragged row and column tails: T not a multiple of any
    row tile, D = 352 (output-projection columns 256 + 96), H*Dh = 320 (U|V|Q|K boundaries inside
    column tiles)."""
    print(f"\n[case] large-tile GEMM tails residual_f32={residual_f32} act_split={act_split}", flush=True)
    rng = np.random.default_rng(971)
    lengths = [int(v) for v in rng.integers(1, 251, size=72)]
    case = I.jagged_layer_case("tails", 971, lengths, D=352, H=5, Dh=64, P=64, Tb=64, dtype="bf16",
                               num_layers=2, bias_std=0.2)
    print(f"  T={sum(lengths)}", flush=True)
    got = host(gpu_layer_stack(case, residual_f32=residual_f32, act_split=act_split))
    assert_close(got, _oracle_stack(case), "bf16", "large-tile GEMM tails", magnitude_aware=True)


def test_layer_candidates_small():
    print("\n[case] layer candidates small", flush=True)
    case = I.jagged_layer_case("candl", 970, [150, 40, 300], D=128, H=2, Dh=128, P=64, Tb=64, dtype="bf16",
                               num_layers=2)
    case.jagged.mask = I.CAUSAL_CANDIDATES
    case.jagged.num_candidates = np.array([50, 1, 100], np.int32)
    got = host(gpu_layer_stack(case))
    assert_close(got, _oracle_stack(case), "bf16", "candidates layer", magnitude_aware=True)


def test_gather_rows_exact():
    print("\n[case] gather rows", flush=True)
    from hstu_sequential_transduction_attn_amd import _lib as ops
    rng = np.random.default_rng(5)
    table = I.Tensor.make(rng.standard_normal((1000, 64)).astype(np.float32), "bf16")
    ids = rng.integers(0, 1000, size=777).astype(np.int64)
    out = ops.gather_rows(dev(table), dev(ids))
    assert np.array_equal(host(out), O.gather_rows(table.values, ids))


def _check_sequences(name, case, y, what):
    offs = case.jagged.seq_offsets
    for seq in workload_sequences(case):
        print(f"  {what}: sequence {seq} (n = {int(case.jagged.lengths[seq])})", flush=True)
        got = y[int(offs[seq]):int(offs[seq + 1])]
        r, m = assert_close(got, oracle_stack_sequence(name, case, seq), "bf16", f"{what} sequence {seq}")
        print(f"    rel_l2={r:.3e} max_abs={m:.3e}", flush=True)


def test_stack8_full_size_shortest_and_longest_sequences():
    """The 8-layer stack workload at full size (T = 145,051), one hstu_layer_fwd call per layer after the
    gather; the two shortest sequences and the longest (4016 tokens through 8 layers) vs the oracle."""
    print("\n[case] stack8_bf16 (config 4), full batch, layer by layer", flush=True)
    case = workload_case("stack8_bf16")
    y = host(gpu_layer_stack(case, use_gather=True, residual_f32=True, act_split=True))
    _check_sequences("stack8_bf16", case, y, "stack8 layer path")


def test_mfalcon_full_size_shortest_and_longest_users():
    """The candidate-masked 3-layer workload at full size; the two shortest users and the longest (its
    history and 1024 candidates) vs the oracle."""
    print("\n[case] mfalcon_bf16 (config 5), full batch, layer by layer", flush=True)
    case = workload_case("mfalcon_bf16")
    y = host(gpu_layer_stack(case, use_gather=True, residual_f32=True))
    _check_sequences("mfalcon_bf16", case, y, "mfalcon layer path")
