"""Outputs and workspaces are written before they are read: each entry point run into a workspace and
outputs filled with NaN bit patterns (0xFF bytes) gives bitwise the result of a run into zero-filled
ones.  A kernel that read a stale or unwritten word (a timestamp range, a statistic, a partial sum, a
tile row past a sequence's end) would carry the NaN into its output or differ from the clean run."""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import _lib as ops
from hstu_sequential_transduction_attn_amd import inputs as I

from _util import dev, jag_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _filled(like_or_shape, dtype, poison):
    t = torch.empty(like_or_shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xFF if poison else 0)
    return t


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _same(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert not torch.isnan(x.float()).any(), "NaN reached an output"
        assert torch.equal(_bits(x), _bits(y))


LENGTHS = [300, 1, 0, 129, 64, 33, 700]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attn_fwd_poisoned(dtype):
    print(f"\n[case] poisoned attn_fwd {dtype}", flush=True)
    case = I.attn_case("poison_a", 3201, LENGTHS, H=2, Dh=128, P=64, Tb=64, dtype=dtype)
    jd = jag_dev(case.jagged)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    wp, wt = dev(case.rab.pos_bias), dev(case.rab.time_bias)
    res = []
    for poison in (False, True):
        ws = _filled(1 << 16, torch.uint8, poison)
        out = _filled(q.shape, q.dtype, poison)
        ops.attn_fwd(jd["seq_offsets"], jd["timestamps"], q, k, v, wp, wt, max_seq_len=jd["max_seq_len"], out=out,
                     workspace=ws)
        torch.cuda.synchronize()
        res.append([out])
    _same(*res)


def test_attn_bwd_poisoned():
    print("\n[case] poisoned attn_bwd", flush=True)
    case = I.attn_case("poison_b", 3202, LENGTHS, H=2, Dh=128, P=64, Tb=64, dtype="bf16", num_candidates=None)
    jd = jag_dev(case.jagged)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    rng = np.random.default_rng(3203)
    g = dev(I.Tensor.make(rng.standard_normal(case.q.values.shape).astype(np.float32), "bf16"))
    wp, wt = dev(case.rab.pos_bias), dev(case.rab.time_bias)
    res = []
    for poison in (False, True):
        outs = [_filled(q.shape, torch.float32, poison) for _ in range(3)]
        outs += [_filled(wp.shape, torch.float32, poison), _filled(wt.shape, torch.float32, poison)]
        ws = _filled(1 << 22, torch.uint8, poison)
        ops.attn_bwd(jd["seq_offsets"], jd["timestamps"], q, k, v, g, wp, wt, max_seq_len=jd["max_seq_len"],
                     workspace=ws, outs=outs)
        torch.cuda.synchronize()
        res.append(outs)
    _same(*res)


@pytest.mark.parametrize("dtype,ln_output", [("bf16", True), ("f32", False)])
def test_layer_fwd_poisoned(dtype, ln_output):
    print(f"\n[case] poisoned layer_fwd {dtype} ln_output={ln_output}", flush=True)
    case = I.jagged_layer_case("poison_l", 3204, LENGTHS, D=128, H=2, Dh=64, P=64, Tb=64, dtype=dtype,
                               num_layers=1, bias_std=0.2)
    L = case.layers[0]
    jd = jag_dev(case.jagged)
    x = dev(case.x)
    args = (jd["seq_offsets"], jd["timestamps"], dev(L.w_uvqk), dev(L.w_out), dev(L.rab.pos_bias),
            dev(L.rab.time_bias), case.num_heads, case.head_dim)
    n = ops.layer_workspace_bytes(x, *args, max_seq_len=jd["max_seq_len"], ln_output=ln_output)
    res = []
    for poison in (False, True):
        ws = _filled(n, torch.uint8, poison)
        y = _filled(x.shape, x.dtype, poison)
        ops.layer_fwd(x, *args, max_seq_len=jd["max_seq_len"], b_uvqk=dev(L.b_uvqk), b_out=dev(L.b_out),
                      ln_eps=L.ln_eps, ln_output=ln_output, workspace=ws, y=y)
        torch.cuda.synchronize()
        res.append([y])
    _same(*res)


@pytest.mark.parametrize("fused", [False, True])
def test_stack_fwd_poisoned(fused):
    """Small stacks take the unfused path (gather, then one layer call at a time); a batch of ~27,000
    tokens at D = 256 takes the fused one (gather and LayerNorm inside the GEMMs)."""
    print(f"\n[case] poisoned stack_fwd fused={fused}", flush=True)
    rng = np.random.default_rng(3205)
    lengths = [1, 0] + [int(v) for v in rng.integers(200, 700, size=60)] if fused else LENGTHS
    # the fused path needs >= 256 row tiles of 64 for the output GEMM (D = 256: one column tile)
    assert (sum(lengths) >= 256 * 64) == fused
    case = I.jagged_layer_case("poison_s", 3205, lengths, D=256, H=2, Dh=128, P=64, Tb=64, dtype="bf16",
                               num_layers=3, bias_std=0.1)
    table = I.Tensor.make(rng.standard_normal((4000, 256)).astype(np.float32), "bf16")
    ids = I.bounded_zipf(rng, 1.1, 4000, case.jagged.total_tokens).astype(np.int64)
    jd = jag_dev(case.jagged)
    layers = [dict(w_uvqk=dev(L.w_uvqk), w_out=dev(L.w_out), pos_bias=dev(L.rab.pos_bias),
                   time_bias=dev(L.rab.time_bias), b_uvqk=dev(L.b_uvqk), b_out=dev(L.b_out), ln_eps=L.ln_eps)
              for L in case.layers]
    tab, idd = dev(table), dev(ids)
    n = ops.stack_workspace_bytes(tab, jd["seq_offsets"], jd["timestamps"], layers, case.num_heads, case.head_dim,
                                  max_seq_len=jd["max_seq_len"])
    res = []
    for poison in (False, True):
        ws = _filled(n, torch.uint8, poison)
        y = _filled((case.jagged.total_tokens, 256), torch.float32, poison)
        ops.stack_fwd(tab, idd, jd["seq_offsets"], jd["timestamps"], layers, case.num_heads, case.head_dim,
                      max_seq_len=jd["max_seq_len"], act_split=True, y_dtype=torch.float32, workspace=ws, y=y)
        torch.cuda.synchronize()
        res.append([y])
    _same(*res)
