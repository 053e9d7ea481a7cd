"""Properties of the GPU path at the workloads' full sizes, where the float64 oracle cannot follow.

Every output of the attention forward is linear in V, and every gradient of the backward is linear in
the upstream gradient.  Multiplying that input by 2 multiplies every intermediate by 2, and rounding
to bf16 or fp32 commutes with a power-of-two scale (barring overflow and subnormals, which these
magnitudes never reach), so the outputs must be exactly twice the originals, bit for bit.  A kernel
that mixed up rows, dropped a tile, or read memory it does not own would break this equality or the
run-to-run determinism checked alongside it.
"""
import pytest

from hstu_sequential_transduction_attn_amd import configs as C

from _util import dev, jag_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _equal_times_two(a, b, name):
    assert torch.isfinite(a).all().item(), f"{name}: non-finite"
    assert a.abs().max().item() > 0, f"{name}: all zero"
    assert torch.equal(b, 2 * a), f"{name}: output of the doubled input is not exactly twice the output"


def test_attn_fwd_L8192_linear_in_v_exactly():
    from hstu_sequential_transduction_attn_amd import _lib as ops
    print("\n[case] attn_L8192 forward, V doubled", flush=True)
    case = C.attn_L8192()
    jd = jag_dev(case.jagged)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    wp, wt = dev(case.rab.pos_bias), dev(case.rab.time_bias)
    run = lambda vv: ops.attn_fwd(jd["seq_offsets"], jd["timestamps"], q, k, vv, wp, wt,
                                  max_seq_len=jd["max_seq_len"])
    o1 = run(v)
    o2 = run(2 * v)
    o3 = run(v)
    torch.cuda.synchronize()
    _equal_times_two(o1.float(), o2.float(), "O")
    assert torch.equal(o1, o3), "two runs differ"


def test_attn_bwd_L8192_linear_in_d_out_exactly():
    from hstu_sequential_transduction_attn_amd import _lib as ops
    print("\n[case] attn_L8192 backward, dO doubled", flush=True)
    case = C.attn_L8192()
    jd = jag_dev(case.jagged)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    wp, wt = dev(case.rab.pos_bias), dev(case.rab.time_bias)
    gen = torch.Generator(device="cuda").manual_seed(11)
    g = torch.randn(q.shape, device="cuda", generator=gen).to(torch.bfloat16)
    run = lambda gg: ops.attn_bwd(jd["seq_offsets"], jd["timestamps"], q, k, v, gg, wp, wt,
                                  max_seq_len=jd["max_seq_len"])
    r1 = run(g)
    r2 = run(2 * g)
    r3 = run(g)
    torch.cuda.synchronize()
    for a, b, c, name in zip(r1, r2, r3, ["dq", "dk", "dv", "d_pos_bias", "d_time_bias"]):
        _equal_times_two(a, b, name)
        assert torch.equal(a, c), f"{name}: two runs differ"


def test_layer_bwd_stack8_layer_shape_linear_in_dy_exactly():
    """One layer of the 8-layer stack (T = 145,051, D = 1024, H = 8 x 128, output LayerNorm, fp32
    activations and gradients, split activation operands), every gradient for dy and 2 dy."""
    from hstu_sequential_transduction_attn_amd import _lib as ops
    print("\n[case] stack8 layer 0 backward, dy doubled", flush=True)
    case = C.stack8_bf16(num_layers=1)
    L = case.layers[0]
    jd = jag_dev(case.jagged)
    T, D = case.jagged.total_tokens, case.d_model
    gen = torch.Generator(device="cuda").manual_seed(12)
    x = torch.randn((T, D), device="cuda", generator=gen)
    dy = torch.randn((T, D), device="cuda", generator=gen)
    args = (jd["seq_offsets"], jd["timestamps"], dev(L.w_uvqk), dev(L.w_out), dev(L.rab.pos_bias),
            dev(L.rab.time_bias), case.num_heads, case.head_dim)
    nws = ops.layer_bwd_workspace_bytes(x, *args, max_seq_len=jd["max_seq_len"], ln_output=True)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    run = lambda gg: {k: v.clone() if v is not None else None for k, v in ops.layer_bwd(
        x, gg, *args, max_seq_len=jd["max_seq_len"], ln_eps=L.ln_eps, ln_output=True, act_split=True,
        workspace=ws).items()}
    r1 = run(dy)
    r2 = run(2 * dy)
    r3 = run(dy)
    torch.cuda.synchronize()
    for name in ("dx", "d_w_uvqk", "d_b_uvqk", "d_w_out", "d_b_out", "d_pos_bias", "d_time_bias"):
        _equal_times_two(r1[name], r2[name], name)
        assert torch.equal(r1[name], r3[name]), f"{name}: two runs differ"
