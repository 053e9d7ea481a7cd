"""GPU parity of hstu_layer_bwd (the whole layer's backward) against the float64 oracle gradients.

The oracle's layer gradients are pinned to finite differences of the forward oracle
(test_oracle_layer_backward).  Cases: fp32 and bf16, with and without the post-layer LayerNorm,
nonzero biases, ragged batches with empty and one-token sequences, odd model widths (plain GEMM
tails), batches large enough for the large-tile and split-K weight-gradient GEMMs, the candidate
mask, an fp32 gradient stream with fp32 activations, an empty batch, and bitwise determinism.
bf16 cases are held to the kernels' own bar plus 8 sigma of the noise that the bf16 storage of the
attention's q, k, v and dO puts on each gradient element (see _check and tests/_noise.py).
"""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import inputs as I
from oracle import hstu_oracle as O

from _noise import operand_noise
from _util import dev, host, jag_dev, max_abs, oracle_jag, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

NAMES = ["dx", "d_w_uvqk", "d_b_uvqk", "d_w_out", "d_b_out", "d_pos_bias", "d_time_bias"]


def _dy(case, seed, dtype):
    rng = np.random.default_rng(seed)
    return I.Tensor.make(rng.standard_normal(case.x.shape).astype(np.float32), dtype)


def _gpu(case, dy, ln_output, x_f32=False, act_split=False):
    from hstu_sequential_transduction_attn_amd import _lib as ops
    jd = jag_dev(case.jagged)
    L = case.layers[0]
    x = dev(case.x) if not x_f32 else torch.from_numpy(case.x.values.copy()).cuda()
    out = ops.layer_bwd(x, dev(dy), jd["seq_offsets"], jd["timestamps"], dev(L.w_uvqk), dev(L.w_out),
                        dev(L.rab.pos_bias), dev(L.rab.time_bias), case.num_heads, case.head_dim,
                        max_seq_len=jd["max_seq_len"], b_uvqk=None if L.b_uvqk is None else dev(L.b_uvqk),
                        b_out=None if L.b_out is None else dev(L.b_out), ln_eps=L.ln_eps, ln_output=ln_output,
                        mask=jd["mask"], num_candidates=jd["num_candidates"], attn_scale=jd["attn_scale"],
                        act_split=act_split)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def _oracle(case, dy, ln_output, noise_samples=0, seed=0):
    """The exact float64 gradients and, with noise_samples, the per-element sigma of the noise that
    the bf16 storage of the attention's q, k, v and dO puts on them (tests/_noise.py)."""
    L = case.layers[0]

    def run(f):
        return O.layer_bwd(case.x.values, oracle_jag(case.jagged), L.w_uvqk.values,
                           None if L.b_uvqk is None else L.b_uvqk.values, L.w_out.values,
                           None if L.b_out is None else L.b_out.values, L.rab.pos_bias, L.rab.time_bias,
                           case.num_heads, case.head_dim, L.ln_eps, ln_output, dy.values, return_sq=True,
                           attn_operands=f)
    if not noise_samples:
        return run(None), None
    return operand_noise(run, samples=noise_samples, seed=seed)


def _check(got, want_sigma, dtype, what):
    """fp32: rel-L2 <= 1e-5 on every gradient.
    bf16: the bar the kernels meet with exact operands, plus 8 sigma of the noise of the attention's
    bf16 operands (q, k, v, dO: independent relative errors up to 2^-8 per element, carried through
    the float64 oracle, so that the correlation of one token's errors over all its pairs is kept):
      dx, weight and bias-vector gradients: |err| <= 2e-2 + 2^-7 max|want| + 8 sigma elementwise and
        rel-L2 <= 5e-3 + 3 ||sigma|| / ||want||;
      bias-table gradients, per bin: |err| <= 4 * 2^-7 sqrt(sum dS^2) + 2^-7 |want| + 1e-6 + 8 sigma
        (the attention-level bin bar: each bin sums many dS terms with their own roundings)."""
    want, sigma = want_sigma
    for name in NAMES:
        x, y = np.asarray(got[name], np.float64), want[name]
        assert np.all(np.isfinite(x)), f"{what} {name}: non-finite"
        r, m = rel_l2(x, y), max_abs(x, y)
        if dtype != "bf16":
            print(f"  {name:12s} rel_l2={r:.3e} max_abs={m:.3e}")
            assert r <= 1e-5, f"{what} {name}: rel_l2={r:.3e} max_abs={m:.3e}"
            continue
        err = np.abs(x - y)
        sg = sigma[name]
        if name in ("d_pos_bias", "d_time_bias"):
            bound = 4 * 2.0 ** -7 * np.sqrt(want[name + "_sq"]) + 2.0 ** -7 * np.abs(y) + 1e-6 + 8 * sg
            rbar = None
        else:
            ymax = float(np.abs(y).max() if y.size else 0.0)
            bound = 2e-2 + 2.0 ** -7 * ymax + 8 * sg
            ny = float(np.linalg.norm(y))
            rbar = 5e-3 + 3 * float(np.linalg.norm(sg)) / (ny if ny > 0 else 1.0)
        use = float((err / bound).max()) if err.size else 0.0
        print(f"  {name:12s} rel_l2={r:.3e} max_abs={m:.3e} max|err|/bar={use:.3f} "
              f"max 8sigma={8 * float(sg.max()) if sg.size else 0.0:.3e}")
        assert use <= 1.0, f"{what} {name}: max|err|/bar={use:.3f} rel_l2={r:.3e} max_abs={m:.3e}"
        if rbar is not None:
            assert r <= rbar, f"{what} {name}: rel_l2={r:.3e} > {rbar:.3e}"


@pytest.mark.parametrize("ln_output", [False, True])
def test_layer_bwd_f32_small(ln_output):
    print(f"\n[case] layer bwd f32 small ln_output={ln_output}", flush=True)
    case = I.jagged_layer_case("lbwd32", 1300, [5, 1, 0, 70, 128, 33], D=64, H=2, Dh=32, P=32, Tb=32, dtype="f32",
                               bias_std=0.3)
    dy = _dy(case, 1301, "f32")
    _check(_gpu(case, dy, ln_output), _oracle(case, dy, ln_output), "f32", "f32 small")


@pytest.mark.parametrize("ln_output", [False, True])
def test_layer_bwd_bf16_ragged_odd_width(ln_output):
    """D = 72 and H*Dh = 192: no GEMM dimension is a multiple of the large tiles."""
    print(f"\n[case] layer bwd bf16 ragged D=72 ln_output={ln_output}", flush=True)
    case = I.jagged_layer_case("lbwd", 1310, [1, 0, 129, 64, 200, 31], D=72, H=3, Dh=64, P=50, Tb=30, dtype="bf16",
                               bias_std=0.3)
    dy = _dy(case, 1311, "bf16")
    _check(_gpu(case, dy, ln_output), _oracle(case, dy, ln_output, 24, 1312), "bf16", "bf16 ragged")


def test_layer_bwd_bf16_large_tiles_split_k():
    """About 20k tokens at D = 512, H*Dh = 512: the dg and dx GEMMs take the large-tile kernel, the
    weight gradients (K = the padded token count) are split over K."""
    print("\n[case] layer bwd bf16 large tiles + split-K", flush=True)
    rng = np.random.default_rng(1320)
    lengths = [int(v) for v in rng.integers(1, 1025, size=40)]
    case = I.jagged_layer_case("lbwdL", 1320, lengths, D=512, H=4, Dh=128, P=128, Tb=128, dtype="bf16",
                               bias_std=0.1)
    print(f"  T={sum(lengths)}", flush=True)
    dy = _dy(case, 1321, "bf16")
    _check(_gpu(case, dy, True), _oracle(case, dy, True, 8, 1322), "bf16", "bf16 large")


def test_layer_bwd_candidates():
    print("\n[case] layer bwd bf16 candidates", flush=True)
    case = I.jagged_layer_case("lbwdc", 1330, [150, 40, 300, 1], D=128, H=2, Dh=128, P=64, Tb=64, dtype="bf16",
                               bias_std=0.2)
    case.jagged.mask = I.CAUSAL_CANDIDATES
    case.jagged.num_candidates = np.array([50, 1, 100, 1], np.int32)
    dy = _dy(case, 1331, "bf16")
    _check(_gpu(case, dy, False), _oracle(case, dy, False, 24, 1332), "bf16", "candidates")


@pytest.mark.parametrize("act_split", [False, True])
def test_layer_bwd_fp32_gradient_stream(act_split):
    """bf16 weights, fp32 x and fp32 dy / dx (the fp32 residual stream of a stack)."""
    print(f"\n[case] layer bwd fp32 stream act_split={act_split}", flush=True)
    case = I.jagged_layer_case("lbwdf", 1340, [70, 1, 300, 129], D=256, H=2, Dh=128, P=64, Tb=64, dtype="bf16",
                               bias_std=0.2)
    case.x = I.Tensor.make(case.x.values, "f32")   # the oracle reads the same fp32 x
    dy = _dy(case, 1341, "f32")
    _check(_gpu(case, dy, True, x_f32=True, act_split=act_split), _oracle(case, dy, True, 24, 1342), "bf16",
           "fp32 stream")


def test_layer_bwd_empty_batch_zeroes_every_gradient():
    from hstu_sequential_transduction_attn_amd import _lib as ops
    print("\n[case] layer bwd empty batch", flush=True)
    case = I.jagged_layer_case("lbwd0", 1350, [0, 0], D=64, H=2, Dh=64, P=16, Tb=16, dtype="bf16", bias_std=0.1)
    L = case.layers[0]
    jd = jag_dev(case.jagged)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    grads = dict(d_w_uvqk=torch.full((512, 64), 7.0, **f32), d_b_uvqk=torch.full((512,), 7.0, **f32),
                 d_w_out=torch.full((64, 128), 7.0, **f32), d_b_out=torch.full((64,), 7.0, **f32),
                 d_pos_bias=torch.full((1, 16), 7.0, **f32), d_time_bias=torch.full((1, 16), 7.0, **f32))
    out = ops.layer_bwd(x, x.clone(), jd["seq_offsets"], jd["timestamps"], dev(L.w_uvqk), dev(L.w_out),
                        dev(L.rab.pos_bias), dev(L.rab.time_bias), 2, 64, max_seq_len=0,
                        b_uvqk=dev(L.b_uvqk), b_out=dev(L.b_out), grads=grads)
    torch.cuda.synchronize()
    assert out["dx"].shape == (0, 64)
    for k, v in grads.items():
        assert out[k] is v
        assert not torch.any(v != 0).item(), k


def test_layer_bwd_is_bitwise_deterministic():
    print("\n[case] layer bwd determinism", flush=True)
    rng = np.random.default_rng(1360)
    lengths = [int(v) for v in rng.integers(1, 700, size=12)]
    case = I.jagged_layer_case("lbwdd", 1360, lengths, D=256, H=2, Dh=128, P=64, Tb=64, dtype="bf16", bias_std=0.1)
    dy = _dy(case, 1361, "bf16")
    a = _gpu(case, dy, True)
    b = _gpu(case, dy, True)
    for name in NAMES:
        assert np.array_equal(a[name], b[name]), name


@pytest.mark.parametrize("dtype,ln_output", [("f32", True), ("bf16", False), ("bf16", True)])
def test_layer_bwd_from_saved_activations_is_bitwise_the_recompute(dtype, ln_output):
    """hstu_layer_fwd_save's y is hstu_layer_fwd's, and hstu_layer_bwd_saved's gradients are
    hstu_layer_bwd's, bit for bit (the recompute path is the one held to the oracle above)."""
    from hstu_sequential_transduction_attn_amd import _lib as ops
    print(f"\n[case] layer bwd from saved activations {dtype} ln_output={ln_output}", flush=True)
    rng = np.random.default_rng(1370)
    lengths = [int(v) for v in rng.integers(1, 700, size=16)] + [0, 1]
    D, H, Dh = (64, 2, 32) if dtype == "f32" else (256, 2, 128)
    case = I.jagged_layer_case("lbwds", 1370, lengths, D=D, H=H, Dh=Dh, P=64, Tb=64, dtype=dtype, bias_std=0.2)
    L = case.layers[0]
    jd = jag_dev(case.jagged)
    x = dev(case.x)
    dy = dev(_dy(case, 1371, dtype))
    args = (jd["seq_offsets"], jd["timestamps"], dev(L.w_uvqk), dev(L.w_out), dev(L.rab.pos_bias),
            dev(L.rab.time_bias), case.num_heads, case.head_dim)
    kw = dict(max_seq_len=jd["max_seq_len"], b_uvqk=dev(L.b_uvqk), b_out=dev(L.b_out), ln_eps=L.ln_eps,
              ln_output=ln_output)
    y_plain = ops.layer_fwd(x, *args, **kw)
    nsv = ops.layer_saved_bytes(x, *args, max_seq_len=jd["max_seq_len"], ln_output=ln_output)
    saved = torch.empty(nsv, dtype=torch.uint8, device="cuda")
    y_saved = ops.layer_fwd(x, *args, saved=saved, **kw)
    want = ops.layer_bwd(x, dy, *args, **kw)
    got = ops.layer_bwd(x, dy, *args, saved=saved, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y_plain, y_saved), "forward with saved activations differs"
    for name in NAMES:
        assert torch.equal(got[name], want[name]), f"{name}: backward from saved activations differs"


@pytest.mark.parametrize("seed", [7021, 7052, 7003, 7037])
def test_layer_bwd_f32_random_shapes(seed):
    """fp32 layers on seeded random shapes (widths that are not multiples of the tiles, tiny and odd
    bias tables, candidates, biases, the output LayerNorm), checked to 1e-5 relative: the arithmetic of
    every step with no bf16 rounding to hide behind."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.integers(0, 300, B)]
    if rng.random() < 0.3:
        lengths[0] = int(rng.integers(300, 1100))
    D = int(rng.choice([32, 64, 72, 96, 128, 200, 256]))
    H, Dh = int(rng.integers(1, 4)), int(rng.choice([32, 64, 128]))
    P, Tb = int(rng.integers(1, 200)), int(rng.integers(1, 70))
    ln_output = bool(rng.random() < 0.5)
    case = I.jagged_layer_case("lrnd", seed, lengths, D=D, H=H, Dh=Dh, P=P, Tb=Tb, dtype="f32",
                               bias_std=float(rng.choice([0.0, 0.2])))
    if rng.random() < 0.4:
        case.jagged.mask = I.CAUSAL_CANDIDATES
        case.jagged.num_candidates = np.array([int(rng.integers(0, n + 1)) for n in lengths], np.int32)
    print(f"\n[case] layer bwd f32 random seed={seed} lengths={lengths} D={D} H={H} Dh={Dh} P={P} Tb={Tb} "
          f"ln_output={ln_output} candidates={case.jagged.num_candidates is not None}", flush=True)
    dy = _dy(case, seed + 1, "f32")
    _check(_gpu(case, dy, ln_output), _oracle(case, dy, ln_output), "f32", f"random {seed}")


@pytest.mark.parametrize("seed", list(range(7101, 7111)))
def test_layer_bwd_bf16_random_shapes(seed):
    """bf16 layers on seeded random shapes: every one of the generator's first ten seeds (tables from 1
    bucket, sequences from 1 token, odd widths, candidates, biases, the output LayerNorm, fp32 streams
    with and without split activations), at the bar of _check: the kernels' own bar plus 8 sigma of
    the noise of the attention's bf16 operands."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.integers(1, 300, B)]
    if rng.random() < 0.3:
        lengths[0] = int(rng.integers(300, 1100))
    D = int(rng.choice([64, 72, 96, 128, 200, 256, 512]))
    H, Dh = int(rng.integers(1, 4)), int(rng.choice([32, 64, 128]))
    P, Tb = int(rng.integers(1, 200)), int(rng.integers(1, 70))
    ln_output = bool(rng.random() < 0.5)
    case = I.jagged_layer_case("lrndb", seed, lengths, D=D, H=H, Dh=Dh, P=P, Tb=Tb, dtype="bf16",
                               bias_std=float(rng.choice([0.0, 0.2])))
    if rng.random() < 0.4:
        case.jagged.mask = I.CAUSAL_CANDIDATES
        case.jagged.num_candidates = np.array([int(rng.integers(0, n // 2 + 1)) for n in lengths], np.int32)
    x_f32 = bool(rng.random() < 0.4)
    act_split = x_f32 and bool(rng.random() < 0.5)
    if x_f32:
        case.x = I.Tensor.make(case.x.values, "f32")
    print(f"\n[case] layer bwd bf16 random seed={seed} lengths={lengths} D={D} H={H} Dh={Dh} P={P} Tb={Tb} "
          f"ln_output={ln_output} candidates={case.jagged.num_candidates is not None} x_f32={x_f32} "
          f"split={act_split}", flush=True)
    dy = _dy(case, seed + 1, "f32" if x_f32 else "bf16")
    got = _gpu(case, dy, ln_output, x_f32=x_f32, act_split=act_split)
    _check(got, _oracle(case, dy, ln_output, 24, seed + 2), "bf16", f"random {seed}")


@pytest.mark.parametrize("P,Tb,ln_output,x_f32,act_split", [
    (1, 1, True, False, False),
    (2, 3, False, True, True),
    (3, 1, True, True, False),
])
def test_layer_bwd_bf16_tiny_tables_and_short_sequences(P, Tb, ln_output, x_f32, act_split):
    """The shapes that break a bar built on independent pair terms: tables of 1 to 3 buckets (one bin
    pools most pairs of every sequence) and sequences of 1 to 7 tokens (each gradient sums few pairs),
    beside one longer sequence, with candidates; held to the same bar as every bf16 case."""
    lengths = [1, 2, 3, 4, 5, 6, 7, 1, 150]
    seed = 7150 + 10 * P + Tb
    case = I.jagged_layer_case("ltiny", seed, lengths, D=128, H=2, Dh=64, P=P, Tb=Tb, dtype="bf16", bias_std=0.2)
    case.jagged.mask = I.CAUSAL_CANDIDATES
    case.jagged.num_candidates = np.array([0, 1, 1, 2, 0, 3, 2, 0, 20], np.int32)
    if x_f32:
        case.x = I.Tensor.make(case.x.values, "f32")
    print(f"\n[case] layer bwd bf16 tiny tables P={P} Tb={Tb} ln_output={ln_output} x_f32={x_f32} split={act_split}",
          flush=True)
    dy = _dy(case, seed + 1, "f32" if x_f32 else "bf16")
    got = _gpu(case, dy, ln_output, x_f32=x_f32, act_split=act_split)
    _check(got, _oracle(case, dy, ln_output, 24, seed + 2), "bf16", f"tiny tables P={P} Tb={Tb}")
