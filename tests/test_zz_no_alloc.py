"""hstu_attn_fwd_noalloc (the forward for callers that cannot allocate device memory) against
hstu_attn_fwd, through the C ABI: the same kernels, so the outputs must agree bit for bit, on two
calls in a row with the second batch smaller than the first (the fixed scratch keeps the last call's
contents, so the second call must not read any of them), and both must meet the oracle bar."""
import numpy as np
import pytest

from hstu_sequential_transduction_attn_amd import _lib as ops
from hstu_sequential_transduction_attn_amd import inputs as I
from oracle import hstu_oracle as O

from _util import assert_close, dev, gpu_attn, host, jag_dev, oracle_jag

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _noalloc(case, out_dtype):
    jd = jag_dev(case.jagged)
    q = dev(case.q)
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=q.device)
    ops.attn_fwd_noalloc(jd["seq_offsets"], jd["timestamps"], q, dev(case.k), dev(case.v), dev(case.rab.pos_bias),
                         dev(case.rab.time_bias), max_seq_len=jd["max_seq_len"], mask=jd["mask"],
                         num_candidates=jd["num_candidates"], attn_scale=jd["attn_scale"], out=out)
    return out


def _oracle(case):
    return O.attn_fwd(oracle_jag(case.jagged), case.q.values, case.k.values, case.v.values, case.rab.pos_bias,
                      case.rab.time_bias)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_attn_fwd_on_two_calls(dtype):
    out_dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    big = I.attn_case("noalloc_big", 3101, [1500, 1, 0, 129, 700, 64], H=4, Dh=128, P=256, Tb=256, dtype=dtype)
    small = I.attn_case("noalloc_small", 3102, [65, 300, 2], H=4, Dh=128, P=256, Tb=256, dtype=dtype)
    for case in (big, small):
        print(f"\n[case] noalloc {case.name} dtype={dtype} T={case.jagged.total_tokens}", flush=True)
        got = _noalloc(case, out_dt)
        want = gpu_attn(case, out_dtype=out_dt)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16 if dtype == "bf16" else torch.int32),
                           want.view(torch.int16 if dtype == "bf16" else torch.int32)), case.name
        assert_close(host(got), _oracle(case), dtype, f"noalloc {case.name}", magnitude_aware=dtype == "bf16")


def test_noalloc_candidates_two_calls():
    for seed, lengths, cands in ((3103, [400, 90, 33], [100, 90, 1]), (3104, [50, 7], [10, 0])):
        case = I.attn_case("noalloc_cand", seed, lengths, H=2, Dh=64, P=64, Tb=32, dtype="bf16",
                           num_candidates=cands)
        print(f"\n[case] noalloc candidates seed={seed} T={case.jagged.total_tokens}", flush=True)
        got = _noalloc(case, torch.float32)
        want = gpu_attn(case, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32))
        assert_close(host(got), _oracle(case), "bf16", "noalloc candidates", magnitude_aware=True)
