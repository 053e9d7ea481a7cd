"""Shared test helpers: host->device marshalling of the seeded inputs, oracle argument packing,
and the error metrics used by every parity check."""
from __future__ import annotations

import numpy as np

from hstu_sequential_transduction_attn_amd import inputs as I

# Tolerances on the final output tensor.
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
F32_REL_L2 = 1e-5


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want.ravel())
    return float(np.linalg.norm((got - want).ravel()) / (den if den > 0 else 1.0))


def max_abs(got: np.ndarray, want: np.ndarray) -> float:
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    return float(d.max()) if d.size else 0.0


# Ad-hoc (non-workload) cases can have outputs of magnitude ~100 (a length-1 sequence has c_b = 1 and
# O = SiLU(s) v with |s| up to ~35), where one bf16 ulp is 0.5.  For them the absolute bar grows with the
# value.  bf16 keeps 8 significant bits, so one round-to-nearest moves a value by up to half an ulp,
# 2^-8 of it; such an output is rounded twice (SiLU(s) as the bf16 AV operand, then the bf16 output),
# which moves it by up to 2^-7 |want|.
BF16_REL_ELEM = 2.0 ** -7


def assert_close(got, want, dtype: str, what: str = "", magnitude_aware: bool = False):
    """The workloads' bar: bf16 max_abs <= 2e-2 and rel_l2 <= 5e-3; f32 rel_l2 <= 1e-5.
    magnitude_aware (ad-hoc bf16 cases only): |got - want| <= 2e-2 + 2^-7 |want| elementwise."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    r, m = rel_l2(got, want), max_abs(got, want)
    if dtype == "bf16":
        assert r <= BF16_REL_L2, f"{what}: rel_l2={r:.3e} max_abs={m:.3e}"
        if magnitude_aware:
            excess = np.abs(got - want) - (BF16_MAX_ABS + BF16_REL_ELEM * np.abs(want))
            assert excess.size == 0 or excess.max() <= 0, f"{what}: elementwise bound exceeded by {excess.max():.3e}"
        else:
            assert m <= BF16_MAX_ABS, f"{what}: max_abs={m:.3e} rel_l2={r:.3e}"
    else:
        assert r <= F32_REL_L2, f"{what}: rel_l2={r:.3e} max_abs={m:.3e}"
    return r, m


def oracle_jag(j: I.Jagged) -> dict:
    return dict(seq_offsets=j.seq_offsets.astype(np.int64), timestamps=j.timestamps, mask=j.mask,
                num_candidates=j.num_candidates, attn_scale=j.attn_scale)


def oracle_layers(case: I.LayerCase):
    out = []
    for L in case.layers:
        out.append(dict(w_uvqk=L.w_uvqk.values, b_uvqk=None if L.b_uvqk is None else L.b_uvqk.values,
                        w_out=L.w_out.values, b_out=None if L.b_out is None else L.b_out.values,
                        pos_bias=L.rab.pos_bias, time_bias=L.rab.time_bias, ln_eps=L.ln_eps))
    return out


def sub_jagged(j: I.Jagged, seqs) -> tuple:
    """Restrict a jagged batch to some sequences: returns (Jagged, token index array)."""
    offs = j.seq_offsets.astype(np.int64)
    idx = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in seqs]) if len(seqs) else np.zeros(0, np.int64)
    lengths = [int(offs[b + 1] - offs[b]) for b in seqs]
    nc = None if j.num_candidates is None else j.num_candidates[list(seqs)]
    sc = None if j.attn_scale is None else j.attn_scale[list(seqs)]
    return I.Jagged(seq_offsets=I.offsets_of(lengths), timestamps=j.timestamps[idx], num_candidates=nc,
                    attn_scale=sc, mask=j.mask), idx


# --------------------------------------------------------------------------- device side (torch)
def dev(t, device="cuda"):
    import torch
    if isinstance(t, I.Tensor):
        if t.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(t.values)).to(device)
    return torch.from_numpy(np.ascontiguousarray(t)).to(device)


def host(x) -> np.ndarray:
    import torch
    return x.detach().to(torch.float32).cpu().numpy()


def jag_dev(j: I.Jagged):
    return dict(seq_offsets=dev(j.seq_offsets.astype(np.int32)), timestamps=dev(j.timestamps.astype(np.int64)),
                num_candidates=None if j.num_candidates is None else dev(j.num_candidates.astype(np.int32)),
                attn_scale=None if j.attn_scale is None else dev(j.attn_scale.astype(np.float32)),
                max_seq_len=j.max_seq_len, mask=j.mask)


def gpu_attn(case: I.AttnCase, out_dtype=None):
    from hstu_sequential_transduction_attn_amd import _lib as ops
    jd = jag_dev(case.jagged)
    return ops.attn_fwd(jd["seq_offsets"], jd["timestamps"], dev(case.q), dev(case.k), dev(case.v),
                        dev(case.rab.pos_bias), dev(case.rab.time_bias), max_seq_len=jd["max_seq_len"],
                        mask=jd["mask"], num_candidates=jd["num_candidates"], attn_scale=jd["attn_scale"],
                        out_dtype=out_dtype)


def gpu_layer_stack(case: I.LayerCase, use_gather: bool = False, residual_f32: bool = False,
                    act_split: bool = False):
    """Run every layer of the case on the GPU (post-layer LayerNorm on all but the last layer).
    residual_f32: the activations between layers (and the final output) are fp32."""
    import torch
    from hstu_sequential_transduction_attn_amd import _lib as ops
    jd = jag_dev(case.jagged)
    x = gather_input(case) if use_gather else dev(case.x)
    ws = None
    for li, L in enumerate(case.layers):
        args = (jd["seq_offsets"], jd["timestamps"], dev(L.w_uvqk), dev(L.w_out), dev(L.rab.pos_bias),
                dev(L.rab.time_bias), case.num_heads, case.head_dim)
        ln_out = li < len(case.layers) - 1
        if ws is None:
            n = ops.layer_workspace_bytes(x, *args, max_seq_len=jd["max_seq_len"], ln_output=True, mask=jd["mask"],
                                          act_split=act_split)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
        x = ops.layer_fwd(x, *args, max_seq_len=jd["max_seq_len"],
                          b_uvqk=None if L.b_uvqk is None else dev(L.b_uvqk),
                          b_out=None if L.b_out is None else dev(L.b_out), ln_eps=L.ln_eps, ln_output=ln_out,
                          mask=jd["mask"], num_candidates=jd["num_candidates"], attn_scale=jd["attn_scale"],
                          y_dtype=torch.float32 if residual_f32 else None, act_split=act_split, workspace=ws)
    return x


def gather_input(case: I.LayerCase):
    """Full-size device table (untouched rows zero) and the hstu_gather_rows staging of X0."""
    import torch
    from hstu_sequential_transduction_attn_amd import _lib as ops
    table = torch.zeros((case.table_rows, case.d_model), dtype=torch.bfloat16, device="cuda")
    rows = dev(case.table_values)
    table.index_copy_(0, dev(case.table_touched.astype(np.int64)), rows)
    return ops.gather_rows(table, dev(case.ids.astype(np.int64)))


# --------------------------------------------------------------------------- full-size workloads
_CACHE = {}


def cached(key, make):
    """Compute make() once per test session (the workload cases and the oracle outputs of their longest
    sequences are shared by the layer-path and stack-path tests)."""
    if key not in _CACHE:
        _CACHE[key] = make()
    return _CACHE[key]


def workload_case(name):
    from hstu_sequential_transduction_attn_amd import configs as C
    return cached(("case", name), getattr(C, name))


def workload_sequences(case, shortest: int = 2):
    """The `shortest` shortest sequences and the longest one (stable order of their lengths)."""
    order = np.argsort(case.jagged.lengths, kind="stable")
    return sorted({int(s) for s in order[:shortest]} | {int(order[-1])})


def oracle_stack_sequence(name, case, seq):
    """The float64 oracle of the whole stack on one sequence of a workload (jagged independence: a
    sequence's output depends on its own tokens only)."""
    from oracle import hstu_oracle as O

    def make():
        jag, idx = sub_jagged(case.jagged, [seq])
        return O.stack_fwd(case.x.values[idx], oracle_jag(jag), oracle_layers(case), case.num_heads, case.head_dim)
    return cached(("oracle", name, seq), make)
