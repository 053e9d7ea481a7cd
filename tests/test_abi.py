"""The C-ABI library on the host: it loads, exports every function include/hstu.h declares, and rejects
invalid arguments with the documented status before anything reaches the GPU.

No call here launches a kernel: every case fails validation (or has zero tokens) first, so these
tests run without a GPU.  Pointers are fake device addresses that are never dereferenced.
"""
import ctypes
import os

import pytest

from hstu_sequential_transduction_attn_amd import _lib as L

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libhstu.so not built")

OK, INVALID, UNSUPPORTED, WS_SMALL, DEVICE = 0, 1, 2, 3, 4
P16 = 0x7F0000000000  # a 16-byte aligned fake device address


def _lib():
    return L.load_library()


def _jag(B=2, T=100, max_len=60, cand=False):
    return L.JaggedT(B, T, max_len, P16, P16 + 0x1000, P16 + 0x2000 if cand else None, None)


def _desc(H=4, Dh=128, P=32, Tb=32, R=1, mask=0):
    return L.AttnDescT(H, Dh, P, Tb, R, P16 + 0x3000, P16 + 0x4000, mask)


def _attn(jag, desc, in_dt=L.HSTU_BF16, out_dt=L.HSTU_BF16, q=P16 + 0x10000, k=P16 + 0x20000000,
          v=P16 + 0x40000000, out=P16 + 0x60000000, ws=P16 + 0x80000000, nws=1 << 20):
    lib = _lib()
    st = lib.hstu_attn_fwd(ctypes.byref(jag) if jag else None, ctypes.byref(desc) if desc else None, in_dt, q, k, v,
                           out, out_dt, ws, nws, None)
    return st, lib.hstu_last_error().decode()


def test_exports_every_declared_symbol():
    names = L.exported_functions_in_header()
    assert len(names) == 22
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = _lib()
    assert lib.hstu_abi_version() == 9
    assert lib.hstu_status_string(OK) == b"HSTU_OK"
    assert lib.hstu_status_string(WS_SMALL) == b"HSTU_ERR_WORKSPACE_TOO_SMALL"
    assert lib.hstu_status_string(99) == b"HSTU_STATUS_UNKNOWN"


def test_attn_argument_errors():
    assert _attn(None, _desc())[0] == INVALID
    assert _attn(_jag(), None)[0] == INVALID
    st, msg = _attn(_jag(), _desc(Dh=48))
    assert st == UNSUPPORTED and "head_dim" in msg
    assert _attn(_jag(), _desc(H=0))[0] == INVALID
    assert _attn(_jag(), _desc(P=0))[0] == INVALID
    assert _attn(_jag(), _desc(Tb=5000))[0] == INVALID
    assert _attn(_jag(), _desc(R=3))[0] == INVALID
    assert _attn(_jag(), _desc(mask=7))[0] == INVALID
    st, msg = _attn(_jag(cand=False), _desc(mask=1))
    assert st == INVALID and "num_candidates" in msg
    assert _attn(_jag(B=-1), _desc())[0] == INVALID
    assert _attn(_jag(max_len=101), _desc())[0] == INVALID           # max_seq_len > total_tokens
    assert _attn(_jag(B=0, T=5, max_len=0), _desc())[0] == INVALID
    assert _attn(_jag(), _desc(), in_dt=L.HSTU_F32, out_dt=L.HSTU_BF16)[0] == UNSUPPORTED
    assert _attn(_jag(), _desc(), in_dt=7)[0] == INVALID
    assert _attn(_jag(), _desc(), q=None)[0] == INVALID
    st, msg = _attn(_jag(), _desc(), q=P16 + 2)
    assert st == INVALID and "aligned" in msg
    st, msg = _attn(_jag(), _desc(), out=P16 + 0x10000 + 64)             # out overlaps q
    assert st == INVALID and "overlaps" in msg
    jag = L.JaggedT(2, 100, 60, None, P16, None, None)
    assert _attn(jag, _desc())[0] == INVALID                              # seq_offsets NULL
    assert _attn(_jag(), L.AttnDescT(4, 128, 32, 32, 1, None, P16, 0))[0] == INVALID


def test_attn_zero_tokens_is_a_no_op():
    jag = L.JaggedT(3, 0, 0, P16, None, None, None)
    assert _lib().hstu_attn_workspace_bytes(ctypes.byref(jag), ctypes.byref(_desc()), L.HSTU_BF16) == 0
    st, msg = _attn(jag, _desc(), q=None, k=None, v=None, out=None, ws=None, nws=0)
    assert st == OK and msg == ""


def _noalloc(jag, desc, in_dt=L.HSTU_BF16, out_dt=L.HSTU_BF16, q=P16 + 0x10000, k=P16 + 0x20000000,
             v=P16 + 0x40000000, out=P16 + 0x60000000):
    lib = _lib()
    st = lib.hstu_attn_fwd_noalloc(ctypes.byref(jag) if jag else None, ctypes.byref(desc) if desc else None, in_dt,
                                   q, k, v, out, out_dt, None)
    return st, lib.hstu_last_error().decode()


def test_noalloc_checks_before_touching_the_device():
    # the argument checks of hstu_attn_fwd, without a workspace
    assert _noalloc(None, _desc())[0] == INVALID
    st, msg = _noalloc(_jag(), _desc(Dh=48))
    assert st == UNSUPPORTED and "head_dim" in msg
    assert _noalloc(_jag(), _desc(), in_dt=L.HSTU_F32, out_dt=L.HSTU_BF16)[0] == UNSUPPORTED
    assert _noalloc(_jag(), _desc(), q=None)[0] == INVALID
    st, msg = _noalloc(_jag(), _desc(), out=P16 + 0x10000 + 64)
    assert st == INVALID and "overlaps" in msg
    # zero tokens: nothing to do, nothing looked up
    jag = L.JaggedT(3, 0, 0, P16, None, None, None)
    assert _noalloc(jag, _desc(), q=None, k=None, v=None, out=None) == (OK, "")
    # the fixed scratch holds T/32 + B + 1 <= 65536 timestamp ranges: the largest batch that fits ...
    B = 5
    T_fit = (65536 - B - 1) * 32 + 31
    big_q = 1 << 44
    fit = L.JaggedT(B, T_fit, 1 << 20, P16, P16 + 0x1000, None, None)
    need = _lib().hstu_attn_workspace_bytes(ctypes.byref(fit), ctypes.byref(_desc()), L.HSTU_BF16)
    assert need == 1 << 20
    # ... and one token more is refused before any launch, naming both sizes
    over = L.JaggedT(B, T_fit + 1, 1 << 20, P16, P16 + 0x1000, None, None)
    st, msg = _noalloc(over, _desc(), q=P16 + big_q, k=P16 + 2 * big_q, v=P16 + 3 * big_q, out=P16 + 4 * big_q)
    assert st == WS_SMALL and str(1 << 20) in msg and str(need + 256) in msg


def test_attn_workspace_checks():
    jag = _jag(B=3, T=1000, max_len=600)
    need = _lib().hstu_attn_workspace_bytes(ctypes.byref(jag), ctypes.byref(_desc()), L.HSTU_BF16)
    assert need >= ((1000 >> 5) + 3 + 1) * 16 and need % 256 == 0
    st, msg = _attn(jag, _desc(), nws=need - 1)
    assert st == WS_SMALL and str(need) in msg
    assert _attn(jag, _desc(), ws=None, nws=need)[0] == INVALID
    assert _attn(jag, _desc(), ws=P16 + 8, nws=need)[0] == INVALID                # misaligned
    assert _attn(jag, _desc(), ws=P16 + 0x10000 + 256, nws=need)[0] == INVALID    # overlaps q


def test_layer_argument_errors():
    lib = _lib()
    jag, desc = _jag(), _desc()

    def call(w, dt=L.HSTU_BF16, x=P16 + 0x100000, y=P16 + 0x200000, ws=P16 + 0x10000000, nws=1 << 40,
             x_dt=L.HSTU_BF16, y_dt=L.HSTU_BF16):
        st = lib.hstu_layer_fwd(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w) if w else None, dt, x_dt, x,
                                y_dt, y, ws, nws, None)
        return st, lib.hstu_last_error().decode()

    good = dict(d_model=512, w_uvqk=P16 + 0x300000, b_uvqk=None, w_out=P16 + 0x400000, b_out=None, ln_eps=1e-6,
                ln_output=0, act_split=0)
    mk = lambda **kw: L.LayerWeightsT(**{**good, **kw})
    assert call(None)[0] == INVALID
    assert call(mk(d_model=12))[0] == UNSUPPORTED
    assert call(mk(ln_eps=0.0))[0] == INVALID
    assert call(mk(w_out=None))[0] == INVALID
    assert call(mk(), x=P16 + 0x100000, y=P16 + 0x100000 + 16)[0] == INVALID   # y overlaps x
    assert call(mk(), dt=L.HSTU_F32, x_dt=L.HSTU_BF16)[0] == UNSUPPORTED        # bf16 x with f32 weights
    assert call(mk(), y_dt=5)[0] == UNSUPPORTED
    need = lib.hstu_layer_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(mk()), L.HSTU_BF16)
    assert need > 0
    st, msg = call(mk(), nws=need - 1)
    assert st == WS_SMALL and str(need) in msg
    need_ln = lib.hstu_layer_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(mk(ln_output=1)),
                                             L.HSTU_BF16)
    assert need_ln > need
    need_split = lib.hstu_layer_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(mk(act_split=1)),
                                                L.HSTU_BF16)
    assert need_split == need                # the gate is formed inside the output GEMM, never stored


def test_gather_argument_errors():
    lib = _lib()

    def call(d=512, dt=L.HSTU_BF16, T=10, rows=100, table=P16, ids=P16 + 0x100000, out=P16 + 0x200000):
        return lib.hstu_gather_rows(table, rows, d, dt, ids, T, out, None)
    assert call(d=12) == UNSUPPORTED          # 24-byte rows
    assert call(T=-1) == INVALID
    assert call(rows=0) == INVALID
    assert call(table=None) == INVALID
    assert call(out=P16 + 8) == INVALID
    assert call(T=0, table=None, ids=None, out=None) == OK
    assert call(out=P16 + 512) == INVALID     # out overlaps table


def test_python_binding_raises_with_message():
    with pytest.raises(L.HstuError) as ei:
        L._check(UNSUPPORTED)
    assert ei.value.name == "HSTU_ERR_UNSUPPORTED"


def _cached(hist, cand, desc, in_dt=L.HSTU_BF16, out_dt=L.HSTU_BF16, kh=P16 + 0x100000, vh=P16 + 0x8000000,
            q=P16 + 0x10000000, k=P16 + 0x20000000, v=P16 + 0x30000000, out=P16 + 0x40000000,
            ws=P16 + 0x80000000, nws=1 << 20):
    lib = _lib()
    st = lib.hstu_attn_fwd_cached(ctypes.byref(hist) if hist else None, ctypes.byref(cand) if cand else None,
                                  ctypes.byref(desc) if desc else None, in_dt, kh, vh, q, k, v, out, out_dt, ws, nws,
                                  None)
    return st, lib.hstu_last_error().decode()


def test_cached_argument_errors():
    hist, cand = _jag(B=2, T=500, max_len=300), _jag(B=2, T=64, max_len=40)
    assert _cached(None, cand, _desc())[0] == INVALID
    assert _cached(hist, None, _desc())[0] == INVALID
    assert _cached(hist, cand, None)[0] == INVALID
    st, msg = _cached(_jag(B=3, T=500, max_len=300), cand, _desc())
    assert st == INVALID and "num_seqs" in msg
    st, msg = _cached(hist, cand, _desc(Dh=96))
    assert st == UNSUPPORTED and "head_dim" in msg
    st, msg = _cached(hist, cand, _desc(), in_dt=L.HSTU_F32, out_dt=L.HSTU_BF16)
    assert st == UNSUPPORTED
    st, msg = _cached(hist, cand, _desc(), nws=16)
    assert st == WS_SMALL
    st, msg = _cached(hist, cand, _desc(), q=P16 + 8)
    assert st == INVALID and "aligned" in msg
    st, msg = _cached(hist, cand, _desc(), out=P16 + 0x10000000)
    assert st == INVALID and "overlaps" in msg
    # the mask field is not read: a candidate mask without num_candidates is fine up to the launch
    st, msg = _cached(hist, cand, _desc(mask=1), nws=16)
    assert st == WS_SMALL


def test_cached_zero_candidates_is_a_no_op():
    hist, cand = _jag(B=2, T=500, max_len=300), _jag(B=2, T=0, max_len=0)
    assert _cached(hist, cand, _desc(), ws=None, nws=0)[0] == OK


def test_cached_workspace_covers_timestamp_ranges_and_partial_sums():
    lib = _lib()
    desc = _desc(H=4, Dh=128)
    cws = lambda h, c: lib.hstu_attn_cached_workspace_bytes(ctypes.byref(h), ctypes.byref(c), ctypes.byref(desc))
    hist, cand = _jag(B=4, T=1000, max_len=300), _jag(B=4, T=64, max_len=40)
    n = cws(hist, cand)
    one = lib.hstu_attn_workspace_bytes(ctypes.byref(cand), ctypes.byref(desc), L.HSTU_BF16)
    assert n > one and n % 256 == 0
    assert n < 64 * 4 * 128 * 4          # short histories: no key split, no partial sums
    # long histories, few candidates: split histories, room for at least two fp32 partial outputs
    long_hist = _jag(B=4, T=40000, max_len=10000)
    assert cws(long_hist, cand) >= n + 2 * 64 * 4 * 128 * 4
    assert cws(_jag(B=3), cand) == 0
    st, msg = _cached(_jag(B=2, T=500, max_len=501), _jag(B=2, T=64, max_len=40), _desc())
    assert st == INVALID and "max_seq_len" in msg


def _bwd(jag, desc, in_dt=L.HSTU_BF16, q=P16 + 0x10000, k=P16 + 0x2000000, v=P16 + 0x4000000, g=P16 + 0x6000000,
         dq=P16 + 0x8000000, dk=P16 + 0xA000000, dv=P16 + 0xC000000, dwp=P16 + 0xE000000, dwt=P16 + 0xE100000,
         ws=P16 + 0x10000000, nws=1 << 24):
    lib = _lib()
    st = lib.hstu_attn_bwd(ctypes.byref(jag) if jag else None, ctypes.byref(desc) if desc else None, in_dt, q, k, v, g,
                           dq, dk, dv, dwp, dwt, ws, nws, None)
    return st, lib.hstu_last_error().decode()


def test_bwd_argument_errors():
    jag, desc = _jag(B=2, T=100, max_len=60), _desc(H=2, Dh=64, P=32, Tb=32)
    assert _bwd(None, desc)[0] == INVALID
    assert _bwd(jag, None)[0] == INVALID
    st, msg = _bwd(jag, _desc(Dh=96))
    assert st == UNSUPPORTED and "head_dim" in msg
    st, msg = _bwd(jag, desc, dwp=None)
    assert st == INVALID and "d_pos_bias" in msg
    st, msg = _bwd(jag, desc, nws=16)
    assert st == WS_SMALL
    st, msg = _bwd(jag, desc, g=None)
    assert st == INVALID and "NULL" in msg
    st, msg = _bwd(jag, desc, dk=P16 + 0x8)
    assert st == INVALID and "aligned" in msg
    st, msg = _bwd(jag, desc, dq=P16 + 0x2000000)          # dq on top of k
    assert st == INVALID and "overlaps" in msg
    st, msg = _bwd(jag, desc, dv=P16 + 0x8000000)          # dv on top of dq
    assert st == INVALID and "overlap" in msg
    st, msg = _bwd(jag, desc, dwt=P16 + 0xE000000)         # the two bias gradients on top of each other
    assert st == INVALID and "overlaps" in msg


def test_bwd_tables_too_large_for_lds_are_unsupported():
    jag = _jag(B=2, T=100, max_len=60)
    st, msg = _bwd(jag, _desc(H=2, Dh=128, P=4096, Tb=64), in_dt=L.HSTU_F32)
    assert st == UNSUPPORTED and "LDS" in msg


def test_bwd_workspace_holds_bins_per_workgroup():
    lib = _lib()
    desc = _desc(H=4, Dh=128, P=256, Tb=256)
    jag = _jag(B=8, T=65536, max_len=8192)
    n = lib.hstu_attn_bwd_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), L.HSTU_BF16)
    workgroups = (8192 // 128) * 4 * 8
    assert n >= workgroups * (256 + 65) * 4 and n % 256 == 0
    assert lib.hstu_attn_bwd_workspace_bytes(ctypes.byref(_jag(B=2, T=0, max_len=0)), ctypes.byref(desc),
                                             L.HSTU_BF16) == 0


def _layer_bwd(jag, desc, w, grads, dt=L.HSTU_BF16, x_dt=L.HSTU_BF16, x=P16 + 0x100000, g_dt=L.HSTU_BF16,
               dy=P16 + 0x200000, dx=P16 + 0x300000, ws=P16 + 0x10000000, nws=1 << 40):
    lib = _lib()
    st = lib.hstu_layer_bwd(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w) if w else None, dt, x_dt, x, g_dt,
                            dy, dx, ctypes.byref(grads) if grads else None, ws, nws, None)
    return st, lib.hstu_last_error().decode()


def test_layer_bwd_argument_errors():
    jag, desc = _jag(B=2, T=100, max_len=60), _desc(H=2, Dh=64, P=32, Tb=32)
    good_w = dict(d_model=256, w_uvqk=P16 + 0x400000, b_uvqk=None, w_out=P16 + 0x500000, b_out=None, ln_eps=1e-6,
                  ln_output=0, act_split=0)
    good_g = dict(d_w_uvqk=P16 + 0x600000, d_b_uvqk=None, d_w_out=P16 + 0x700000, d_b_out=None,
                  d_pos_bias=P16 + 0x800000, d_time_bias=P16 + 0x810000)
    w = lambda **kw: L.LayerWeightsT(**{**good_w, **kw})
    g = lambda **kw: L.LayerGradsT(**{**good_g, **kw})
    assert _layer_bwd(jag, desc, None, g())[0] == INVALID
    st, msg = _layer_bwd(jag, desc, w(), None)
    assert st == INVALID and "grads" in msg
    st, msg = _layer_bwd(jag, desc, w(), g(d_w_out=None))
    assert st == INVALID and "d_w_out" in msg
    assert _layer_bwd(jag, desc, w(), g(d_time_bias=None))[0] == INVALID
    st, msg = _layer_bwd(jag, desc, w(), g(d_w_uvqk=P16 + 0x600008))
    assert st == INVALID and "aligned" in msg
    assert _layer_bwd(jag, desc, w(d_model=20), g())[0] == UNSUPPORTED
    assert _layer_bwd(jag, desc, w(ln_eps=-1.0), g())[0] == INVALID
    assert _layer_bwd(jag, desc, w(), g(), dt=L.HSTU_F32, x_dt=L.HSTU_BF16)[0] == UNSUPPORTED
    assert _layer_bwd(jag, desc, w(), g(), dt=L.HSTU_F32, x_dt=L.HSTU_F32, g_dt=L.HSTU_BF16)[0] == UNSUPPORTED
    st, msg = _layer_bwd(jag, desc, w(), g(), dx=None)
    assert st == INVALID and "NULL" in msg
    st, msg = _layer_bwd(jag, desc, w(), g(), dx=P16 + 0x100000 + 64)             # dx on top of x
    assert st == INVALID and "overlaps" in msg
    st, msg = _layer_bwd(jag, desc, w(), g(d_w_out=P16 + 0x600000 + 256))         # two weight gradients overlap
    assert st == INVALID and "overlap" in msg
    st, msg = _layer_bwd(jag, desc, w(), g(d_pos_bias=P16 + 0x3000))               # gradient on the bias table
    assert st == INVALID and "overlaps" in msg
    st, msg = _layer_bwd(jag, _desc(H=2, Dh=128, P=4096, Tb=64), w(), g(), dt=L.HSTU_F32, x_dt=L.HSTU_F32,
                         g_dt=L.HSTU_F32)
    assert st == UNSUPPORTED and "LDS" in msg


def test_layer_bwd_workspace_sizing():
    lib = _lib()
    desc = _desc(H=2, Dh=64, P=32, Tb=32)
    jag = _jag(B=2, T=100, max_len=60)
    w = L.LayerWeightsT(256, P16, None, P16, None, 1e-6, 0, 0)
    w_ln = L.LayerWeightsT(256, P16, None, P16, None, 1e-6, 1, 0)
    g = L.LayerGradsT(P16 + 0x600000, None, P16 + 0x700000, None, P16 + 0x800000, P16 + 0x810000)
    need = lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), L.HSTU_BF16)
    need_ln = lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w_ln),
                                                 L.HSTU_BF16)
    assert need > 0 and need % 256 == 0
    assert need_ln >= need + 100 * 256 * 4      # the pre-LayerNorm sum r (fp32) is kept only with ln_output
    # every [T, 4*H*Dh] activation is at least there: the projection's pre-activation and its transpose
    assert need >= 2 * 100 * 4 * 128 * 2
    st, msg = _layer_bwd(jag, desc, w, g, nws=need - 1)
    assert st == WS_SMALL and str(need) in msg
    f32 = lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), L.HSTU_F32)
    assert f32 > need


def _stack(jag, descs, ws, L, dt=L.HSTU_BF16, table=P16 + 0x1000000, rows=1000, ids=P16 + 0x5000, y_dt=L.HSTU_BF16,
           y=P16 + 0x8000000, wsp=P16 + 0x10000000, nws=1 << 40):
    lib = _lib()
    st = lib.hstu_stack_fwd(ctypes.byref(jag), descs, ws, L, dt, table, rows, ids, y_dt, y, wsp, nws, None)
    return st, lib.hstu_last_error().decode()


def test_stack_argument_errors():
    jag = _jag(B=2, T=100, max_len=60)
    mkd = lambda n, **kw: (L.AttnDescT * n)(*[_desc(**{**dict(H=2, Dh=64, P=32, Tb=32), **kw}) for _ in range(n)])
    mkw = lambda n, **kw: (L.LayerWeightsT * n)(*[L.LayerWeightsT(**{**dict(
        d_model=256, w_uvqk=P16 + 0x400000, b_uvqk=None, w_out=P16 + 0x500000, b_out=None, ln_eps=1e-6,
        ln_output=0, act_split=0), **kw}) for _ in range(n)])
    assert _stack(jag, mkd(2), mkw(2), 0)[0] == INVALID                      # no layers
    descs = mkd(2)
    descs[1].head_dim = 32
    st, msg = _stack(jag, descs, mkw(2), 2)
    assert st == UNSUPPORTED and "layer 1" in msg
    ws = mkw(2)
    ws[1].d_model = 128
    st, msg = _stack(jag, mkd(2), ws, 2)
    assert st == INVALID and "d_model" in msg
    ws = mkw(2)
    ws[1].w_out = None
    assert _stack(jag, mkd(2), ws, 2)[0] == INVALID
    assert _stack(jag, mkd(2), mkw(2), 2, y_dt=7)[0] == UNSUPPORTED
    st, msg = _stack(jag, mkd(2), mkw(2), 2, ids=None, rows=50)               # identity rows need rows >= T
    assert st == INVALID and "table_rows" in msg
    st, msg = _stack(jag, mkd(2), mkw(2), 2, y=P16 + 0x1000000 + 512)          # y on top of the table
    assert st == INVALID and "overlaps" in msg
    need = _lib().hstu_stack_workspace_bytes(ctypes.byref(jag), mkd(2), mkw(2), 2, L.HSTU_BF16)
    assert need > 0
    st, msg = _stack(jag, mkd(2), mkw(2), 2, nws=need - 1)
    assert st == WS_SMALL and str(need) in msg
    # zero tokens: nothing to do
    assert _stack(_jag(B=2, T=0, max_len=0), mkd(2), mkw(2), 2, table=None, y=None, wsp=None, nws=0)[0] == OK


def test_layer_saved_sizes_and_errors():
    lib = _lib()
    jag, desc = _jag(B=2, T=100, max_len=60), _desc(H=2, Dh=64, P=32, Tb=32)
    w = L.LayerWeightsT(256, P16 + 0x400000, None, P16 + 0x500000, None, 1e-6, 0, 0)
    w_ln = L.LayerWeightsT(256, P16 + 0x400000, None, P16 + 0x500000, None, 1e-6, 1, 0)
    sv = lib.hstu_layer_saved_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), L.HSTU_BF16)
    sv_ln = lib.hstu_layer_saved_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w_ln), L.HSTU_BF16)
    bw = lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), L.HSTU_BF16)
    assert 0 < sv < bw and sv % 256 == 0
    assert sv_ln >= sv + 100 * 256 * 4              # the pre-LayerNorm sum is kept only with the LayerNorm
    assert sv >= 100 * 4 * 128 * 2                   # at least the projection's pre-activation z

    def fwd(saved=P16 + 0x10000000, nsv=1 << 30, y=P16 + 0x200000):
        st = lib.hstu_layer_fwd_save(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), L.HSTU_BF16, L.HSTU_BF16,
                                     P16 + 0x100000, L.HSTU_BF16, y, saved, nsv, None)
        return st, lib.hstu_last_error().decode()
    st, msg = fwd(nsv=sv - 1)
    assert st == WS_SMALL and str(sv) in msg
    assert fwd(saved=None)[0] == INVALID
    st, msg = fwd(saved=P16 + 0x100000 + 64)         # saved on top of x
    assert st == INVALID and "overlaps" in msg

    g = L.LayerGradsT(P16 + 0x600000, None, P16 + 0x700000, None, P16 + 0x800000, P16 + 0x810000)

    def bwd(saved=P16 + 0x10000000, nsv=1 << 30, ws=P16 + 0x40000000, nws=1 << 30):
        st = lib.hstu_layer_bwd_saved(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), L.HSTU_BF16,
                                      L.HSTU_BF16, P16 + 0x100000, L.HSTU_BF16, P16 + 0x200000, P16 + 0x300000,
                                      ctypes.byref(g), saved, nsv, ws, nws, None)
        return st, lib.hstu_last_error().decode()
    assert bwd(saved=None)[0] == INVALID
    st, msg = bwd(nsv=sv - 1)
    assert st == WS_SMALL and "saved" in msg
    st, msg = bwd(nws=bw - sv - 1)
    assert st == WS_SMALL
    st, msg = bwd(saved=P16 + 0x40000000 + 256)      # saved on top of the workspace
    assert st == INVALID and "overlap" in msg


def test_softmax_attn_argument_checks():
    lib = _lib()

    def call(jag, H=4, Dh=128, in_dt=L.HSTU_BF16, out_dt=L.HSTU_BF16, q=P16 + 0x10000, k=P16 + 0x20000000,
             v=P16 + 0x40000000, out=P16 + 0x60000000):
        st = lib.hstu_softmax_attn_fwd(ctypes.byref(jag) if jag else None, H, Dh, in_dt, q, k, v, out, out_dt, None)
        return st, lib.hstu_last_error().decode()
    assert call(None)[0] == INVALID
    assert call(_jag(), Dh=64)[0] == UNSUPPORTED
    assert call(_jag(), in_dt=L.HSTU_F32)[0] == UNSUPPORTED
    assert call(_jag(), H=0)[0] == INVALID
    assert call(_jag(), out_dt=9)[0] == INVALID
    assert call(_jag(), q=None)[0] == INVALID
    st, msg = call(_jag(), out=P16 + 0x10000 + 64)
    assert st == INVALID and "overlaps" in msg
    assert call(L.JaggedT(3, 0, 0, P16, None, None, None), q=None, k=None, v=None, out=None) == (OK, "")


def test_id_errors_rejects_a_null_count_before_touching_the_device():
    lib = _lib()
    assert lib.hstu_id_errors(None, 1, None) == INVALID
    assert "count" in lib.hstu_last_error().decode()
