"""ctypes binding of libhstu (include/hstu.h): argument marshalling only.

Every computation runs in the HIP library; this module turns torch tensors into device
pointers, fills the C structs, allocates the caller-owned workspace and raises on a non-OK
status.  It never falls back to another implementation: if the library is missing, the first
call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libhstu.so")
HEADER_PATH = os.path.join(PKG_DIR, "..", "include", "hstu.h")

HSTU_F32, HSTU_BF16 = 0, 1
MASK_CAUSAL, MASK_CAUSAL_CANDIDATES = 0, 1

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class HstuError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class JaggedT(ctypes.Structure):
    _fields_ = [("num_seqs", c_i32), ("total_tokens", c_i32), ("max_seq_len", c_i32),
                ("seq_offsets", c_vp), ("timestamps", c_vp), ("num_candidates", c_vp), ("attn_scale", c_vp)]


class AttnDescT(ctypes.Structure):
    _fields_ = [("num_heads", c_i32), ("head_dim", c_i32), ("num_pos_buckets", c_i32), ("num_time_buckets", c_i32),
                ("rab_rows", c_i32), ("pos_bias", c_vp), ("time_bias", c_vp), ("mask", c_i32)]


class LayerWeightsT(ctypes.Structure):
    _fields_ = [("d_model", c_i32), ("w_uvqk", c_vp), ("b_uvqk", c_vp), ("w_out", c_vp), ("b_out", c_vp),
                ("ln_eps", c_f32), ("ln_output", c_i32), ("act_split", c_i32)]


class LayerGradsT(ctypes.Structure):
    _fields_ = [("d_w_uvqk", c_vp), ("d_b_uvqk", c_vp), ("d_w_out", c_vp), ("d_b_out", c_vp), ("d_pos_bias", c_vp),
                ("d_time_bias", c_vp)]


_lib = None


def exported_functions_in_header(path: str = HEADER_PATH):
    """Names of the functions that include/hstu.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hstu_[a-z0-9_]+)\s*\(", text)))


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libhstu.so and declare its signatures (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libhstu.so not found at {p}: build it with "
                           "`python -m hstu_sequential_transduction_attn_amd.build`")
    lib = ctypes.CDLL(p)
    lib.hstu_abi_version.restype = ctypes.c_int
    lib.hstu_abi_version.argtypes = []
    lib.hstu_status_string.restype = ctypes.c_char_p
    lib.hstu_status_string.argtypes = [ctypes.c_int]
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_last_error.argtypes = []
    lib.hstu_attn_workspace_bytes.restype = c_sz
    lib.hstu_attn_workspace_bytes.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT), ctypes.c_int]
    lib.hstu_attn_fwd.restype = ctypes.c_int
    lib.hstu_attn_fwd.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT), ctypes.c_int, c_vp, c_vp, c_vp,
                                  c_vp, ctypes.c_int, c_vp, c_sz, c_vp]
    lib.hstu_attn_fwd_noalloc.restype = ctypes.c_int
    lib.hstu_attn_fwd_noalloc.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT), ctypes.c_int, c_vp, c_vp,
                                          c_vp, c_vp, ctypes.c_int, c_vp]
    lib.hstu_softmax_attn_fwd.restype = ctypes.c_int
    lib.hstu_softmax_attn_fwd.argtypes = [ctypes.POINTER(JaggedT), c_i32, c_i32, ctypes.c_int, c_vp, c_vp, c_vp, c_vp,
                                          ctypes.c_int, c_vp]
    lib.hstu_attn_cached_workspace_bytes.restype = c_sz
    lib.hstu_attn_cached_workspace_bytes.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(JaggedT),
                                                     ctypes.POINTER(AttnDescT)]
    lib.hstu_attn_fwd_cached.restype = ctypes.c_int
    lib.hstu_attn_fwd_cached.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT),
                                         ctypes.c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_int, c_vp, c_sz,
                                         c_vp]
    lib.hstu_attn_bwd_workspace_bytes.restype = c_sz
    lib.hstu_attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT), ctypes.c_int]
    lib.hstu_attn_bwd.restype = ctypes.c_int
    lib.hstu_attn_bwd.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT), ctypes.c_int, c_vp, c_vp, c_vp,
                                  c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.hstu_layer_workspace_bytes.restype = c_sz
    lib.hstu_layer_workspace_bytes.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT),
                                               ctypes.POINTER(LayerWeightsT), ctypes.c_int]
    lib.hstu_layer_fwd.restype = ctypes.c_int
    lib.hstu_layer_fwd.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT), ctypes.POINTER(LayerWeightsT),
                                   ctypes.c_int, ctypes.c_int, c_vp, ctypes.c_int, c_vp, c_vp, c_sz, c_vp]
    lib.hstu_layer_bwd_workspace_bytes.restype = c_sz
    lib.hstu_layer_bwd_workspace_bytes.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT),
                                                   ctypes.POINTER(LayerWeightsT), ctypes.c_int]
    lib.hstu_layer_bwd.restype = ctypes.c_int
    lib.hstu_layer_bwd.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT), ctypes.POINTER(LayerWeightsT),
                                   ctypes.c_int, ctypes.c_int, c_vp, ctypes.c_int, c_vp, c_vp,
                                   ctypes.POINTER(LayerGradsT), c_vp, c_sz, c_vp]
    lib.hstu_stack_workspace_bytes.restype = c_sz
    lib.hstu_stack_workspace_bytes.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT),
                                               ctypes.POINTER(LayerWeightsT), c_i32, ctypes.c_int]
    lib.hstu_stack_fwd.restype = ctypes.c_int
    lib.hstu_stack_fwd.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT), ctypes.POINTER(LayerWeightsT),
                                   c_i32, ctypes.c_int, c_vp, c_i64, c_vp, ctypes.c_int, c_vp, c_vp, c_sz, c_vp]
    lib.hstu_layer_saved_bytes.restype = c_sz
    lib.hstu_layer_saved_bytes.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT),
                                           ctypes.POINTER(LayerWeightsT), ctypes.c_int]
    lib.hstu_layer_fwd_save.restype = ctypes.c_int
    lib.hstu_layer_fwd_save.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT),
                                        ctypes.POINTER(LayerWeightsT), ctypes.c_int, ctypes.c_int, c_vp, ctypes.c_int,
                                        c_vp, c_vp, c_sz, c_vp]
    lib.hstu_layer_bwd_saved.restype = ctypes.c_int
    lib.hstu_layer_bwd_saved.argtypes = [ctypes.POINTER(JaggedT), ctypes.POINTER(AttnDescT),
                                         ctypes.POINTER(LayerWeightsT), ctypes.c_int, ctypes.c_int, c_vp, ctypes.c_int,
                                         c_vp, c_vp, ctypes.POINTER(LayerGradsT), c_vp, c_sz, c_vp, c_sz, c_vp]
    lib.hstu_gather_rows.restype = ctypes.c_int
    lib.hstu_gather_rows.argtypes = [c_vp, c_i64, c_i32, ctypes.c_int, c_vp, c_i32, c_vp, c_vp]
    lib.hstu_id_errors.restype = ctypes.c_int
    lib.hstu_id_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32), c_i32, c_vp]
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise HstuError(status, lib.hstu_status_string(status).decode(), lib.hstu_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HSTU_BF16
    if t.dtype == torch.float32:
        return HSTU_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_jagged(seq_offsets: torch.Tensor, timestamps: torch.Tensor, max_seq_len: int,
                num_candidates: Optional[torch.Tensor] = None, attn_scale: Optional[torch.Tensor] = None) -> JaggedT:
    B = seq_offsets.numel() - 1
    return JaggedT(B, timestamps.numel(), int(max_seq_len), _ptr(seq_offsets), _ptr(timestamps),
                   _ptr(num_candidates), _ptr(attn_scale))


def make_desc(num_heads: int, head_dim: int, pos_bias: torch.Tensor, time_bias: torch.Tensor,
              mask: int = MASK_CAUSAL) -> AttnDescT:
    R, P = pos_bias.shape
    Tb = time_bias.shape[1]
    return AttnDescT(num_heads, head_dim, P, Tb, R, _ptr(pos_bias), _ptr(time_bias), int(mask))


def attn_workspace_bytes(seq_offsets, timestamps, q, pos_bias, time_bias, *, max_seq_len: int,
                         mask: int = MASK_CAUSAL) -> int:
    """hstu_attn_workspace_bytes for attn_fwd's arguments (q [T, H, Dh] sets H, Dh and the dtype)."""
    lib = load_library()
    T, H, Dh = q.shape
    jag = make_jagged(seq_offsets, timestamps, max_seq_len)
    desc = make_desc(H, Dh, pos_bias, time_bias, mask)
    return int(lib.hstu_attn_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), _dtype_code(q)))


def attn_fwd(seq_offsets, timestamps, q, k, v, pos_bias, time_bias, *, max_seq_len: int, mask: int = MASK_CAUSAL,
             num_candidates=None, attn_scale=None, out_dtype: Optional[torch.dtype] = None, out=None, workspace=None,
             stream=None):
    """O = hstu_attn_fwd(...): q, k, v [T, H, Dh] (bf16 or f32, contiguous); returns out [T, H, Dh]."""
    lib = load_library()
    T, H, Dh = q.shape
    if out is None:
        out = torch.empty((T, H, Dh), dtype=out_dtype or q.dtype, device=q.device)
    jag = make_jagged(seq_offsets, timestamps, max_seq_len, num_candidates, attn_scale)
    desc = make_desc(H, Dh, pos_bias, time_bias, mask)
    dt = _dtype_code(q)
    nws = int(lib.hstu_attn_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), dt))
    if nws and (workspace is None or workspace.numel() < nws):
        workspace = torch.empty(nws, dtype=torch.uint8, device=q.device)
    _check(lib.hstu_attn_fwd(ctypes.byref(jag), ctypes.byref(desc), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                             _dtype_code(out), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                             _stream(stream)))
    return out


def attn_fwd_noalloc(seq_offsets, timestamps, q, k, v, pos_bias, time_bias, *, max_seq_len: int,
                     mask: int = MASK_CAUSAL, num_candidates=None, attn_scale=None, out=None, out_dtype=None,
                     stream=None):
    """hstu_attn_fwd_noalloc(...): as attn_fwd, with the library's fixed device scratch instead of a
    workspace; pass `out` to make the call allocate nothing on the Python side either."""
    lib = load_library()
    T, H, Dh = q.shape
    if out is None:
        out = torch.empty((T, H, Dh), dtype=out_dtype or q.dtype, device=q.device)
    jag = make_jagged(seq_offsets, timestamps, max_seq_len, num_candidates, attn_scale)
    desc = make_desc(H, Dh, pos_bias, time_bias, mask)
    _check(lib.hstu_attn_fwd_noalloc(ctypes.byref(jag), ctypes.byref(desc), _dtype_code(q), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(out), _dtype_code(out), _stream(stream)))
    return out


def softmax_attn_fwd(seq_offsets, q, k, v, *, max_seq_len: int, out_dtype=None, out=None, stream=None):
    """O = hstu_softmax_attn_fwd(...): causal softmax attention, q, k, v [T, H, 128] bf16."""
    lib = load_library()
    T, H, Dh = q.shape
    if out is None:
        out = torch.empty((T, H, Dh), dtype=out_dtype or q.dtype, device=q.device)
    jag = JaggedT(seq_offsets.numel() - 1, T, int(max_seq_len), _ptr(seq_offsets), None, None, None)
    _check(lib.hstu_softmax_attn_fwd(ctypes.byref(jag), H, Dh, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                     _dtype_code(out), _stream(stream)))
    return out


def attn_bwd(seq_offsets, timestamps, q, k, v, d_out, pos_bias, time_bias, *, max_seq_len: int,
             mask: int = MASK_CAUSAL, num_candidates=None, attn_scale=None, workspace=None, outs=None, stream=None):
    """(dq, dk, dv, d_pos_bias, d_time_bias) = hstu_attn_bwd(...): gradients of attn_fwd's output for
    the upstream gradient d_out [T, H, Dh] (q's dtype); all returned in fp32 (into `outs` when given)."""
    lib = load_library()
    T, H, Dh = q.shape
    f32 = dict(dtype=torch.float32, device=q.device)
    if outs is None:
        dq, dk, dv = (torch.empty((T, H, Dh), **f32) for _ in range(3))
        d_pos, d_time = torch.empty(pos_bias.shape, **f32), torch.empty(time_bias.shape, **f32)
    else:
        dq, dk, dv, d_pos, d_time = outs
    jag = make_jagged(seq_offsets, timestamps, max_seq_len, num_candidates, attn_scale)
    desc = make_desc(H, Dh, pos_bias, time_bias, mask)
    dt = _dtype_code(q)
    nws = int(lib.hstu_attn_bwd_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), dt))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device)
    _check(lib.hstu_attn_bwd(ctypes.byref(jag), ctypes.byref(desc), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(d_out),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(d_pos), _ptr(d_time), _ptr(workspace),
                             workspace.numel(), _stream(stream)))
    return dq, dk, dv, d_pos, d_time


def attn_cached_workspace_bytes(hist_offsets, hist_timestamps, cand_offsets, cand_timestamps, num_heads: int,
                                head_dim: int, pos_bias, time_bias, *, max_candidates: int, max_history: int) -> int:
    lib = load_library()
    hist = make_jagged(hist_offsets, hist_timestamps, max_history)
    cand = make_jagged(cand_offsets, cand_timestamps, max_candidates)
    desc = make_desc(num_heads, head_dim, pos_bias, time_bias)
    return int(lib.hstu_attn_cached_workspace_bytes(ctypes.byref(hist), ctypes.byref(cand), ctypes.byref(desc)))


def attn_fwd_cached(hist_offsets, hist_timestamps, k_hist, v_hist, cand_offsets, cand_timestamps, q, k, v,
                    pos_bias, time_bias, *, max_candidates: int, max_history: int, attn_scale=None,
                    out_dtype: Optional[torch.dtype] = None, out=None, workspace=None, stream=None):
    """O = hstu_attn_fwd_cached(...): candidates q, k, v [T_c, H, Dh] against the cached history
    k_hist, v_hist [T_h, H, Dh]; returns out [T_c, H, Dh]."""
    lib = load_library()
    T, H, Dh = q.shape
    if out is None:
        out = torch.empty((T, H, Dh), dtype=out_dtype or q.dtype, device=q.device)
    hist = make_jagged(hist_offsets, hist_timestamps, max_history)
    cand = make_jagged(cand_offsets, cand_timestamps, max_candidates, None, attn_scale)
    desc = make_desc(H, Dh, pos_bias, time_bias)
    nws = int(lib.hstu_attn_cached_workspace_bytes(ctypes.byref(hist), ctypes.byref(cand), ctypes.byref(desc)))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device)
    _check(lib.hstu_attn_fwd_cached(ctypes.byref(hist), ctypes.byref(cand), ctypes.byref(desc), _dtype_code(q),
                                    _ptr(k_hist), _ptr(v_hist), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                    _dtype_code(out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def layer_workspace_bytes(x, seq_offsets, timestamps, w_uvqk, w_out, pos_bias, time_bias, num_heads, head_dim, *,
                          max_seq_len, ln_output=False, mask=MASK_CAUSAL, act_split=False) -> int:
    lib = load_library()
    jag = make_jagged(seq_offsets, timestamps, max_seq_len)
    desc = make_desc(num_heads, head_dim, pos_bias, time_bias, mask)
    w = LayerWeightsT(x.shape[1], _ptr(w_uvqk), None, _ptr(w_out), None, 1e-6, int(bool(ln_output)),
                      int(bool(act_split)))
    return int(lib.hstu_layer_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w),
                                              _dtype_code(w_uvqk)))


def layer_fwd(x, seq_offsets, timestamps, w_uvqk, w_out, pos_bias, time_bias, num_heads: int, head_dim: int, *,
              max_seq_len: int, b_uvqk=None, b_out=None, ln_eps: float = 1e-6, ln_output: bool = False,
              mask: int = MASK_CAUSAL, num_candidates=None, attn_scale=None, y_dtype: Optional[torch.dtype] = None,
              act_split: bool = False, workspace=None, y=None, saved=None, stream=None):
    """y = hstu_layer_fwd(...): x [T, D] (fp32 or the weights' dtype); returns y [T, D] in y_dtype
    (default: x's dtype).  The weights' dtype (bf16 or f32) sets the MFMA operand type.  With `saved`
    (a uint8 device tensor of layer_saved_bytes), hstu_layer_fwd_save keeps the activations there for
    layer_bwd(..., saved=saved)."""
    lib = load_library()
    T, D = x.shape
    if y is None:
        y = torch.empty((T, D), dtype=y_dtype or x.dtype, device=x.device)
    jag = make_jagged(seq_offsets, timestamps, max_seq_len, num_candidates, attn_scale)
    desc = make_desc(num_heads, head_dim, pos_bias, time_bias, mask)
    w = LayerWeightsT(D, _ptr(w_uvqk), _ptr(b_uvqk), _ptr(w_out), _ptr(b_out), float(ln_eps), int(bool(ln_output)),
                      int(bool(act_split)))
    dt = _dtype_code(w_uvqk)
    if saved is not None:
        _check(lib.hstu_layer_fwd_save(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), dt, _dtype_code(x),
                                       _ptr(x), _dtype_code(y), _ptr(y), _ptr(saved), saved.numel(), _stream(stream)))
        return y
    nws = int(lib.hstu_layer_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), dt))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device)
    _check(lib.hstu_layer_fwd(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), dt, _dtype_code(x), _ptr(x),
                              _dtype_code(y), _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def layer_bwd_workspace_bytes(x, seq_offsets, timestamps, w_uvqk, w_out, pos_bias, time_bias, num_heads, head_dim, *,
                              max_seq_len: int, ln_output: bool = False, mask: int = MASK_CAUSAL,
                              num_candidates=None) -> int:
    lib = load_library()
    jag = make_jagged(seq_offsets, timestamps, max_seq_len, num_candidates, None)
    desc = make_desc(num_heads, head_dim, pos_bias, time_bias, mask)
    w = LayerWeightsT(x.shape[1], _ptr(w_uvqk), None, _ptr(w_out), None, 1e-6, int(bool(ln_output)), 0)
    return int(lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w),
                                                  _dtype_code(w_uvqk)))


def layer_saved_bytes(x, seq_offsets, timestamps, w_uvqk, w_out, pos_bias, time_bias, num_heads, head_dim, *,
                      max_seq_len: int, ln_output: bool = False, mask: int = MASK_CAUSAL, num_candidates=None) -> int:
    lib = load_library()
    jag = make_jagged(seq_offsets, timestamps, max_seq_len, num_candidates, None)
    desc = make_desc(num_heads, head_dim, pos_bias, time_bias, mask)
    w = LayerWeightsT(x.shape[1], _ptr(w_uvqk), None, _ptr(w_out), None, 1e-6, int(bool(ln_output)), 0)
    return int(lib.hstu_layer_saved_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w),
                                          _dtype_code(w_uvqk)))


def layer_bwd(x, dy, seq_offsets, timestamps, w_uvqk, w_out, pos_bias, time_bias, num_heads: int, head_dim: int, *,
              max_seq_len: int, b_uvqk=None, b_out=None, ln_eps: float = 1e-6, ln_output: bool = False,
              mask: int = MASK_CAUSAL, num_candidates=None, attn_scale=None, act_split: bool = False,
              bias_grads: bool = True, workspace=None, dx=None, grads=None, saved=None, stream=None):
    """hstu_layer_bwd(...): gradients of layer_fwd for the upstream gradient dy (dy's dtype is the
    gradient dtype, fp32 or the weights' dtype).  Returns a dict with dx [T, D] (dy's dtype) and fp32
    d_w_uvqk, d_b_uvqk, d_w_out, d_b_out (None unless bias_grads), d_pos_bias, d_time_bias; `grads`
    may supply any of the fp32 gradient tensors to write into."""
    lib = load_library()
    T, D = x.shape
    dev = x.device
    if dx is None:
        dx = torch.empty((T, D), dtype=dy.dtype, device=dev)
    hd = num_heads * head_dim
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dx=dx, d_w_uvqk=torch.empty((4 * hd, D), **f32), d_w_out=torch.empty((D, hd), **f32),
               d_b_uvqk=torch.empty(4 * hd, **f32) if bias_grads else None,
               d_b_out=torch.empty(D, **f32) if bias_grads else None,
               d_pos_bias=torch.empty(pos_bias.shape, **f32), d_time_bias=torch.empty(time_bias.shape, **f32))
    out.update(grads or {})
    jag = make_jagged(seq_offsets, timestamps, max_seq_len, num_candidates, attn_scale)
    desc = make_desc(num_heads, head_dim, pos_bias, time_bias, mask)
    w = LayerWeightsT(D, _ptr(w_uvqk), _ptr(b_uvqk), _ptr(w_out), _ptr(b_out), float(ln_eps), int(bool(ln_output)),
                      int(bool(act_split)))
    grads = LayerGradsT(_ptr(out["d_w_uvqk"]), _ptr(out["d_b_uvqk"]), _ptr(out["d_w_out"]), _ptr(out["d_b_out"]),
                        _ptr(out["d_pos_bias"]), _ptr(out["d_time_bias"]))
    dt = _dtype_code(w_uvqk)
    nws = int(lib.hstu_layer_bwd_workspace_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), dt))
    if saved is not None:   # the saved activations stand in for the workspace's recompute block
        nws -= int(lib.hstu_layer_saved_bytes(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), dt))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    if saved is not None:
        _check(lib.hstu_layer_bwd_saved(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), dt, _dtype_code(x),
                                        _ptr(x), _dtype_code(dy), _ptr(dy), _ptr(dx), ctypes.byref(grads),
                                        _ptr(saved), saved.numel(), _ptr(workspace), workspace.numel(),
                                        _stream(stream)))
        return out
    _check(lib.hstu_layer_bwd(ctypes.byref(jag), ctypes.byref(desc), ctypes.byref(w), dt, _dtype_code(x), _ptr(x),
                              _dtype_code(dy), _ptr(dy), _ptr(dx), ctypes.byref(grads), _ptr(workspace),
                              workspace.numel(), _stream(stream)))
    return out


def _stack_structs(table, seq_offsets, timestamps, layers, num_heads, head_dim, max_seq_len, mask, num_candidates,
                   attn_scale, act_split):
    jag = make_jagged(seq_offsets, timestamps, max_seq_len, num_candidates, attn_scale)
    n = len(layers)
    D = int(table.shape[1])
    descs = (AttnDescT * n)(*[make_desc(num_heads, head_dim, L["pos_bias"], L["time_bias"], mask) for L in layers])
    ws = (LayerWeightsT * n)(*[LayerWeightsT(D, _ptr(L["w_uvqk"]), _ptr(L.get("b_uvqk")), _ptr(L["w_out"]),
                                             _ptr(L.get("b_out")), float(L.get("ln_eps", 1e-6)), 0,
                                             int(bool(act_split))) for L in layers])
    return jag, descs, ws, _dtype_code(layers[0]["w_uvqk"])


def stack_workspace_bytes(table, seq_offsets, timestamps, layers, num_heads: int, head_dim: int, *, max_seq_len: int,
                          mask: int = MASK_CAUSAL, num_candidates=None) -> int:
    jag, descs, ws, dt = _stack_structs(table, seq_offsets, timestamps, layers, num_heads, head_dim, max_seq_len,
                                        mask, num_candidates, None, False)
    return int(load_library().hstu_stack_workspace_bytes(ctypes.byref(jag), descs, ws, len(layers), dt))


def stack_fwd(table, ids, seq_offsets, timestamps, layers, num_heads: int, head_dim: int, *, max_seq_len: int,
              mask: int = MASK_CAUSAL, num_candidates=None, attn_scale=None, act_split: bool = False,
              y_dtype: Optional[torch.dtype] = None, workspace=None, y=None, stream=None):
    """y = hstu_stack_fwd(...): the layers over x_0 = table[ids] (table itself when ids is None).
    layers: list of dicts with w_uvqk, w_out, pos_bias, time_bias and optional b_uvqk, b_out, ln_eps."""
    lib = load_library()
    T = int(timestamps.numel())   # total tokens (the table may hold more rows than that)
    D = int(table.shape[1])
    if y is None:
        y = torch.empty((T, D), dtype=y_dtype or table.dtype, device=table.device)
    jag, descs, ws, dt = _stack_structs(table, seq_offsets, timestamps, layers, num_heads, head_dim, max_seq_len,
                                        mask, num_candidates, attn_scale, act_split)
    n = len(layers)
    nws = int(lib.hstu_stack_workspace_bytes(ctypes.byref(jag), descs, ws, n, dt))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=table.device)
    _check(lib.hstu_stack_fwd(ctypes.byref(jag), descs, ws, n, dt, _ptr(table), int(table.shape[0]), _ptr(ids),
                              _dtype_code(y), _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def gather_rows(table: torch.Tensor, ids: torch.Tensor, out=None, stream=None):
    """out[t] = table[ids[t]] (hstu_gather_rows)."""
    lib = load_library()
    rows, d = table.shape
    T = ids.numel()
    if out is None:
        out = torch.empty((T, d), dtype=table.dtype, device=table.device)
    _check(lib.hstu_gather_rows(_ptr(table), rows, d, _dtype_code(table), _ptr(ids), T, _ptr(out), _stream(stream)))
    return out


def id_errors(reset: bool = True, stream=None) -> int:
    """Out-of-range row ids met by the gathers on the current device since the last reset: 0, or the
    number of clamped reads (hstu_id_errors; waits for the stream)."""
    lib = load_library()
    n = ctypes.c_uint32(0)
    _check(lib.hstu_id_errors(ctypes.byref(n), 1 if reset else 0, _stream(stream)))
    return int(n.value)


def abi_version() -> int:
    return int(load_library().hstu_abi_version())
