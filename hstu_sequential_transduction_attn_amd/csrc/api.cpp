// C-ABI entry points of libhstu: argument validation, workspace layout, kernel dispatch.
// Declarations and the contract of every entry point are in include/hstu.h.
#include "../../include/hstu.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "kernels.h"

static_assert(hstu::kNoallocScratchBytes == HSTU_NOALLOC_SCRATCH_BYTES, "scratch size of the header");

namespace {

thread_local std::string g_last_error;

hstu_status_t fail(hstu_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hstu_status_t ok() {
  g_last_error.clear();
  return HSTU_OK;
}

hstu_status_t from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(HSTU_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

size_t esize(hstu_dtype_t d) { return d == HSTU_BF16 ? 2 : 4; }
bool valid_dtype(hstu_dtype_t d) { return d == HSTU_F32 || d == HSTU_BF16; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

hstu_status_t check_jagged_desc(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc) {
  if (!jag) return fail(HSTU_ERR_INVALID_ARGUMENT, "jag is NULL");
  if (!desc) return fail(HSTU_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (jag->num_seqs < 0) return fail(HSTU_ERR_INVALID_ARGUMENT, "num_seqs = %d < 0", jag->num_seqs);
  if (jag->total_tokens < 0) return fail(HSTU_ERR_INVALID_ARGUMENT, "total_tokens = %d < 0", jag->total_tokens);
  if (jag->max_seq_len < 0 || jag->max_seq_len > jag->total_tokens)
    return fail(HSTU_ERR_INVALID_ARGUMENT, "max_seq_len = %d outside [0, total_tokens = %d]", jag->max_seq_len,
                jag->total_tokens);
  if (jag->num_seqs > 0 && !jag->seq_offsets) return fail(HSTU_ERR_INVALID_ARGUMENT, "seq_offsets is NULL");
  if (jag->num_seqs == 0 && jag->total_tokens != 0)
    return fail(HSTU_ERR_INVALID_ARGUMENT, "num_seqs = 0 but total_tokens = %d", jag->total_tokens);
  if (jag->total_tokens > 0 && !jag->timestamps) return fail(HSTU_ERR_INVALID_ARGUMENT, "timestamps is NULL");
  if (desc->num_heads < 1) return fail(HSTU_ERR_INVALID_ARGUMENT, "num_heads = %d < 1", desc->num_heads);
  if (desc->head_dim != 32 && desc->head_dim != 64 && desc->head_dim != 128)
    return fail(HSTU_ERR_UNSUPPORTED, "head_dim = %d not in {32, 64, 128}", desc->head_dim);
  if (desc->num_pos_buckets < 1 || desc->num_pos_buckets > 4096)
    return fail(HSTU_ERR_INVALID_ARGUMENT, "num_pos_buckets = %d outside [1, 4096]", desc->num_pos_buckets);
  if (desc->num_time_buckets < 1 || desc->num_time_buckets > 4096)
    return fail(HSTU_ERR_INVALID_ARGUMENT, "num_time_buckets = %d outside [1, 4096]", desc->num_time_buckets);
  if (desc->rab_rows != 1 && desc->rab_rows != desc->num_heads)
    return fail(HSTU_ERR_INVALID_ARGUMENT, "rab_rows = %d is neither 1 nor num_heads = %d", desc->rab_rows,
                desc->num_heads);
  if (!desc->pos_bias || !desc->time_bias) return fail(HSTU_ERR_INVALID_ARGUMENT, "pos_bias/time_bias is NULL");
  if (desc->mask != HSTU_MASK_CAUSAL && desc->mask != HSTU_MASK_CAUSAL_CANDIDATES)
    return fail(HSTU_ERR_INVALID_ARGUMENT, "mask = %d is not a hstu_mask_t", (int)desc->mask);
  if (desc->mask == HSTU_MASK_CAUSAL_CANDIDATES && jag->num_seqs > 0 && !jag->num_candidates)
    return fail(HSTU_ERR_INVALID_ARGUMENT, "mask = CAUSAL_CANDIDATES needs num_candidates");
  const long long hd = (long long)desc->num_heads * desc->head_dim;
  if (hd > 4096) return fail(HSTU_ERR_UNSUPPORTED, "num_heads * head_dim = %lld > 4096", hd);
  const long long blocks = ((long long)jag->max_seq_len + 127) / 128 * desc->num_heads * jag->num_seqs;
  if (blocks > 0x7fffffffLL) return fail(HSTU_ERR_UNSUPPORTED, "launch too large (%lld workgroups)", blocks);
  return HSTU_OK;
}

hstu::AttnArgs attn_args(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc) {
  hstu::AttnArgs a{};
  a.seq_offsets = jag->seq_offsets;
  a.timestamps = jag->timestamps;
  a.num_candidates = desc->mask == HSTU_MASK_CAUSAL_CANDIDATES ? jag->num_candidates : nullptr;
  a.attn_scale = jag->attn_scale;
  a.pos_bias = desc->pos_bias;
  a.time_bias = desc->time_bias;
  a.num_seqs = jag->num_seqs;
  a.num_heads = desc->num_heads;
  a.head_dim = desc->head_dim;
  a.max_seq_len = jag->max_seq_len;
  a.num_rows_total = jag->total_tokens;
  a.num_pos_buckets = desc->num_pos_buckets;
  a.num_time_buckets = desc->num_time_buckets;
  a.rab_rows = desc->rab_rows;
  a.mask = desc->mask == HSTU_MASK_CAUSAL_CANDIDATES ? hstu::kCausalCandidates : hstu::kCausal;
  return a;
}

// Layer workspace regions, each 256-byte aligned: U ([T][HD] fp32), V, Q, K ([T][HD] dtype),
// O ([T][HD] fp32), per-(token, head) statistics of O ([T][H][2] fp32), Y32 ([T][D] fp32, only when
// ln_output), timestamp ranges of the attention.
struct LayerWs {
  size_t u, v, q, k, o, ostat, y32, stats, total;
};

LayerWs layer_ws(int64_t T, int64_t B, int64_t H, int64_t HD, int64_t D, hstu_dtype_t dt, bool ln_output) {
  LayerWs w{};
  const size_t part = round_up((size_t)T * HD * esize(dt), 256);
  const size_t part32 = round_up((size_t)T * HD * 4, 256);
  size_t off = 0;
  w.u = off; off += part32;
  w.v = off; off += part;
  w.q = off; off += part;
  w.k = off; off += part;
  w.o = off; off += part32;
  w.ostat = off; off += round_up((size_t)T * H * 8, 256);
  w.y32 = off; off += ln_output ? round_up((size_t)T * D * 4, 256) : 0;
  w.stats = off; off += round_up(hstu::attn_tau_stats_bytes(T, B), 256);
  w.total = off;
  return w;
}

// Everything hstu_attn_fwd and hstu_attn_fwd_noalloc check before a launch, except the scratch.
hstu_status_t check_attn_fwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype,
                             const void *q, const void *k, const void *v, const void *out, hstu_dtype_t out_dtype) {
  hstu_status_t st = check_jagged_desc(jag, desc);
  if (st != HSTU_OK) return st;
  if (!valid_dtype(in_dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "in_dtype = %d invalid", (int)in_dtype);
  if (!valid_dtype(out_dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "out_dtype = %d invalid", (int)out_dtype);
  if (in_dtype == HSTU_F32 && out_dtype != HSTU_F32) return fail(HSTU_ERR_UNSUPPORTED, "f32 inputs need an f32 output");
  const int64_t T = jag->total_tokens;
  if (T == 0) return HSTU_OK;
  if (!q || !k || !v || !out) return fail(HSTU_ERR_INVALID_ARGUMENT, "q/k/v/out is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(HSTU_ERR_INVALID_ARGUMENT, "q/k/v/out must be 16-byte aligned");
  const size_t nin = (size_t)T * desc->num_heads * desc->head_dim * esize(in_dtype);
  const size_t nout = (size_t)T * desc->num_heads * desc->head_dim * esize(out_dtype);
  if (overlaps(out, nout, q, nin) || overlaps(out, nout, k, nin) || overlaps(out, nout, v, nin))
    return fail(HSTU_ERR_INVALID_ARGUMENT, "out overlaps q, k or v");
  return HSTU_OK;
}

// The forward's launch once every argument has been checked; `workspace` holds the timestamp ranges.
hstu_status_t launch_attn_fwd_checked(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype,
                                      const void *q, const void *k, const void *v, void *out, hstu_dtype_t out_dtype,
                                      void *workspace, void *stream) {
  hstu::AttnArgs a = attn_args(jag, desc);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.row_stride = (int64_t)desc->num_heads * desc->head_dim;
  a.out_row_stride = a.row_stride;
  a.in_dtype = in_dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
  a.out_dtype = out_dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
  a.tau_stats = (int64_t *)workspace;
  return from_hip(hstu::launch_attn_fwd(a, (hipStream_t)stream), "attn_fwd launch");
}

}  // namespace

extern "C" {

int hstu_abi_version(void) { return HSTU_ABI_VERSION; }

const char *hstu_status_string(hstu_status_t s) {
  switch (s) {
    case HSTU_OK: return "HSTU_OK";
    case HSTU_ERR_INVALID_ARGUMENT: return "HSTU_ERR_INVALID_ARGUMENT";
    case HSTU_ERR_UNSUPPORTED: return "HSTU_ERR_UNSUPPORTED";
    case HSTU_ERR_WORKSPACE_TOO_SMALL: return "HSTU_ERR_WORKSPACE_TOO_SMALL";
    case HSTU_ERR_DEVICE: return "HSTU_ERR_DEVICE";
  }
  return "HSTU_STATUS_UNKNOWN";
}

const char *hstu_last_error(void) { return g_last_error.c_str(); }

size_t hstu_attn_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype) {
  (void)desc;
  (void)in_dtype;
  if (!jag || jag->total_tokens <= 0 || jag->num_seqs < 0) return 0;
  return round_up(hstu::attn_tau_stats_bytes(jag->total_tokens, jag->num_seqs), 256);
}

hstu_status_t hstu_attn_fwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype,
                            const void *q, const void *k, const void *v, void *out, hstu_dtype_t out_dtype,
                            void *workspace, size_t workspace_bytes, void *stream) {
  try {
    hstu_status_t st = check_attn_fwd(jag, desc, in_dtype, q, k, v, out, out_dtype);
    if (st != HSTU_OK) return st;
    const size_t need = hstu_attn_workspace_bytes(jag, desc, in_dtype);
    if (workspace_bytes < need)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    const int64_t T = jag->total_tokens;
    if (T == 0) return ok();
    if (!workspace) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (!aligned16(workspace)) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    const size_t nin = (size_t)T * desc->num_heads * desc->head_dim * esize(in_dtype);
    const size_t nout = (size_t)T * desc->num_heads * desc->head_dim * esize(out_dtype);
    if (overlaps(workspace, need, out, nout) || overlaps(workspace, need, q, nin) ||
        overlaps(workspace, need, k, nin) || overlaps(workspace, need, v, nin))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace overlaps q, k, v or out");
    return launch_attn_fwd_checked(jag, desc, in_dtype, q, k, v, out, out_dtype, workspace, stream);
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_attn_fwd");
  }
}

hstu_status_t hstu_attn_fwd_noalloc(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype,
                                    const void *q, const void *k, const void *v, void *out, hstu_dtype_t out_dtype,
                                    void *stream) {
  try {
    hstu_status_t st = check_attn_fwd(jag, desc, in_dtype, q, k, v, out, out_dtype);
    if (st != HSTU_OK) return st;
    const size_t need = hstu_attn_workspace_bytes(jag, desc, in_dtype);
    if (need > hstu::kNoallocScratchBytes)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL,
                  "this batch needs %zu bytes of scratch (total_tokens / 32 + num_seqs + 1 timestamp ranges of 16 "
                  "bytes); the fixed device scratch of hstu_attn_fwd_noalloc holds %zu",
                  need, (size_t)hstu::kNoallocScratchBytes);
    if (jag->total_tokens == 0) return ok();
    void *scratch = nullptr;
    const hipError_t e = hstu::noalloc_scratch(&scratch);
    if (e != hipSuccess) return from_hip(e, "device address of the fixed scratch");
    return launch_attn_fwd_checked(jag, desc, in_dtype, q, k, v, out, out_dtype, scratch, stream);
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_attn_fwd_noalloc");
  }
}

hstu_status_t hstu_softmax_attn_fwd(const hstu_jagged_t *jag, int32_t num_heads, int32_t head_dim,
                                    hstu_dtype_t in_dtype, const void *q, const void *k, const void *v, void *out,
                                    hstu_dtype_t out_dtype, void *stream) {
  try {
    if (!jag) return fail(HSTU_ERR_INVALID_ARGUMENT, "jag is NULL");
    if (jag->num_seqs < 0 || jag->total_tokens < 0)
      return fail(HSTU_ERR_INVALID_ARGUMENT, "num_seqs = %d, total_tokens = %d", jag->num_seqs, jag->total_tokens);
    if (jag->max_seq_len < 0 || jag->max_seq_len > jag->total_tokens)
      return fail(HSTU_ERR_INVALID_ARGUMENT, "max_seq_len = %d outside [0, total_tokens = %d]", jag->max_seq_len,
                  jag->total_tokens);
    if (jag->num_seqs > 0 && !jag->seq_offsets) return fail(HSTU_ERR_INVALID_ARGUMENT, "seq_offsets is NULL");
    if (jag->num_seqs == 0 && jag->total_tokens != 0)
      return fail(HSTU_ERR_INVALID_ARGUMENT, "num_seqs = 0 but total_tokens = %d", jag->total_tokens);
    if (num_heads < 1) return fail(HSTU_ERR_INVALID_ARGUMENT, "num_heads = %d < 1", num_heads);
    if (head_dim != 128) return fail(HSTU_ERR_UNSUPPORTED, "head_dim = %d (only 128)", head_dim);
    if (in_dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, "in_dtype must be HSTU_BF16");
    if (!valid_dtype(out_dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "out_dtype = %d invalid", (int)out_dtype);
    const long long blocks = ((long long)jag->max_seq_len + 127) / 128 * num_heads * jag->num_seqs;
    if (blocks > 0x7fffffffLL) return fail(HSTU_ERR_UNSUPPORTED, "launch too large (%lld workgroups)", blocks);
    const int64_t T = jag->total_tokens;
    if (T == 0) return ok();
    if (!q || !k || !v || !out) return fail(HSTU_ERR_INVALID_ARGUMENT, "q/k/v/out is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "q/k/v/out must be 16-byte aligned");
    const size_t nin = (size_t)T * num_heads * head_dim * 2;
    const size_t nout = (size_t)T * num_heads * head_dim * esize(out_dtype);
    if (overlaps(out, nout, q, nin) || overlaps(out, nout, k, nin) || overlaps(out, nout, v, nin))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "out overlaps q, k or v");
    hstu::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.row_stride = (int64_t)num_heads * head_dim;
    a.out_row_stride = a.row_stride;
    a.seq_offsets = jag->seq_offsets;
    a.num_seqs = jag->num_seqs;
    a.num_heads = num_heads;
    a.head_dim = head_dim;
    a.max_seq_len = jag->max_seq_len;
    a.num_rows_total = T;
    a.in_dtype = hstu::kBF16;
    a.out_dtype = out_dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
    return from_hip(hstu::launch_softmax_attn(a, (hipStream_t)stream), "softmax_attn launch");
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_softmax_attn_fwd");
  }
}

namespace {
// Cached-scoring workspace: timestamp ranges of the candidates and of the history, then (with key
// splits) the partial sums [kv_splits][T_c][H][Dh] fp32; each region 256-byte aligned.
struct CachedWs {
  size_t cand_stats, hist_stats, partial, total;
  int splits;
  int32_t tiles_per_split;
};

CachedWs cached_ws(const hstu_jagged_t *hist, const hstu_jagged_t *cand, const hstu_attn_desc_t *desc) {
  CachedWs w{};
  const int64_t Th = hist->total_tokens > 0 ? hist->total_tokens : 0;
  w.splits = hstu::attn_cached_splits(cand->num_seqs, desc->num_heads, cand->max_seq_len,
                                      hist->max_seq_len > 0 ? hist->max_seq_len : 0, &w.tiles_per_split);
  size_t off = 0;
  w.cand_stats = off; off += round_up(hstu::attn_tau_stats_bytes(cand->total_tokens, cand->num_seqs), 256);
  w.hist_stats = off; off += round_up(hstu::attn_tau_stats_bytes(Th, hist->num_seqs), 256);
  w.partial = off;
  if (w.splits > 1) off += round_up((size_t)w.splits * cand->total_tokens * desc->num_heads * desc->head_dim * 4, 256);
  w.total = off;
  return w;
}
}  // namespace

size_t hstu_attn_cached_workspace_bytes(const hstu_jagged_t *hist, const hstu_jagged_t *cand,
                                        const hstu_attn_desc_t *desc) {
  if (!hist || !cand || !desc || hist->num_seqs < 0 || cand->num_seqs != hist->num_seqs) return 0;
  if (cand->total_tokens <= 0 || desc->num_heads < 1 || desc->head_dim < 1) return 0;
  return cached_ws(hist, cand, desc).total;
}

hstu_status_t hstu_attn_fwd_cached(const hstu_jagged_t *hist, const hstu_jagged_t *cand, const hstu_attn_desc_t *desc,
                                   hstu_dtype_t in_dtype, const void *k_hist, const void *v_hist, const void *q,
                                   const void *k, const void *v, void *out, hstu_dtype_t out_dtype, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  try {
    if (!hist) return fail(HSTU_ERR_INVALID_ARGUMENT, "hist is NULL");
    if (!desc) return fail(HSTU_ERR_INVALID_ARGUMENT, "desc is NULL");
    hstu_attn_desc_t d = *desc;   // the mask field is not read: the candidate mask is implied
    d.mask = HSTU_MASK_CAUSAL;
    hstu_status_t st = check_jagged_desc(cand, &d);
    if (st != HSTU_OK) return st;
    if (hist->num_seqs != cand->num_seqs)
      return fail(HSTU_ERR_INVALID_ARGUMENT, "hist->num_seqs = %d != cand->num_seqs = %d", hist->num_seqs,
                  cand->num_seqs);
    if (hist->total_tokens < 0)
      return fail(HSTU_ERR_INVALID_ARGUMENT, "hist->total_tokens = %d < 0", hist->total_tokens);
    if (hist->max_seq_len < 0 || hist->max_seq_len > hist->total_tokens)
      return fail(HSTU_ERR_INVALID_ARGUMENT, "hist->max_seq_len = %d outside [0, hist->total_tokens = %d]",
                  hist->max_seq_len, hist->total_tokens);
    if (!valid_dtype(in_dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "in_dtype = %d invalid", (int)in_dtype);
    if (!valid_dtype(out_dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "out_dtype = %d invalid", (int)out_dtype);
    if (in_dtype == HSTU_F32 && out_dtype != HSTU_F32)
      return fail(HSTU_ERR_UNSUPPORTED, "f32 inputs need an f32 output");
    const CachedWs cw = cached_ws(hist, cand, &d);
    const size_t need = cand->total_tokens > 0 ? cw.total : 0;
    const long long blocks = ((long long)cand->max_seq_len + 127) / 128 * d.num_heads * cand->num_seqs * cw.splits;
    if (blocks > 0x7fffffffLL) return fail(HSTU_ERR_UNSUPPORTED, "launch too large (%lld workgroups)", blocks);
    if (workspace_bytes < need)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    const int64_t Tc = cand->total_tokens, Th = hist->total_tokens;
    if (Tc == 0) return ok();
    if (cand->num_seqs > 0 && !hist->seq_offsets) return fail(HSTU_ERR_INVALID_ARGUMENT, "hist->seq_offsets is NULL");
    if (Th > 0 && !hist->timestamps) return fail(HSTU_ERR_INVALID_ARGUMENT, "hist->timestamps is NULL");
    if (Th > 0 && (!k_hist || !v_hist)) return fail(HSTU_ERR_INVALID_ARGUMENT, "k_hist/v_hist is NULL");
    if (!workspace) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (!aligned16(workspace)) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (!q || !k || !v || !out) return fail(HSTU_ERR_INVALID_ARGUMENT, "q/k/v/out is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(k_hist) ||
        !aligned16(v_hist))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "q/k/v/out/k_hist/v_hist must be 16-byte aligned");
    const size_t hd = (size_t)desc->num_heads * desc->head_dim;
    const size_t nin = (size_t)Tc * hd * esize(in_dtype), nhist = (size_t)Th * hd * esize(in_dtype);
    const size_t nout = (size_t)Tc * hd * esize(out_dtype);
    if (overlaps(out, nout, q, nin) || overlaps(out, nout, k, nin) || overlaps(out, nout, v, nin) ||
        overlaps(out, nout, k_hist, nhist) || overlaps(out, nout, v_hist, nhist))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "out overlaps an input");
    if (overlaps(workspace, need, out, nout) || overlaps(workspace, need, q, nin) ||
        overlaps(workspace, need, k, nin) || overlaps(workspace, need, v, nin) ||
        overlaps(workspace, need, k_hist, nhist) || overlaps(workspace, need, v_hist, nhist))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace overlaps an input or out");
    hstu::AttnArgs a = attn_args(cand, &d);
    a.num_candidates = nullptr;
    a.mask = hstu::kCausalCandidates;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.row_stride = (int64_t)hd;
    a.out_row_stride = a.row_stride;
    a.in_dtype = in_dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
    a.out_dtype = out_dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
    a.tau_stats = (int64_t *)((char *)workspace + cw.cand_stats);
    a.k_hist = k_hist;
    a.v_hist = v_hist;
    a.hist_offsets = hist->seq_offsets;
    a.hist_timestamps = hist->timestamps;
    a.hist_tau_stats = (int64_t *)((char *)workspace + cw.hist_stats);
    a.num_rows = (int32_t)Tc;
    a.num_hist_rows = Th;
    a.kv_splits = cw.splits;
    a.tiles_per_split = cw.tiles_per_split;
    a.partial = cw.splits > 1 ? (float *)((char *)workspace + cw.partial) : nullptr;
    return from_hip(hstu::launch_attn_cached(a, (hipStream_t)stream), "attn_fwd_cached launch");
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_attn_fwd_cached");
  }
}

size_t hstu_attn_bwd_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype) {
  (void)in_dtype;
  if (!jag || !desc || jag->total_tokens <= 0 || jag->num_seqs < 0 || desc->num_heads < 1 ||
      desc->num_pos_buckets < 1)
    return 0;
  return round_up(hstu::attn_tau_stats_bytes(jag->total_tokens, jag->num_seqs), 256) +
         round_up((size_t)hstu::attn_bwd_partial_floats(jag->num_seqs, desc->num_heads, jag->max_seq_len,
                                                        desc->num_pos_buckets) * 4, 256);
}

hstu_status_t hstu_attn_bwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype,
                            const void *q, const void *k, const void *v, const void *d_out, float *dq, float *dk,
                            float *dv, float *d_pos_bias, float *d_time_bias, void *workspace,
                            size_t workspace_bytes, void *stream) {
  try {
    hstu_status_t st = check_jagged_desc(jag, desc);
    if (st != HSTU_OK) return st;
    if (!valid_dtype(in_dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "in_dtype = %d invalid", (int)in_dtype);
    if (!d_pos_bias || !d_time_bias) return fail(HSTU_ERR_INVALID_ARGUMENT, "d_pos_bias/d_time_bias is NULL");
    const int ityp = in_dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
    const size_t lds = std::max(hstu::attn_bwd_dq_lds_bytes(ityp, desc->head_dim, desc->num_pos_buckets),
                                hstu::attn_bwd_dkdv_lds_bytes(ityp, desc->head_dim, desc->num_pos_buckets));
    if (lds > 160 * 1024)
      return fail(HSTU_ERR_UNSUPPORTED, "num_pos_buckets = %d needs %zu bytes of LDS in the backward (160 KB max)",
                  desc->num_pos_buckets, lds);
    const size_t need = hstu_attn_bwd_workspace_bytes(jag, desc, in_dtype);
    if (workspace_bytes < need)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    const int64_t T = jag->total_tokens;
    const size_t R = desc->rab_rows, P = desc->num_pos_buckets, Tb = desc->num_time_buckets;
    if (overlaps(d_pos_bias, R * P * 4, d_time_bias, R * Tb * 4))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "d_pos_bias overlaps d_time_bias");
    if (T > 0) {
      if (!workspace) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace is NULL");
      if (!aligned16(workspace)) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
      if (!q || !k || !v || !d_out || !dq || !dk || !dv)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "q/k/v/d_out/dq/dk/dv is NULL");
      if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_out) || !aligned16(dq) || !aligned16(dk) ||
          !aligned16(dv))
        return fail(HSTU_ERR_INVALID_ARGUMENT, "q/k/v/d_out/dq/dk/dv must be 16-byte aligned");
      const size_t nin = (size_t)T * desc->num_heads * desc->head_dim * esize(in_dtype);
      const size_t ng = (size_t)T * desc->num_heads * desc->head_dim * 4;
      const void *ins[4] = {q, k, v, d_out};
      const void *outs[6] = {dq, dk, dv, d_pos_bias, d_time_bias, workspace};
      const size_t out_n[6] = {ng, ng, ng, R * P * 4, R * Tb * 4, need};
      for (int o = 0; o < 6; ++o) {
        for (int i = 0; i < 4; ++i)
          if (overlaps(outs[o], out_n[o], ins[i], nin))
            return fail(HSTU_ERR_INVALID_ARGUMENT, "an output or the workspace overlaps an input");
        for (int o2 = o + 1; o2 < 6; ++o2)
          if (overlaps(outs[o], out_n[o], outs[o2], out_n[o2]))
            return fail(HSTU_ERR_INVALID_ARGUMENT, "two outputs (or an output and the workspace) overlap");
      }
    }
    hstu::AttnArgs a = attn_args(jag, desc);
    a.q = q;
    a.k = k;
    a.v = v;
    a.d_out = d_out;
    a.out = dq;
    a.dk = dk;
    a.dv = dv;
    a.d_pos_bias = d_pos_bias;
    a.d_time_bias = d_time_bias;
    a.row_stride = (int64_t)desc->num_heads * desc->head_dim;
    a.out_row_stride = a.row_stride;
    a.in_dtype = ityp;
    a.out_dtype = hstu::kF32;
    a.tau_stats = (int64_t *)workspace;
    a.partial = T > 0 ? (float *)((char *)workspace +
                                  round_up(hstu::attn_tau_stats_bytes(T, jag->num_seqs), 256))
                      : nullptr;
    hipError_t e = hstu::launch_attn_bwd_dq(a, (hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e, "attn_bwd dq launch");
    if (T == 0) return ok();
    return from_hip(hstu::launch_attn_bwd_dkdv(a, (hipStream_t)stream), "attn_bwd dk/dv launch");
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_attn_bwd");
  }
}

size_t hstu_layer_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                  const hstu_layer_weights_t *w, hstu_dtype_t dtype) {
  if (!jag || !desc || !w || jag->total_tokens < 0 || desc->num_heads < 1 || desc->head_dim < 1 || w->d_model < 1)
    return 0;
  return layer_ws(jag->total_tokens, jag->num_seqs, desc->num_heads, (int64_t)desc->num_heads * desc->head_dim,
                  w->d_model, dtype, w->ln_output != 0)
      .total;
}

hstu_status_t hstu_layer_fwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, const hstu_layer_weights_t *w,
                             hstu_dtype_t dtype, hstu_dtype_t x_dtype, const void *x, hstu_dtype_t y_dtype, void *y,
                             void *workspace, size_t workspace_bytes, void *stream) {
  try {
    hstu_status_t st = check_jagged_desc(jag, desc);
    if (st != HSTU_OK) return st;
    if (!w) return fail(HSTU_ERR_INVALID_ARGUMENT, "weights is NULL");
    if (!valid_dtype(dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "dtype = %d invalid", (int)dtype);
    if (!valid_dtype(x_dtype) || (x_dtype != dtype && x_dtype != HSTU_F32))
      return fail(HSTU_ERR_UNSUPPORTED, "x_dtype = %d must be HSTU_F32 or dtype", (int)x_dtype);
    if (!valid_dtype(y_dtype) || (y_dtype != dtype && y_dtype != HSTU_F32))
      return fail(HSTU_ERR_UNSUPPORTED, "y_dtype = %d must be HSTU_F32 or dtype", (int)y_dtype);
    const int64_t T = jag->total_tokens;
    const int64_t D = w->d_model;
    const int64_t HD = (int64_t)desc->num_heads * desc->head_dim;
    if (D < 1 || D % 8 != 0 || D > 4096)
      return fail(HSTU_ERR_UNSUPPORTED, "d_model = %lld must be a multiple of 8 in [8, 4096]", (long long)D);
    if (!(w->ln_eps > 0.0f)) return fail(HSTU_ERR_INVALID_ARGUMENT, "ln_eps must be > 0");
    if (!w->w_uvqk || !w->w_out) return fail(HSTU_ERR_INVALID_ARGUMENT, "w_uvqk/w_out is NULL");
    if (!aligned16(w->w_uvqk) || !aligned16(w->w_out))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "weights must be 16-byte aligned");
    const bool split = dtype == HSTU_BF16 && w->act_split != 0;
    const LayerWs ws = layer_ws(T, jag->num_seqs, desc->num_heads, HD, D, dtype, w->ln_output != 0);
    if (workspace_bytes < ws.total)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, ws.total);
    if (T == 0) return ok();
    if (!x || !y) return fail(HSTU_ERR_INVALID_ARGUMENT, "x/y is NULL");
    if (!workspace) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (!aligned16(x) || !aligned16(y) || !aligned16(workspace))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "x/y/workspace must be 16-byte aligned");
    const size_t nx = (size_t)T * D * esize(x_dtype), ny = (size_t)T * D * esize(y_dtype);
    if (overlaps(x, nx, y, ny)) return fail(HSTU_ERR_INVALID_ARGUMENT, "y overlaps x");
    if (overlaps(workspace, ws.total, x, nx) || overlaps(workspace, ws.total, y, ny))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace overlaps x or y");

    hipStream_t s = (hipStream_t)stream;
    char *wsb = (char *)workspace;
    const int dt = dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
    const int x_f32 = x_dtype == HSTU_F32, y_f32 = y_dtype == HSTU_F32;

    hstu::GemmUvqkArgs g1{};
    g1.x = x; g1.w = w->w_uvqk; g1.bias = w->b_uvqk;
    g1.u = (float *)(wsb + ws.u); g1.v = wsb + ws.v; g1.q = wsb + ws.q; g1.k = wsb + ws.k;
    g1.M = (int32_t)T; g1.K = (int32_t)D; g1.HD = (int32_t)HD;
    g1.dtype = dt; g1.x_f32 = x_f32; g1.split = split;
    hipError_t e = hstu::launch_gemm_uvqk(g1, s);
    if (e != hipSuccess) return from_hip(e, "projection GEMM launch");

    hstu::AttnArgs a = attn_args(jag, desc);
    a.q = wsb + ws.q; a.k = wsb + ws.k; a.v = wsb + ws.v; a.out = wsb + ws.o;
    a.row_stride = HD; a.out_row_stride = HD;
    a.in_dtype = dt; a.out_dtype = hstu::kF32;
    a.tau_stats = (int64_t *)(wsb + ws.stats);
    a.row_stats = (float *)(wsb + ws.ostat);
    e = hstu::launch_attn_fwd(a, s);
    if (e != hipSuccess) return from_hip(e, "attention launch");

    hstu::GemmOutArgs g2{};
    g2.o = (const float *)(wsb + ws.o); g2.u = (const float *)(wsb + ws.u);
    g2.row_stats = (const float *)(wsb + ws.ostat);
    g2.heads = desc->num_heads; g2.head_dim = desc->head_dim; g2.eps = w->ln_eps;
    g2.w = w->w_out; g2.bias = w->b_out; g2.x = x;
    g2.y = y; g2.y32 = w->ln_output ? (float *)(wsb + ws.y32) : nullptr;
    g2.M = (int32_t)T; g2.N = (int32_t)D; g2.K = (int32_t)HD;
    g2.dtype = dt; g2.split = split; g2.x_f32 = x_f32; g2.y_f32 = y_f32;
    e = hstu::launch_gemm_out(g2, s);
    if (e != hipSuccess) return from_hip(e, "output GEMM launch");

    if (w->ln_output) {
      hstu::RowLnArgs ln{};
      ln.in = (const float *)(wsb + ws.y32); ln.out = y; ln.M = (int32_t)T; ln.N = (int32_t)D;
      ln.eps = w->ln_eps; ln.out_f32 = y_f32;
      e = hstu::launch_row_layernorm(ln, s);
      if (e != hipSuccess) return from_hip(e, "output LayerNorm launch");
    }
    return ok();
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_layer_fwd");
  }
}

namespace {

// The forward activations the layer backward needs (256-byte aligned regions): U (fp32), V, Q, K
// (dtype), Z = the projection's pre-activation (dtype; overwritten by dz), O (fp32) and its per-head
// statistics, the timestamp ranges, the pre-LayerNorm sum r (fp32, ln_output only; overwritten by dr).
// hstu_layer_fwd_save leaves them in the caller's saved buffer; hstu_layer_bwd recomputes them at the
// start of its workspace.
struct LayerSaved {
  size_t u, v, q, k, z, o, ostat, stats, r32, total;
};

LayerSaved layer_saved(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, int64_t D, hstu_dtype_t dt,
                       bool ln_output) {
  LayerSaved w{};
  const int64_t T = jag->total_tokens, B = jag->num_seqs, H = desc->num_heads;
  const int64_t HD = H * desc->head_dim;
  const size_t es = esize(dt);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes, 256);
    return at;
  };
  w.u = take((size_t)T * HD * 4);
  w.v = take((size_t)T * HD * es);
  w.q = take((size_t)T * HD * es);
  w.k = take((size_t)T * HD * es);
  w.z = take((size_t)T * 4 * HD * es);
  w.o = take((size_t)T * HD * 4);
  w.ostat = take((size_t)T * H * 8);
  w.stats = take(hstu::attn_tau_stats_bytes(T, B));
  w.r32 = take(ln_output ? (size_t)T * D * 4 : 0);
  w.total = off;
  return w;
}

// Layer-backward workspace regions (256-byte aligned): without saved activations, first the
// LayerSaved block; then W1^T, W2^T (dtype), dg (fp32), g and dO (dtype), the attention backward's
// bias-gradient bins, the token-contiguous transposes x^T, dr^T, g^T, dz^T
// (dtype, T padded to Tp, a multiple of 32) and the split-K partial products of the weight gradients.
struct LayerBwdWs {
  size_t fwd, w1t, w2t, dg, g, d_o, bins, xt, drt, gt, dzt, part, bsum, total;
  int64_t Tp;
  int split_w1, split_w2;
};

LayerBwdWs layer_bwd_ws(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, int64_t D, hstu_dtype_t dt,
                        bool ln_output, bool with_saved = false) {
  LayerBwdWs w{};
  const int64_t T = jag->total_tokens, B = jag->num_seqs, H = desc->num_heads;
  const int64_t HD = H * desc->head_dim;
  const size_t es = esize(dt);
  const int dtc = dt == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
  w.Tp = (T + 31) / 32 * 32;
  w.split_w1 = hstu::gemm_plain_splits(4 * HD, D, w.Tp, dtc, 0);
  w.split_w2 = hstu::gemm_plain_splits(D, HD, w.Tp, dtc, 0);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes, 256);
    return at;
  };
  w.fwd = take(with_saved ? 0 : layer_saved(jag, desc, D, dt, ln_output).total);
  w.w1t = take((size_t)4 * HD * D * es);
  w.w2t = take((size_t)HD * D * es);
  w.dg = take((size_t)T * HD * 4);
  w.g = take((size_t)T * HD * es);
  w.d_o = take((size_t)T * HD * es);
  w.bins = take((size_t)hstu::attn_bwd_partial_floats(B, H, jag->max_seq_len, desc->num_pos_buckets) * 4);
  w.xt = take((size_t)D * w.Tp * es);
  w.drt = take((size_t)D * w.Tp * es);
  w.gt = take((size_t)HD * w.Tp * es);
  w.dzt = take((size_t)4 * HD * w.Tp * es);
  const size_t p1 = w.split_w1 > 1 ? (size_t)w.split_w1 * 4 * HD * D : 0;
  const size_t p2 = w.split_w2 > 1 ? (size_t)w.split_w2 * D * HD : 0;
  w.part = take((p1 > p2 ? p1 : p2) * 4);
  w.bsum = take((size_t)(4 * HD + D) * hstu::transpose_colsum_ld((int)w.Tp) * 4);   // bias-sum tile partials
  w.total = off;
  return w;
}

}  // namespace

size_t hstu_layer_bwd_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                      const hstu_layer_weights_t *w, hstu_dtype_t dtype) {
  if (!jag || !desc || !w || jag->total_tokens < 0 || jag->num_seqs < 0 || desc->num_heads < 1 ||
      desc->head_dim < 1 || desc->num_pos_buckets < 1 || w->d_model < 1 || !valid_dtype(dtype))
    return 0;
  return layer_bwd_ws(jag, desc, w->d_model, dtype, w->ln_output != 0).total;
}

namespace {

// The layer forward into the LayerSaved block at fb: the projection (also storing z), the attention,
// and the output projection where it is needed: into r (fp32) when the output LayerNorm follows, then
// y = LN(r) if y is given; otherwise straight into y if y is given.
hstu_status_t run_layer_forward(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, const hstu_layer_weights_t *w,
                                hstu_dtype_t dtype, hstu_dtype_t x_dtype, const void *x, char *fb, const LayerSaved &sv,
                                void *y, hstu_dtype_t y_dtype, hipStream_t s) {
  const int64_t T = jag->total_tokens, D = w->d_model, H = desc->num_heads, HD = H * desc->head_dim;
  const int dt = dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
  const int x_f32 = x_dtype == HSTU_F32;
  const bool split = dtype == HSTU_BF16 && w->act_split != 0;
  const bool ln_out = w->ln_output != 0;
  hstu::GemmUvqkArgs g1{};
  g1.x = x; g1.w = w->w_uvqk; g1.bias = w->b_uvqk;
  g1.u = (float *)(fb + sv.u); g1.v = fb + sv.v; g1.q = fb + sv.q; g1.k = fb + sv.k; g1.z = fb + sv.z;
  g1.M = (int32_t)T; g1.K = (int32_t)D; g1.HD = (int32_t)HD;
  g1.dtype = dt; g1.x_f32 = x_f32; g1.split = split;
  hipError_t e = hstu::launch_gemm_uvqk(g1, s);
  if (e != hipSuccess) return from_hip(e, "projection GEMM launch");
  hstu::AttnArgs a = attn_args(jag, desc);
  a.q = fb + sv.q; a.k = fb + sv.k; a.v = fb + sv.v; a.out = fb + sv.o;
  a.row_stride = HD; a.out_row_stride = HD;
  a.in_dtype = dt; a.out_dtype = hstu::kF32;
  a.tau_stats = (int64_t *)(fb + sv.stats);
  a.row_stats = (float *)(fb + sv.ostat);
  e = hstu::launch_attn_fwd(a, s);
  if (e != hipSuccess) return from_hip(e, "attention launch");
  if (!ln_out && !y) return HSTU_OK;
  hstu::GemmOutArgs g2{};
  g2.o = (const float *)(fb + sv.o); g2.u = (const float *)(fb + sv.u);
  g2.row_stats = (const float *)(fb + sv.ostat);
  g2.heads = (int32_t)H; g2.head_dim = desc->head_dim; g2.eps = w->ln_eps;
  g2.w = w->w_out; g2.bias = w->b_out; g2.x = x;
  g2.y = y; g2.y32 = ln_out ? (float *)(fb + sv.r32) : nullptr;
  g2.M = (int32_t)T; g2.N = (int32_t)D; g2.K = (int32_t)HD;
  g2.dtype = dt; g2.split = split; g2.x_f32 = x_f32; g2.y_f32 = y_dtype == HSTU_F32;
  e = hstu::launch_gemm_out(g2, s);
  if (e != hipSuccess) return from_hip(e, "output GEMM launch");
  if (ln_out && y) {
    hstu::RowLnArgs ln{};
    ln.in = (const float *)(fb + sv.r32); ln.out = y; ln.M = (int32_t)T; ln.N = (int32_t)D;
    ln.eps = w->ln_eps; ln.out_f32 = y_dtype == HSTU_F32;
    e = hstu::launch_row_layernorm(ln, s);
    if (e != hipSuccess) return from_hip(e, "output LayerNorm launch");
  }
  return HSTU_OK;
}

// The layer backward; saved: the activations of a hstu_layer_fwd_save call (consumed), or NULL to
// recompute them in the workspace.
hstu_status_t layer_bwd_impl(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, const hstu_layer_weights_t *w,
                             hstu_dtype_t dtype, hstu_dtype_t x_dtype, const void *x, hstu_dtype_t grad_dtype,
                             const void *dy, void *dx, const hstu_layer_grads_t *grads, void *saved,
                             size_t saved_bytes, void *workspace, size_t workspace_bytes, void *stream) {
  try {
    hstu_status_t st = check_jagged_desc(jag, desc);
    if (st != HSTU_OK) return st;
    if (!w) return fail(HSTU_ERR_INVALID_ARGUMENT, "weights is NULL");
    if (!grads) return fail(HSTU_ERR_INVALID_ARGUMENT, "grads is NULL");
    if (!valid_dtype(dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "dtype = %d invalid", (int)dtype);
    if (!valid_dtype(x_dtype) || (x_dtype != dtype && x_dtype != HSTU_F32))
      return fail(HSTU_ERR_UNSUPPORTED, "x_dtype = %d must be HSTU_F32 or dtype", (int)x_dtype);
    if (!valid_dtype(grad_dtype) || (grad_dtype != dtype && grad_dtype != HSTU_F32))
      return fail(HSTU_ERR_UNSUPPORTED, "grad_dtype = %d must be HSTU_F32 or dtype", (int)grad_dtype);
    const int64_t T = jag->total_tokens;
    const int64_t D = w->d_model;
    const int64_t H = desc->num_heads, HD = H * desc->head_dim;
    if (D < 1 || D % 8 != 0 || D > 4096)
      return fail(HSTU_ERR_UNSUPPORTED, "d_model = %lld must be a multiple of 8 in [8, 4096]", (long long)D);
    if (!(w->ln_eps > 0.0f)) return fail(HSTU_ERR_INVALID_ARGUMENT, "ln_eps must be > 0");
    if (!w->w_uvqk || !w->w_out) return fail(HSTU_ERR_INVALID_ARGUMENT, "w_uvqk/w_out is NULL");
    if (!aligned16(w->w_uvqk) || !aligned16(w->w_out))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "weights must be 16-byte aligned");
    if (!grads->d_w_uvqk || !grads->d_w_out || !grads->d_pos_bias || !grads->d_time_bias)
      return fail(HSTU_ERR_INVALID_ARGUMENT, "d_w_uvqk/d_w_out/d_pos_bias/d_time_bias is NULL");
    if (!aligned16(grads->d_w_uvqk) || !aligned16(grads->d_w_out))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "d_w_uvqk/d_w_out must be 16-byte aligned");
    const int ityp = dtype == HSTU_BF16 ? hstu::kBF16 : hstu::kF32;
    const size_t lds = std::max(hstu::attn_bwd_dq_lds_bytes(ityp, desc->head_dim, desc->num_pos_buckets),
                                hstu::attn_bwd_dkdv_lds_bytes(ityp, desc->head_dim, desc->num_pos_buckets));
    if (lds > 160 * 1024)
      return fail(HSTU_ERR_UNSUPPORTED, "num_pos_buckets = %d needs %zu bytes of LDS in the backward (160 KB max)",
                  desc->num_pos_buckets, lds);
    const bool ln_out = w->ln_output != 0;
    const LayerSaved sv = layer_saved(jag, desc, D, dtype, ln_out);
    const LayerBwdWs ws = layer_bwd_ws(jag, desc, D, dtype, ln_out, saved != nullptr);
    if (workspace_bytes < ws.total)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, ws.total);
    if (saved && saved_bytes < sv.total)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL, "saved %zu < %zu bytes", saved_bytes, sv.total);
    if (saved && !aligned16(saved)) return fail(HSTU_ERR_INVALID_ARGUMENT, "saved must be 16-byte aligned");
    if (!workspace) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (!aligned16(workspace)) return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (T > 0) {
      if (!x || !dy || !dx) return fail(HSTU_ERR_INVALID_ARGUMENT, "x/dy/dx is NULL");
      if (!aligned16(x) || !aligned16(dy) || !aligned16(dx))
        return fail(HSTU_ERR_INVALID_ARGUMENT, "x/dy/dx must be 16-byte aligned");
    }
    const size_t R = desc->rab_rows, P = desc->num_pos_buckets, Tb = desc->num_time_buckets, es = esize(dtype);
    const size_t nx = (size_t)T * D * esize(x_dtype), ng = (size_t)T * D * esize(grad_dtype);
    const void *ins[8] = {x, dy, w->w_uvqk, w->b_uvqk, w->w_out, w->b_out, desc->pos_bias, desc->time_bias};
    const size_t in_n[8] = {nx, ng, (size_t)4 * HD * D * es, (size_t)4 * HD * es, (size_t)D * HD * es, (size_t)D * es,
                            R * P * 4, R * Tb * 4};
    const void *outs[9] = {dx, grads->d_w_uvqk, grads->d_b_uvqk, grads->d_w_out, grads->d_b_out, grads->d_pos_bias,
                           grads->d_time_bias, workspace, saved};
    const size_t out_n[9] = {ng, (size_t)4 * HD * D * 4, (size_t)4 * HD * 4, (size_t)D * HD * 4, (size_t)D * 4,
                             R * P * 4, R * Tb * 4, ws.total, saved ? sv.total : 0};
    for (int o = 0; o < 9; ++o) {
      for (int i = 0; i < 8; ++i)
        if (overlaps(outs[o], out_n[o], ins[i], in_n[i]))
          return fail(HSTU_ERR_INVALID_ARGUMENT, "an output, the workspace or the saved activations overlaps an input");
      for (int o2 = o + 1; o2 < 9; ++o2)
        if (overlaps(outs[o], out_n[o], outs[o2], out_n[o2]))
          return fail(HSTU_ERR_INVALID_ARGUMENT, "two outputs (or an output and the workspace) overlap");
    }

    hipStream_t s = (hipStream_t)stream;
    char *wsb = (char *)workspace;
    const int dt = ityp, f32w = dtype == HSTU_F32;
    const int x_f32 = x_dtype == HSTU_F32, g_f32 = grad_dtype == HSTU_F32;
    hipError_t e;
#define HSTU_TRY(call, what)                 \
  do {                                       \
    e = (call);                              \
    if (e != hipSuccess) return from_hip(e, what); \
  } while (0)

    char *fb = saved ? (char *)saved : wsb + ws.fwd;   // the forward activations
    hstu::AttnArgs a = attn_args(jag, desc);
    a.row_stride = HD; a.out_row_stride = HD;
    a.in_dtype = dt;
    a.out_dtype = hstu::kF32;
    a.tau_stats = (int64_t *)(fb + sv.stats);
    if (T == 0) {
      // no tokens: every gradient is 0 (the attention backward clears its two tables itself)
      HSTU_TRY(hstu::launch_fill_zero(grads->d_w_uvqk, 4 * HD * D, s), "zero fill");
      HSTU_TRY(hstu::launch_fill_zero(grads->d_b_uvqk, grads->d_b_uvqk ? 4 * HD : 0, s), "zero fill");
      HSTU_TRY(hstu::launch_fill_zero(grads->d_w_out, D * HD, s), "zero fill");
      HSTU_TRY(hstu::launch_fill_zero(grads->d_b_out, grads->d_b_out ? D : 0, s), "zero fill");
      a.d_pos_bias = grads->d_pos_bias; a.d_time_bias = grads->d_time_bias;
      HSTU_TRY(hstu::launch_attn_bwd_dq(a, s), "attention backward launch");
      return ok();
    }

    HSTU_TRY(hstu::launch_transpose(w->w_uvqk, f32w, wsb + ws.w1t, f32w, (int)(4 * HD), (int)D, (int)(4 * HD), s),
             "W1 transpose");
    HSTU_TRY(hstu::launch_transpose(w->w_out, f32w, wsb + ws.w2t, f32w, (int)D, (int)HD, (int)D, s), "W2 transpose");
    if (!saved) {
      // ---- recompute the forward (z, U, V, Q, K, O and, with the output LayerNorm, r)
      hstu_status_t r = run_layer_forward(jag, desc, w, dtype, x_dtype, x, fb, sv, nullptr, HSTU_F32, s);
      if (r != HSTU_OK) return r;
    }

    // ---- dr
    const void *dr = dy;
    int dr_f32 = g_f32;
    if (ln_out) {
      hstu::LnBwdArgs lb{};
      lb.r = (float *)(fb + sv.r32); lb.dy = dy; lb.M = (int32_t)T; lb.N = (int32_t)D; lb.dy_f32 = g_f32;
      lb.eps = w->ln_eps;
      HSTU_TRY(hstu::launch_ln_bwd_rows(lb, s), "LayerNorm backward launch");
      dr = fb + sv.r32;
      dr_f32 = 1;
    }

    // ---- dg = dr W2, then the norm-gate backward (g, dO, dz_U)
    hstu::GemmPlainArgs pg{};
    pg.a = dr; pg.a_f32 = dr_f32; pg.b = wsb + ws.w2t; pg.c = wsb + ws.dg; pg.c_f32 = 1;
    pg.M = (int32_t)T; pg.N = (int32_t)HD; pg.K = (int32_t)D; pg.dtype = dt; pg.splits = 1;
    HSTU_TRY(hstu::launch_gemm_plain(pg, s), "dg GEMM launch");
    hstu::NormGateBwdArgs nb{};
    nb.o = (const float *)(fb + sv.o); nb.u = (const float *)(fb + sv.u); nb.dg = (const float *)(wsb + ws.dg);
    nb.z = fb + sv.z; nb.g = wsb + ws.g; nb.d_o = wsb + ws.d_o;
    nb.M = (int32_t)T; nb.N = (int32_t)HD; nb.dtype = dt; nb.eps = w->ln_eps;
    HSTU_TRY(hstu::launch_norm_gate_bwd(nb, s), "norm-gate backward launch");

    // ---- attention backward, whose epilogues turn dV, dQ, dK into the rest of dz in place over z
    a.q = fb + sv.q; a.k = fb + sv.k; a.v = fb + sv.v;
    a.d_out = wsb + ws.d_o;
    a.out = nullptr; a.dk = nullptr; a.dv = nullptr;
    char *zb = fb + sv.z;
    a.z_v = zb + (size_t)HD * es; a.z_q = zb + (size_t)2 * HD * es; a.z_k = zb + (size_t)3 * HD * es;
    a.z_row_stride = 4 * HD;
    a.d_pos_bias = grads->d_pos_bias; a.d_time_bias = grads->d_time_bias;
    a.partial = (float *)(wsb + ws.bins);
    a.row_stats = nullptr;
    HSTU_TRY(hstu::launch_attn_bwd_dq(a, s), "attention backward dq launch");
    HSTU_TRY(hstu::launch_attn_bwd_dkdv(a, s), "attention backward dk/dv launch");

    // ---- dx = dr + dz W1
    hstu::GemmPlainArgs px{};
    px.a = fb + sv.z; px.a_f32 = f32w; px.b = wsb + ws.w1t; px.resid = dr; px.resid_f32 = dr_f32;
    px.c = dx; px.c_f32 = g_f32;
    px.M = (int32_t)T; px.N = (int32_t)D; px.K = (int32_t)(4 * HD); px.dtype = dt; px.splits = 1;
    HSTU_TRY(hstu::launch_gemm_plain(px, s), "dx GEMM launch");

    // ---- weight and bias gradients from token-contiguous transposes
    const int Tp = (int)ws.Tp;
    HSTU_TRY(hstu::launch_transpose(x, x_f32, wsb + ws.xt, f32w, (int)T, (int)D, Tp, s), "x transpose");
    // the bias gradients (column sums of dz and dr over the tokens) come from the same tiles
    const int ldp = hstu::transpose_colsum_ld(Tp);
    float *bsum = (float *)(wsb + ws.bsum);
    float *bsum_out = bsum + (size_t)4 * HD * ldp;
    HSTU_TRY(hstu::launch_transpose(dr, dr_f32, wsb + ws.drt, f32w, (int)T, (int)D, Tp, s,
                                    grads->d_b_out ? bsum_out : nullptr), "dr transpose");
    HSTU_TRY(hstu::launch_transpose(wsb + ws.g, f32w, wsb + ws.gt, f32w, (int)T, (int)HD, Tp, s), "g transpose");
    HSTU_TRY(hstu::launch_transpose(fb + sv.z, f32w, wsb + ws.dzt, f32w, (int)T, (int)(4 * HD), Tp, s,
                                    grads->d_b_uvqk ? bsum : nullptr), "dz transpose");
    hstu::GemmPlainArgs pw{};
    pw.a = wsb + ws.dzt; pw.a_f32 = f32w; pw.b = wsb + ws.xt; pw.c = grads->d_w_uvqk; pw.c_f32 = 1;
    pw.M = (int32_t)(4 * HD); pw.N = (int32_t)D; pw.K = Tp; pw.dtype = dt;
    pw.splits = ws.split_w1; pw.partial = (float *)(wsb + ws.part);
    HSTU_TRY(hstu::launch_gemm_plain(pw, s), "d_w_uvqk GEMM launch");
    pw.a = wsb + ws.drt; pw.b = wsb + ws.gt; pw.c = grads->d_w_out;
    pw.M = (int32_t)D; pw.N = (int32_t)HD; pw.splits = ws.split_w2;
    HSTU_TRY(hstu::launch_gemm_plain(pw, s), "d_w_out GEMM launch");
    if (grads->d_b_uvqk)
      HSTU_TRY(hstu::launch_row_sum(bsum, 1, grads->d_b_uvqk, (int)(4 * HD), ldp, s), "d_b_uvqk launch");
    if (grads->d_b_out)
      HSTU_TRY(hstu::launch_row_sum(bsum_out, 1, grads->d_b_out, (int)D, ldp, s), "d_b_out launch");
#undef HSTU_TRY
    return ok();
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in the layer backward");
  }
}

}  // namespace

hstu_status_t hstu_layer_bwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, const hstu_layer_weights_t *w,
                             hstu_dtype_t dtype, hstu_dtype_t x_dtype, const void *x, hstu_dtype_t grad_dtype,
                             const void *dy, void *dx, const hstu_layer_grads_t *grads, void *workspace,
                             size_t workspace_bytes, void *stream) {
  return layer_bwd_impl(jag, desc, w, dtype, x_dtype, x, grad_dtype, dy, dx, grads, nullptr, 0, workspace,
                        workspace_bytes, stream);
}

hstu_status_t hstu_layer_bwd_saved(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                   const hstu_layer_weights_t *w, hstu_dtype_t dtype, hstu_dtype_t x_dtype,
                                   const void *x, hstu_dtype_t grad_dtype, const void *dy, void *dx,
                                   const hstu_layer_grads_t *grads, void *saved, size_t saved_bytes, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  if (!saved) return fail(HSTU_ERR_INVALID_ARGUMENT, "saved is NULL");
  return layer_bwd_impl(jag, desc, w, dtype, x_dtype, x, grad_dtype, dy, dx, grads, saved, saved_bytes, workspace,
                        workspace_bytes, stream);
}

size_t hstu_layer_saved_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, const hstu_layer_weights_t *w,
                              hstu_dtype_t dtype) {
  if (!jag || !desc || !w || jag->total_tokens < 0 || jag->num_seqs < 0 || desc->num_heads < 1 ||
      desc->head_dim < 1 || w->d_model < 1 || !valid_dtype(dtype))
    return 0;
  return layer_saved(jag, desc, w->d_model, dtype, w->ln_output != 0).total;
}

hstu_status_t hstu_layer_fwd_save(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                  const hstu_layer_weights_t *w, hstu_dtype_t dtype, hstu_dtype_t x_dtype,
                                  const void *x, hstu_dtype_t y_dtype, void *y, void *saved, size_t saved_bytes,
                                  void *stream) {
  try {
    hstu_status_t st = check_jagged_desc(jag, desc);
    if (st != HSTU_OK) return st;
    if (!w) return fail(HSTU_ERR_INVALID_ARGUMENT, "weights is NULL");
    if (!valid_dtype(dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "dtype = %d invalid", (int)dtype);
    if (!valid_dtype(x_dtype) || (x_dtype != dtype && x_dtype != HSTU_F32))
      return fail(HSTU_ERR_UNSUPPORTED, "x_dtype = %d must be HSTU_F32 or dtype", (int)x_dtype);
    if (!valid_dtype(y_dtype) || (y_dtype != dtype && y_dtype != HSTU_F32))
      return fail(HSTU_ERR_UNSUPPORTED, "y_dtype = %d must be HSTU_F32 or dtype", (int)y_dtype);
    const int64_t T = jag->total_tokens, D = w->d_model;
    if (D < 1 || D % 8 != 0 || D > 4096)
      return fail(HSTU_ERR_UNSUPPORTED, "d_model = %lld must be a multiple of 8 in [8, 4096]", (long long)D);
    if (!(w->ln_eps > 0.0f)) return fail(HSTU_ERR_INVALID_ARGUMENT, "ln_eps must be > 0");
    if (!w->w_uvqk || !w->w_out) return fail(HSTU_ERR_INVALID_ARGUMENT, "w_uvqk/w_out is NULL");
    if (!aligned16(w->w_uvqk) || !aligned16(w->w_out))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "weights must be 16-byte aligned");
    const LayerSaved sv = layer_saved(jag, desc, D, dtype, w->ln_output != 0);
    if (saved_bytes < sv.total)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL, "saved %zu < %zu bytes", saved_bytes, sv.total);
    if (T == 0) return ok();
    if (!x || !y || !saved) return fail(HSTU_ERR_INVALID_ARGUMENT, "x/y/saved is NULL");
    if (!aligned16(x) || !aligned16(y) || !aligned16(saved))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "x/y/saved must be 16-byte aligned");
    const size_t nx = (size_t)T * D * esize(x_dtype), ny = (size_t)T * D * esize(y_dtype);
    if (overlaps(x, nx, y, ny)) return fail(HSTU_ERR_INVALID_ARGUMENT, "y overlaps x");
    if (overlaps(saved, sv.total, x, nx) || overlaps(saved, sv.total, y, ny))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "saved overlaps x or y");
    hstu_status_t r = run_layer_forward(jag, desc, w, dtype, x_dtype, x, (char *)saved, sv, y, y_dtype,
                                        (hipStream_t)stream);
    return r == HSTU_OK ? ok() : r;
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_layer_fwd_save");
  }
}

hstu_status_t hstu_gather_rows(const void *table, int64_t table_rows, int32_t d, hstu_dtype_t dtype,
                               const int64_t *ids, int32_t T, void *out, void *stream) {
  try {
    if (!valid_dtype(dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "dtype = %d invalid", (int)dtype);
    if (T < 0) return fail(HSTU_ERR_INVALID_ARGUMENT, "T = %d < 0", T);
    if (d < 1) return fail(HSTU_ERR_INVALID_ARGUMENT, "d = %d < 1", d);
    const int64_t row_bytes = (int64_t)d * esize(dtype);
    if (row_bytes % 16 != 0) return fail(HSTU_ERR_UNSUPPORTED, "row of %lld bytes is not a multiple of 16",
                                         (long long)row_bytes);
    if (table_rows < 1) return fail(HSTU_ERR_INVALID_ARGUMENT, "table_rows = %lld < 1", (long long)table_rows);
    if (T == 0) return ok();
    if (!table || !ids || !out) return fail(HSTU_ERR_INVALID_ARGUMENT, "table/ids/out is NULL");
    if (!aligned16(table) || !aligned16(out))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "table/out must be 16-byte aligned");
    if (overlaps(out, (size_t)T * row_bytes, table, (size_t)table_rows * row_bytes))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "out overlaps table");
    return from_hip(hstu::launch_gather_rows(table, table_rows, (int32_t)row_bytes, ids, T, out, (hipStream_t)stream),
                    "gather launch");
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_gather_rows");
  }
}

hstu_status_t hstu_id_errors(uint32_t *count, int32_t reset, void *stream) {
  try {
    if (!count) return fail(HSTU_ERR_INVALID_ARGUMENT, "count is NULL");
    unsigned int *word = nullptr;
    hipError_t e = hstu::id_error_word(&word);
    if (e != hipSuccess) return from_hip(e, "id-error word lookup");
    e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e, "stream synchronize");
    unsigned int v = 0;
    e = hipMemcpy(&v, word, sizeof v, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return from_hip(e, "id-error word read");
    if (reset) {
      const unsigned int zero = 0;
      e = hipMemcpy(word, &zero, sizeof zero, hipMemcpyHostToDevice);
      if (e != hipSuccess) return from_hip(e, "id-error word reset");
    }
    *count = v;
    return ok();
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_id_errors");
  }
}

namespace {

// Stack workspace.  Fused path (bf16, large-tile shapes): U (fp32), V, Q, K (bf16), O (fp32) and its
// per-head statistics, the timestamp ranges, two fp32 pre-LayerNorm sums r (ping-pong between layers),
// the per-tile row statistics of the output GEMM and two per-row (mean, rstd) arrays.  Otherwise: the
// gathered x0 (dtype), two fp32 inter-layer activations and one layer workspace.
struct StackWs {
  bool fused;
  size_t u, v, q, k, o, ostat, stats, r32[2], tstats, rowstat[2];
  size_t x0, act[2], layer, layer_bytes;
  size_t total;
};

StackWs stack_ws(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc0, int64_t D, hstu_dtype_t dt) {
  StackWs w{};
  const int64_t T = jag->total_tokens, B = jag->num_seqs, H = desc0->num_heads, HD = H * desc0->head_dim;
  w.fused = dt == HSTU_BF16 && T > 0 && hstu::stack_gemms_fit(T, D, HD);
  if (T == 0) return w;                 // nothing to stage
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes, 256);
    return at;
  };
  if (w.fused) {
    w.u = take((size_t)T * HD * 4);
    w.v = take((size_t)T * HD * 2);
    w.q = take((size_t)T * HD * 2);
    w.k = take((size_t)T * HD * 2);
    w.o = take((size_t)T * HD * 4);
    w.ostat = take((size_t)T * H * 8);
    w.stats = take(hstu::attn_tau_stats_bytes(T, B));
    w.r32[0] = take((size_t)T * D * 4);
    w.r32[1] = take((size_t)T * D * 4);
    w.tstats = take((size_t)T * hstu::stack_out_col_tiles(D) * 8);
    w.rowstat[0] = take((size_t)T * 8);
    w.rowstat[1] = take((size_t)T * 8);
  } else {
    w.x0 = take((size_t)T * D * esize(dt));
    w.act[0] = take((size_t)T * D * 4);
    w.act[1] = take((size_t)T * D * 4);
    w.layer_bytes = layer_ws(T, B, H, HD, D, dt, true).total;
    w.layer = take(w.layer_bytes);
  }
  w.total = off;
  return w;
}

// Checks shared by the stack's size query and the stack call: every layer's descriptor and weights,
// one d_model and one H x Dh for all layers.
hstu_status_t check_stack(const hstu_jagged_t *jag, const hstu_attn_desc_t *descs, const hstu_layer_weights_t *ws,
                          int32_t L, hstu_dtype_t dtype) {
  if (L < 1) return fail(HSTU_ERR_INVALID_ARGUMENT, "num_layers = %d < 1", L);
  if (!descs || !ws) return fail(HSTU_ERR_INVALID_ARGUMENT, "descs/weights is NULL");
  if (!valid_dtype(dtype)) return fail(HSTU_ERR_INVALID_ARGUMENT, "dtype = %d invalid", (int)dtype);
  for (int32_t l = 0; l < L; ++l) {
    hstu_status_t st = check_jagged_desc(jag, &descs[l]);
    if (st != HSTU_OK) return st;
    if (descs[l].num_heads != descs[0].num_heads || descs[l].head_dim != descs[0].head_dim)
      return fail(HSTU_ERR_UNSUPPORTED, "layer %d: num_heads/head_dim differ from layer 0", l);
    if (descs[l].mask != descs[0].mask) return fail(HSTU_ERR_INVALID_ARGUMENT, "layer %d: mask differs", l);
    const hstu_layer_weights_t &w = ws[l];
    if (w.d_model != ws[0].d_model) return fail(HSTU_ERR_INVALID_ARGUMENT, "layer %d: d_model differs", l);
    if (w.d_model < 8 || w.d_model % 8 != 0 || w.d_model > 4096)
      return fail(HSTU_ERR_UNSUPPORTED, "d_model = %d must be a multiple of 8 in [8, 4096]", w.d_model);
    if (!(w.ln_eps > 0.0f)) return fail(HSTU_ERR_INVALID_ARGUMENT, "layer %d: ln_eps must be > 0", l);
    if (!w.w_uvqk || !w.w_out) return fail(HSTU_ERR_INVALID_ARGUMENT, "layer %d: w_uvqk/w_out is NULL", l);
    if (!aligned16(w.w_uvqk) || !aligned16(w.w_out))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "layer %d: weights must be 16-byte aligned", l);
  }
  return HSTU_OK;
}

}  // namespace

size_t hstu_stack_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *descs,
                                  const hstu_layer_weights_t *weights, int32_t num_layers, hstu_dtype_t dtype) {
  if (!jag || !descs || !weights || num_layers < 1 || jag->total_tokens < 0 || jag->num_seqs < 0 ||
      descs[0].num_heads < 1 || descs[0].head_dim < 1 || weights[0].d_model < 1 || !valid_dtype(dtype))
    return 0;
  return stack_ws(jag, &descs[0], weights[0].d_model, dtype).total;
}

hstu_status_t hstu_stack_fwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *descs,
                             const hstu_layer_weights_t *weights, int32_t num_layers, hstu_dtype_t dtype,
                             const void *table, int64_t table_rows, const int64_t *ids, hstu_dtype_t y_dtype,
                             void *y, void *workspace, size_t workspace_bytes, void *stream) {
  try {
    hstu_status_t st = check_stack(jag, descs, weights, num_layers, dtype);
    if (st != HSTU_OK) return st;
    if (!valid_dtype(y_dtype) || (y_dtype != dtype && y_dtype != HSTU_F32))
      return fail(HSTU_ERR_UNSUPPORTED, "y_dtype = %d must be HSTU_F32 or dtype", (int)y_dtype);
    const int64_t T = jag->total_tokens, D = weights[0].d_model;
    const int64_t H = descs[0].num_heads, HD = H * descs[0].head_dim;
    if (ids ? table_rows < 1 : table_rows < T)
      return fail(HSTU_ERR_INVALID_ARGUMENT, "table_rows = %lld too small", (long long)table_rows);
    const StackWs ws = stack_ws(jag, &descs[0], D, dtype);
    if (workspace_bytes < ws.total)
      return fail(HSTU_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, ws.total);
    if (T == 0) return ok();
    if (!table || !y || !workspace) return fail(HSTU_ERR_INVALID_ARGUMENT, "table/y/workspace is NULL");
    if (!aligned16(table) || !aligned16(y) || !aligned16(workspace))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "table/y/workspace must be 16-byte aligned");
    const size_t ntab = (size_t)table_rows * D * esize(dtype), ny = (size_t)T * D * esize(y_dtype);
    if (overlaps(y, ny, table, ntab)) return fail(HSTU_ERR_INVALID_ARGUMENT, "y overlaps the table");
    if (overlaps(workspace, ws.total, table, ntab) || overlaps(workspace, ws.total, y, ny))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace overlaps the table or y");
    if (ids && overlaps(workspace, ws.total, ids, (size_t)T * 8))
      return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace overlaps ids");

    hipStream_t s = (hipStream_t)stream;
    char *wsb = (char *)workspace;
    const int L = num_layers;
    if (!ws.fused) {
      // gather once, then one layer at a time through hstu_layer_fwd with fp32 activations between layers
      const void *x = table;
      if (ids) {
        hstu_status_t g = hstu_gather_rows(table, table_rows, (int32_t)D, dtype, ids, (int32_t)T, wsb + ws.x0, stream);
        if (g != HSTU_OK) return g;
        x = wsb + ws.x0;
      }
      hstu_dtype_t x_dt = dtype;
      for (int l = 0; l < L; ++l) {
        hstu_layer_weights_t w = weights[l];
        const bool last = l == L - 1;
        w.ln_output = last ? 0 : 1;
        void *out = last ? y : (void *)(wsb + ws.act[l % 2]);
        hstu_status_t r = hstu_layer_fwd(jag, &descs[l], &w, dtype, x_dt, x, last ? y_dtype : HSTU_F32, out,
                                         wsb + ws.layer, ws.layer_bytes, stream);
        if (r != HSTU_OK) return r;
        x = out;
        x_dt = HSTU_F32;
      }
      return ok();
    }

    hipError_t e;
    unsigned int *id_err = nullptr;
    if (ids) {
      e = hstu::id_error_word(&id_err);
      if (e != hipSuccess) return from_hip(e, "id-error word lookup");
    }
    for (int l = 0; l < L; ++l) {
      const hstu_layer_weights_t &w = weights[l];
      const bool last = l == L - 1;
      const int prev = (l + 1) % 2;   // buffers written by layer l - 1
      hstu::GemmStackProjArgs g1{};
      g1.a_mode = l == 0 ? (ids ? 1 : 0) : 2;
      g1.a = l == 0 ? table : (const void *)(wsb + ws.r32[prev]);
      g1.ids = ids; g1.id_rows = table_rows; g1.id_err = id_err;
      g1.a_rowstat = (const float *)(wsb + ws.rowstat[prev]);
      g1.w = w.w_uvqk; g1.bias = w.b_uvqk;
      g1.u = (float *)(wsb + ws.u); g1.v = wsb + ws.v; g1.q = wsb + ws.q; g1.k = wsb + ws.k;
      g1.M = (int32_t)T; g1.K = (int32_t)D; g1.HD = (int32_t)HD; g1.split = w.act_split != 0;
      e = hstu::launch_gemm_stack_proj(g1, s);
      if (e != hipSuccess) return from_hip(e, "projection GEMM launch");

      hstu::AttnArgs a = attn_args(jag, &descs[l]);
      a.q = wsb + ws.q; a.k = wsb + ws.k; a.v = wsb + ws.v; a.out = wsb + ws.o;
      a.row_stride = HD; a.out_row_stride = HD;
      a.in_dtype = hstu::kBF16; a.out_dtype = hstu::kF32;
      a.tau_stats = (int64_t *)(wsb + ws.stats);
      a.row_stats = (float *)(wsb + ws.ostat);
      e = hstu::launch_attn_fwd(a, s);
      if (e != hipSuccess) return from_hip(e, "attention launch");

      hstu::GemmStackOutArgs g2{};
      g2.o = (const float *)(wsb + ws.o); g2.u = (const float *)(wsb + ws.u);
      g2.row_stats = (const float *)(wsb + ws.ostat);
      g2.heads = (int32_t)H; g2.head_dim = descs[0].head_dim; g2.eps = w.ln_eps;
      g2.w = w.w_out; g2.bias = w.b_out;
      g2.resid_mode = g1.a_mode; g2.resid = g1.a; g2.ids = ids; g2.id_rows = table_rows; g2.id_err = id_err;
      g2.resid_rowstat = g1.a_rowstat;
      g2.y32 = last ? nullptr : (float *)(wsb + ws.r32[l % 2]);
      g2.out_stats = last ? nullptr : (float *)(wsb + ws.tstats);
      g2.y = last ? y : nullptr; g2.y_f32 = y_dtype == HSTU_F32;
      g2.M = (int32_t)T; g2.N = (int32_t)D; g2.K = (int32_t)HD; g2.split = w.act_split != 0;
      e = hstu::launch_gemm_stack_out(g2, s);
      if (e != hipSuccess) return from_hip(e, "output GEMM launch");
      if (!last) {
        e = hstu::launch_row_stats_combine((const float *)(wsb + ws.tstats), (float *)(wsb + ws.rowstat[l % 2]),
                                           (int)T, (int)D, w.ln_eps, s);
        if (e != hipSuccess) return from_hip(e, "row statistics launch");
      }
    }
    return ok();
  } catch (...) {
    return fail(HSTU_ERR_DEVICE, "unexpected C++ exception in hstu_stack_fwd");
  }
}

}  // extern "C"
