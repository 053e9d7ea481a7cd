// Internal launch interface between the C-ABI host code (api.cpp) and the HIP kernels.
// Host-side validation happens in api.cpp; every launcher here assumes valid arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hstu {

enum Dtype : int { kF32 = 0, kBF16 = 1 };
enum Mask : int { kCausal = 0, kCausalCandidates = 1 };

// Pointwise attention over a jagged batch.
struct AttnArgs {
  const void *q, *k, *v;          // [T][row_stride] elements, head h at column h*Dh
  void *out;                      // [T][out_row_stride] elements, head h at column h*Dh
  int64_t row_stride;             // elements between tokens in q/k/v
  int64_t out_row_stride;         // elements between tokens in out
  const int32_t *seq_offsets;     // [B+1]
  const int64_t *timestamps;      // [T]
  const int32_t *num_candidates;  // [B] or null
  const float *attn_scale;        // [B] or null
  const float *pos_bias;          // [R][P]
  const float *time_bias;         // [R][Tb]
  int32_t num_seqs, num_heads, head_dim, max_seq_len;
  int64_t num_rows_total;         // T (rows of q, k, v, timestamps)
  int32_t num_pos_buckets, num_time_buckets, rab_rows;
  int32_t mask;
  int32_t in_dtype, out_dtype;
  int64_t *tau_stats;             // workspace: attn_tau_stats_bytes() of per-32-token timestamp ranges
  float *row_stats;               // [T][H][2] mean and sum of squared deviations of each stored head row
                                  // (fp32 output only; the gate of the output projection uses them), or null
  // Cached-history scoring only (launch_attn_cached): the fields above describe the candidate rows
  // (q, k, v, out, seq_offsets, timestamps, tau_stats; max_seq_len = most candidates of one user);
  // the keys are each user's cached history rows.
  const void *k_hist, *v_hist;     // [T_h][row_stride] elements
  const int32_t *hist_offsets;     // [B+1]
  const int64_t *hist_timestamps;  // [T_h]
  int64_t *hist_tau_stats;         // workspace: attn_tau_stats_bytes(T_h, B)
  int32_t num_rows;                // T_c (candidate rows)
  int64_t num_hist_rows;           // T_h
  int32_t kv_splits;               // workgroups per (candidate block, user, head) along the history, >= 1
  int32_t tiles_per_split;         // 64-key history tiles per split (the last split takes the rest)
  float *partial;                  // kv_splits > 1: workspace [kv_splits][T_c][H][Dh] fp32 raw sums;
                                   // backward dQ pass: [workgroups][P + 65] bias-gradient bins
  // Backward only (launch_attn_bwd_dq / launch_attn_bwd_dkdv)
  const void *d_out;               // [T][row_stride] upstream gradient of out, in_dtype
  float *d_pos_bias, *d_time_bias; // [R][P], [R][Tb]
  float *dk, *dv;                  // [T][row_stride] fp32 (dQ goes to out, fp32)
  // Layer path: when z_q is set, the gradients instead become those of the projection's pre-activation,
  // dz = d{q,k,v} * SiLU'(z), written in place over z (in_dtype) at z_q, z_k, z_v (head h at column
  // h*Dh of each row, z_row_stride elements between tokens); out, dk and dv are not written.
  void *z_q, *z_k, *z_v;
  int64_t z_row_stride;
};

// Key splits of cached scoring for a batch: enough workgroups to fill the chip, each split a whole
// number of 64-key tiles.  Returns kv_splits (>= 1) and sets tiles_per_split.
int attn_cached_splits(int64_t num_seqs, int64_t num_heads, int64_t max_candidates, int64_t max_history,
                       int32_t *tiles_per_split);

// Workspace bytes of the per-32-token timestamp ranges the attention kernel classifies tiles with.
size_t attn_tau_stats_bytes(int64_t total_tokens, int64_t num_seqs);
// Allocation-free forward: bytes of the file-scope device scratch array (noalloc.hip), and its device
// address on the current device (looked up once per device, then cached).
constexpr size_t kNoallocScratchBytes = (size_t)1 << 20;
hipError_t noalloc_scratch(void **ptr);
// Device address of the current device's id-error word: gathers add 1 for each read whose row id lies
// outside [0, table_rows) (the read is clamped to the nearest row).
hipError_t id_error_word(unsigned int **ptr);
hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t stream);
// Causal softmax attention (bf16 inputs, Dh = 128), the comparison point of the pointwise forward:
// q, k, v, out, row strides, seq_offsets, num_seqs, num_heads, max_seq_len, out_dtype are read.
hipError_t launch_softmax_attn(const AttnArgs &a, hipStream_t stream);
// Candidates against a cached history: each candidate sees every history key of its user and itself.
hipError_t launch_attn_cached(const AttnArgs &a, hipStream_t stream);

// Backward of the pointwise attention.  The dQ pass (query-major, the forward's tiles) writes dQ to
// `out` and the bias-table gradients; the dK/dV pass (key-major) writes dk and dv.  Both recompute the
// scores.  Workspace of the dQ pass: tau_stats and `partial` (attn_bwd_partial_floats floats).
hipError_t launch_attn_bwd_dq(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_bwd_dkdv(const AttnArgs &a, hipStream_t stream);
size_t attn_bwd_dq_lds_bytes(int in_dtype, int head_dim, int num_pos_buckets);
size_t attn_bwd_dkdv_lds_bytes(int in_dtype, int head_dim, int num_pos_buckets);
inline int64_t attn_bwd_partial_floats(int64_t num_seqs, int64_t num_heads, int64_t max_seq_len, int64_t P) {
  return (max_seq_len + 127) / 128 * num_heads * num_seqs * (P + 65);
}

// C[M][N] = epilogue(A[M][K] * B[N][K]^T): bf16 or f32 weights (MFMA operand type `dtype`), fp32
// accumulation.  With bf16 weights the activation A may be fp32 (x_f32 / g_f32): rounded to bf16, or with
// split = 1 entered as a bf16 hi + lo pair (two MFMA passes).
struct GemmUvqkArgs {
  const void *x;                  // [M][K], fp32 if x_f32 else dtype
  const void *w;                  // [4*HD][K] dtype
  const void *bias;               // [4*HD] dtype or null
  float *u;                       // [M][HD] fp32
  void *v, *q, *k;                // each [M][HD] dtype
  void *z;                        // [M][4*HD] dtype: the pre-activation x W1^T + b1, or null
  int32_t M, K, HD;
  int32_t dtype, x_f32, split;
};
hipError_t launch_gemm_uvqk(const GemmUvqkArgs &a, hipStream_t stream);

// Output projection with the gate fused into its A operand:
//   A[m][k] = (o[m][k] - mean_m) * rstd_m * u[m][k],   y = x + A W2^T + b2
// (LayerNorm over the whole H*Dh row of o, biased variance, no affine).  mean_m and rstd_m are
// combined from the per-head statistics the attention kernel wrote next to o.  y goes to y, or in fp32
// to y32 when a LayerNorm follows.
struct GemmOutArgs {
  const float *o;                 // [M][K] fp32 attention output (K = H*Dh)
  const float *u;                 // [M][K] fp32
  const float *row_stats;         // [M][H][2] per-head mean and sum of squared deviations of o
  int32_t heads, head_dim;
  float eps;
  const void *w;                  // [N][K] dtype (N = D)
  const void *bias;               // [N] dtype or null
  const void *x;                  // [M][N] residual: fp32 if x_f32 else dtype
  void *y;                        // [M][N]: fp32 if y_f32 else dtype (unused when y32 is set)
  float *y32;                     // [M][N] fp32 pre-LayerNorm result, or null
  int32_t M, N, K;
  int32_t dtype, split, x_f32, y_f32;
};
hipError_t launch_gemm_out(const GemmOutArgs &a, hipStream_t stream);

struct RowLnArgs {
  const float *in;                // [M][N] fp32
  void *out;                      // [M][N]: fp32 if out_f32 else bf16
  int32_t M, N;
  float eps;
  int32_t out_f32;
};
hipError_t launch_row_layernorm(const RowLnArgs &a, hipStream_t stream);

// Plain product c = A B^T (+ resid), A [M][K] (fp32 if a_f32 else dtype), B [N][K] dtype, c fp32 if c_f32
// else dtype, resid [M][N] (fp32 if resid_f32 else dtype) or null.  splits > 1 (bf16 A and B, K a
// multiple of 32, no resid, fp32 c): K is cut into `splits` ranges whose fp32 products go to
// partial [splits][M][N] and are then summed in split order.
struct GemmPlainArgs {
  const void *a, *b, *resid;
  void *c;
  float *partial;
  int32_t M, N, K, dtype, a_f32, resid_f32, c_f32, splits;
};
hipError_t launch_gemm_plain(const GemmPlainArgs &a, hipStream_t stream);
int gemm_plain_splits(int64_t M, int64_t N, int64_t K, int dtype, int a_f32);

// ---- fused stack (bf16 weights, large-tile kernels only: stack_gemms_fit must hold)
// Projection with its A operand read as bf16 rows of `a` (a_mode 0), bf16 table rows a[ids[m]]
// (a_mode 1: the embedding gather), or LN of fp32 rows of `a` with per-row (mean, rstd) a_rowstat
// (a_mode 2: the previous layer's post-LayerNorm; split: bf16 hi + lo).  Outputs as GemmUvqkArgs.
struct GemmStackProjArgs {
  int32_t a_mode;
  const void *a;
  const int64_t *ids;      // a_mode 1: row ids, clamped into [0, id_rows) (each clamp counted in id_err)
  int64_t id_rows;
  unsigned int *id_err;
  const float *a_rowstat;
  const void *w, *bias;
  float *u;
  void *v, *q, *k;
  int32_t M, K, HD, split;
};
hipError_t launch_gemm_stack_proj(const GemmStackProjArgs &a, hipStream_t stream);
// Gated output projection (A as GemmOutArgs) with the residual read as bf16 rows (resid_mode 0),
// gathered bf16 table rows resid[ids[m]] (1), or LN of fp32 rows with resid_rowstat (2).  Either the
// fp32 sum y32 plus per-row (mean, M2) of every 256-column tile (out_stats [M][stack_out_col_tiles(N)][2])
// for a LayerNorm that the next layer applies, or y (bf16, or fp32 if y_f32).
struct GemmStackOutArgs {
  const float *o, *u, *row_stats;
  int32_t heads, head_dim;
  float eps;
  const void *w, *bias;
  int32_t resid_mode;
  const void *resid;
  const int64_t *ids;      // resid_mode 1: row ids, clamped into [0, id_rows) (each clamp counted in id_err)
  int64_t id_rows;
  unsigned int *id_err;
  const float *resid_rowstat;
  float *y32, *out_stats;
  void *y;
  int32_t y_f32, M, N, K, split;
};
hipError_t launch_gemm_stack_out(const GemmStackOutArgs &a, hipStream_t stream);
bool stack_gemms_fit(int64_t M, int64_t D, int64_t HD);
int stack_out_col_tiles(int64_t N);
// rowstat[m] = (mean, 1/sqrt(var + eps)) of row m from its column tiles' (mean, M2) (tile c holds
// min(256, N - 256 c) columns), combined in tile order.
hipError_t launch_row_stats_combine(const float *tile_stats, float *rowstat, int M, int N, float eps,
                                    hipStream_t stream);

// ---- layer backward, HBM-bound pieces
// dr = LN'(r) dy in place over r: r fp32 [M][N] (the pre-LayerNorm sum), dy [M][N] fp32 if dy_f32 else bf16.
struct LnBwdArgs {
  float *r;
  const void *dy;
  int32_t M, N, dy_f32;
  float eps;
};
hipError_t launch_ln_bwd_rows(const LnBwdArgs &a, hipStream_t stream);

// Norm-gate backward: o, u, dg fp32 [M][N]; z dtype [M][4N] (its U slice becomes dz_U); g, d_o dtype [M][N].
struct NormGateBwdArgs {
  const float *o, *u, *dg;
  void *z, *g, *d_o;
  int32_t M, N, dtype;
  float eps;
};
hipError_t launch_norm_gate_bwd(const NormGateBwdArgs &a, hipStream_t stream);

// dst [C][Rp] = src[R][C]^T with rows R..Rp-1 zero (C % 4 == 0, Rp % 4 == 0, Rp >= R).  With colsum,
// also colsum[c * transpose_colsum_ld(Rp) + t] = the sum of column c over the 64 source rows of tile t
// (0 past the rows), for launch_row_sum to add in a fixed order.
hipError_t launch_transpose(const void *src, int src_f32, void *dst, int dst_f32, int R, int C, int Rp,
                            hipStream_t stream, float *colsum = nullptr);
int transpose_colsum_ld(int Rp);   // 64-row tiles of Rp rows, rounded up to a multiple of 4
// out[c] = sum of row c of src [rows][Rp] (Rp % 4 == 0), fixed summation order.
hipError_t launch_row_sum(const void *src, int src_f32, float *out, int rows, int Rp, hipStream_t stream);
// p[0..n) = 0 (a kernel, not a memset, so that a captured graph replays it faithfully).
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream);

hipError_t launch_gather_rows(const void *table, int64_t table_rows, int32_t row_bytes, const int64_t *ids,
                              int32_t T, void *out, hipStream_t stream);

}  // namespace hstu
