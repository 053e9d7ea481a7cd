/*
 * hstu.h -- C ABI of libhstu, the MI355X (gfx950) HSTU layer: forward, a fused layer stack over
 * embedding-table input, cached-history candidate scoring, and the backward of the attention and of
 * the whole layer.
 *
 * What it computes.  The HSTU layer as the pages describe it: "DLRMv4：MLPerfの推薦システム訓練
 * ベンチマークがシーケンス化時代へ", section "モデルアーキテクチャ：HSTUが従来の特徴インタラクション
 * スタックに取って代わる" -- one projection makes every internal representation of the layer,
 * pointwise attention aggregates the sequence with a bias from the positional and temporal distance
 * of two events, and a gated transformation lets the aggregated features interact.  Section
 * "1つの訓練サンプルがHSTUでどのように処理されるか" of the same page: a time-ordered per-user event
 * sequence, candidates appended at the end, the whole sequence processed as one causal block.
 * "Actions Speak Louder than Words: Trillion-Parameter Sequential Transducers for Generative
 * Recommendations", abstract: HSTU, an attention variant for high-cardinality, non-stationary
 * streaming data, at sequence length 8192.
 *
 * Formulas (the pages fix the structure, not the algebra; these are the readings implemented):
 *   projection  z_t = W1 x_t + b1;  U|V|Q|K = SiLU(z_t) split into four H*Dh slices, head-major
 *   scores      s_ij = q_i . k_j + pos_bias[r][bp] + time_bias[r][bt]     (no 1/sqrt(Dh))
 *               bp = min(|pos_i - pos_j|, P-1), bt = min(bitlen(|tau_i - tau_j|), Tb-1) (exact int64)
 *   attention   O_i = c_b * sum_{allowed j} SiLU(s_ij) v_j,  c_b = attn_scale[b] or 1/n_b   (no softmax)
 *   gate        g_t = LN(concat_h O_t) * U_t     (LN over H*Dh, biased variance, no affine)
 *   output      y_t = x_t + W2 g_t + b2;  if ln_output: y_t = LN(y_t)
 * Masks: HSTU_MASK_CAUSAL allows j <= i.  HSTU_MASK_CAUSAL_CANDIDATES: the last m_b tokens of
 * sequence b are candidates (n_h = n_b - m_b); history rows allow j <= i; a candidate row allows
 * every j < n_h and j = i (never another candidate); candidates take position n_h.
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are device addresses owned by the caller; the library keeps none of
 *    them after the call returns and never allocates or frees device memory.  Scratch memory comes
 *    from the caller's `workspace`, sized by the matching *_workspace_bytes() call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All work is enqueued on
 *    it; calls return before the work completes; nothing is synchronised and nothing is copied
 *    between host and device, so the calls can be captured in a HIP graph.
 *  - Everything the host can check is checked before any launch (null pointers, sizes, supported
 *    head_dim / dtype pairs, workspace size, 16-byte alignment).  A failure returns a status and
 *    leaves a message for hstu_last_error(); no C++ exception crosses the ABI; a failed launch
 *    returns HSTU_ERR_DEVICE with the HIP error text.
 *  - Device-resident content is the caller's contract and is not validated on the hot path:
 *    offsets must be non-decreasing from 0 to total_tokens, 0 <= num_candidates[b] <= n_b,
 *    and ids must be in [0, table_rows) (an id outside is clamped and counted: hstu_id_errors).
 *  - Outputs are bitwise deterministic for identical inputs on one device (no float atomics).
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSTU_ABI_VERSION 9

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARGUMENT = 1,
  HSTU_ERR_UNSUPPORTED = 2,
  HSTU_ERR_WORKSPACE_TOO_SMALL = 3,
  HSTU_ERR_DEVICE = 4
} hstu_status_t;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype_t;

typedef enum { HSTU_MASK_CAUSAL = 0, HSTU_MASK_CAUSAL_CANDIDATES = 1 } hstu_mask_t;

/* The jagged batch: B per-user event sequences packed back to back (T tokens in total). */
typedef struct {
  int32_t num_seqs;              /* B >= 0 (host)                                                  */
  int32_t total_tokens;          /* T = seq_offsets[B] (host); sizes the launch, never read back   */
  int32_t max_seq_len;           /* >= max_b n_b (host); sizes the launch, never read back         */
  const int32_t *seq_offsets;    /* [B+1] (device): 0 = o_0 <= o_1 <= ... <= o_B = T               */
  const int64_t *timestamps;     /* [T] (device): any int64 (seconds in the shipped workloads)     */
  const int32_t *num_candidates; /* [B] (device): m_b, required iff mask == CAUSAL_CANDIDATES       */
  const float *attn_scale;       /* [B] (device) c_b, or NULL for c_b = 1/n_b                      */
} hstu_jagged_t;

/* The pointwise attention and its relative-attention bias (rab) tables. */
typedef struct {
  int32_t num_heads;             /* H >= 1                                                         */
  int32_t head_dim;              /* Dh in {32, 64, 128}                                            */
  int32_t num_pos_buckets;       /* P in [1, 4096]                                                 */
  int32_t num_time_buckets;      /* Tb in [1, 4096]                                                */
  int32_t rab_rows;              /* R = 1 (one table pair shared by all heads) or R = H            */
  const float *pos_bias;         /* [R][P] fp32 (device)                                           */
  const float *time_bias;        /* [R][Tb] fp32 (device)                                          */
  hstu_mask_t mask;
} hstu_attn_desc_t;

/* Weights and numerics options of one layer; weight element type is the call's `dtype`. */
typedef struct {
  int32_t d_model;               /* D, a multiple of 8 in [8, 4096]                                */
  const void *w_uvqk;            /* [4*H*Dh][D] (device): rows U | V | Q | K, head-major in each  */
  const void *b_uvqk;            /* [4*H*Dh] (device) or NULL                                      */
  const void *w_out;             /* [D][H*Dh] (device)                                             */
  const void *b_out;             /* [D] (device) or NULL                                           */
  float ln_eps;                  /* > 0; used by the gate's LayerNorm and the output LayerNorm    */
  int32_t ln_output;             /* 1: y = LN(x + branch) (between stacked layers); 0: y = x + branch */
  int32_t act_split;             /* bf16 only.  0: fp32 activations (x, and the gate g) are rounded
                                    to bf16 before the GEMMs.  1: they enter both GEMMs as a bf16
                                    hi + lo pair (two MFMA passes, ~16 significant bits), so long
                                    stacks keep fp32-activation accuracy.  Ignored for f32.        */
} hstu_layer_weights_t;

/* ABI version of the loaded library (HSTU_ABI_VERSION). */
int hstu_abi_version(void);

/* Text of a status code (static storage). */
const char *hstu_status_string(hstu_status_t status);

/* Detail of the last non-OK return on the calling thread (thread-local storage; "" if none). */
const char *hstu_last_error(void);

/*
 * Workspace needed by hstu_attn_fwd for this batch shape (bytes; 0 is possible).  Depends only on
 * the host fields of `jag` and `desc`.
 */
size_t hstu_attn_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                 hstu_dtype_t in_dtype);

/*
 * Pointwise attention forward (steps 2-3 of the layer; the causal-jagged kernel).  Passage: "DLRMv4"
 * page, section "モデルアーキテクチャ：HSTUが従来の特徴インタラクションスタックに取って代わる" --
 * pointwise attention aggregates the sequence, with a bias from the positional and the temporal
 * distance of two events; section "1つの訓練サンプルがHSTUでどのように処理されるか" -- each user's
 * time-ordered events form one causal block, candidates appended at its end (the mask
 * HSTU_MASK_CAUSAL_CANDIDATES); "Actions Speak Louder than Words ...", abstract -- the attention
 * variant run at sequence length 8192.  What it computes:
 *   out[t][h][:] = c_b * sum_{allowed j} SiLU(q_t . k_j + rab) v_j   for every token t of every sequence.
 * q, k, v: [T][H][Dh] row-major (device), dtype in_dtype (HSTU_BF16 or HSTU_F32).
 * out:     [T][H][Dh] row-major (device), out_dtype = HSTU_F32 or in_dtype; may not alias q, k, v.
 * bf16 inputs: QK^T and AV on bf16 MFMA with fp32 accumulation; SiLU(s) is rounded to bf16 as the
 * AV operand.  f32 inputs: fp32 MFMA throughout.
 * Returns HSTU_ERR_UNSUPPORTED for a head_dim outside {32, 64, 128}.
 */
hstu_status_t hstu_attn_fwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype,
                            const void *q, const void *k, const void *v, void *out, hstu_dtype_t out_dtype,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Scratch held by the allocation-free forward on each GPU (bytes): it serves every batch with
 * total_tokens / 32 + num_seqs + 1 <= 65536. */
#define HSTU_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)

/*
 * hstu_attn_fwd for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same kernels and bitwise the same result as
 * hstu_attn_fwd; the scratch (the per-32-token timestamp ranges) comes from a fixed device array of
 * HSTU_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process ends,
 * instead of from a caller workspace.  The caller passes only inputs and outputs, exactly as for
 * hstu_attn_fwd.  Nothing is allocated or freed (no hipMalloc, hipFree or allocating library call);
 * the first call on a device looks the array's device address up, with that device current, and keeps
 * it.  The scratch needs no clearing: each call writes every entry it later reads.  All calls on one GPU
 * share that GPU's array, which keeps the last call's contents, so calls that can overlap in time on
 * one GPU (several streams or host threads) race and must be serialised by the caller.
 * Errors: as hstu_attn_fwd; a batch with total_tokens / 32 + num_seqs + 1 > 65536 needs more scratch
 * than the array holds and is HSTU_ERR_WORKSPACE_TOO_SMALL, returned before anything is launched.
 */
hstu_status_t hstu_attn_fwd_noalloc(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype,
                                    const void *q, const void *k, const void *v, void *out, hstu_dtype_t out_dtype,
                                    void *stream);

/*
 * Causal softmax attention over the same jagged batch, for comparison with the pointwise attention:
 * "Actions Speak Louder than Words ...", abstract, measures HSTU against FlashAttention2-based
 * Transformers at sequence length 8192; this is the textbook attention of such a Transformer, timed on
 * the same shapes and hardware.  It is not a step of the HSTU layer.
 *   out[t][h][:] = sum_{j <= i} softmax_j(q_t . k_j / sqrt(Dh)) v_j     (sequence-local i, j; causal)
 * jag: num_seqs, total_tokens, max_seq_len and seq_offsets are read (timestamps, num_candidates and
 * attn_scale are not).  q, k, v: [T][num_heads][head_dim] bf16, row-major, 16-byte aligned (device).
 * out: [T][num_heads][head_dim], out_dtype HSTU_BF16 or HSTU_F32; may not overlap an input.
 * bf16 MFMA with fp32 accumulation; the online (running-maximum) softmax in fp32; the probabilities are
 * rounded to bf16 as the AV operand.  No workspace; nothing is allocated or synchronised.
 * Errors: HSTU_ERR_UNSUPPORTED unless in_dtype is HSTU_BF16 and head_dim is 128; the argument checks
 * of hstu_attn_fwd otherwise (HSTU_ERR_INVALID_ARGUMENT).
 */
hstu_status_t hstu_softmax_attn_fwd(const hstu_jagged_t *jag, int32_t num_heads, int32_t head_dim,
                                    hstu_dtype_t in_dtype, const void *q, const void *k, const void *v, void *out,
                                    hstu_dtype_t out_dtype, void *stream);

/*
 * Workspace needed by hstu_attn_fwd_cached (bytes; 0 is possible): the per-32-token timestamp ranges
 * of the candidate rows and of the history rows and, when a user's history is split over several
 * workgroups, their fp32 partial sums.  Depends only on the host fields of hist, cand and desc.
 */
size_t hstu_attn_cached_workspace_bytes(const hstu_jagged_t *hist, const hstu_jagged_t *cand,
                                        const hstu_attn_desc_t *desc);

/*
 * Candidates scored against a cached history: mini-batched candidate scoring ("Actions Speak Louder
 * than Words ..." summary page, key contributions and technical approach: M-FALCON), with each
 * candidate seeing the whole history of its user and itself ("DLRMv4" page, section on how one training
 * sample is processed).  For every candidate row c of user b (n_h history tokens, m_b candidates in
 * this call, every candidate at position n_h):
 *   out[c][h][:] = c_b * ( sum_{j < n_h} SiLU(q_c . k_hist_j + w_p[min(n_h - j, P-1)] + w_t[bt(tau_c, tau_j)]) v_hist_j
 *                          + SiLU(q_c . k_c + w_p[0] + w_t[0]) v_c ),
 *   c_b = cand->attn_scale[b], or 1 / (n_h + m_b) when attn_scale is NULL.
 * With all of a user's candidates in one call (or with attn_scale carrying that c_b) this equals the
 * candidate rows of hstu_attn_fwd with HSTU_MASK_CAUSAL_CANDIDATES over [history | candidates], so the
 * history's keys and values, computed once, serve any number of candidate micro-batches.
 * hist: num_seqs = B, total_tokens = T_h, max_seq_len = the longest history (host; it only sets how
 *       finely histories are split over workgroups, any value in [0, T_h] gives the same result),
 *       seq_offsets [B+1], timestamps [T_h] (device); num_candidates and attn_scale are not read.
 * cand: num_seqs = B (the same users, in the same order), total_tokens = T_c, max_seq_len = the most
 *       candidates of one user, seq_offsets [B+1], timestamps [T_c], attn_scale [B] or NULL (device);
 *       num_candidates is not read.
 * desc: as for hstu_attn_fwd; desc->mask is not read.
 * k_hist, v_hist: [T_h][H][Dh]; q, k, v (the candidates' own rows): [T_c][H][Dh]; all in_dtype,
 * row-major, 16-byte aligned (device).  out: [T_c][H][Dh], out_dtype = HSTU_F32 or in_dtype; may not
 * overlap an input or the workspace.  Caller-owned; nothing is allocated or retained.
 * The partial sums of a split history are added in a fixed order: the result is bitwise deterministic.
 * Errors: as for hstu_attn_fwd; hist->num_seqs != cand->num_seqs, hist->max_seq_len outside [0, T_h],
 * or a NULL pointer that the sizes require, is HSTU_ERR_INVALID_ARGUMENT.
 */
hstu_status_t hstu_attn_fwd_cached(const hstu_jagged_t *hist, const hstu_jagged_t *cand, const hstu_attn_desc_t *desc,
                                   hstu_dtype_t in_dtype, const void *k_hist, const void *v_hist, const void *q,
                                   const void *k, const void *v, void *out, hstu_dtype_t out_dtype, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * Workspace needed by hstu_attn_bwd (bytes; 0 is possible): the timestamp ranges and the per-workgroup
 * bias-gradient bins.  Depends only on the host fields of `jag` and `desc`.
 */
size_t hstu_attn_bwd_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                     hstu_dtype_t in_dtype);

/*
 * Backward of hstu_attn_fwd (the attention of "DLRMv4" page, section on the model architecture, is
 * trained: the page describes a training benchmark).  For an upstream gradient d_out of out:
 *   dv_j = c_b sum_i SiLU(s_ij) dO_i,   dS_ij = c_b (dO_i . v_j) SiLU'(s_ij) on allowed pairs,
 *   dq_i = sum_j dS_ij k_j,   dk_j = sum_i dS_ij q_i,
 *   d_pos_bias[r][p] = sum of dS_ij over the pairs with position bucket p (heads of table row r),
 *   d_time_bias[r][t] likewise over the time buckets,
 * with s_ij, the buckets, the masks and c_b exactly as in hstu_attn_fwd (c_b is a constant here).
 * q, k, v, d_out: [T][H][Dh], in_dtype, row-major, 16-byte aligned (device).
 * dq, dk, dv: [T][H][Dh] fp32; d_pos_bias: [R][P] fp32; d_time_bias: [R][Tb] fp32 (device, written, not
 * accumulated into; no output may overlap an input, another output or the workspace).
 * bf16 inputs: the products run on bf16 MFMA with fp32 accumulation (SiLU(s) and dS rounded to bf16 as
 * MFMA operands); f32 inputs: fp32 MFMA.  The result is bitwise deterministic (bias gradients are
 * summed per wave, per workgroup and across workgroups in a fixed order).
 * Errors: as hstu_attn_fwd; HSTU_ERR_UNSUPPORTED when the tables do not fit the kernels' LDS
 * (P up to 4096 fits for bf16 inputs).
 */
hstu_status_t hstu_attn_bwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc, hstu_dtype_t in_dtype,
                            const void *q, const void *k, const void *v, const void *d_out, float *dq, float *dk,
                            float *dv, float *d_pos_bias, float *d_time_bias, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Workspace needed by hstu_layer_fwd (bytes). */
size_t hstu_layer_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                  const hstu_layer_weights_t *w, hstu_dtype_t dtype);

/*
 * One HSTU layer forward (steps 1-4):  y = [LN](x + W2 (LN(O) * U) + b2).  Passage: "DLRMv4" page,
 * section "モデルアーキテクチャ：HSTUが従来の特徴インタラクションスタックに取って代わる" -- inside a
 * layer a single projection produces every internal representation, pointwise attention with a
 * position/time bias aggregates the sequence, and a gated transformation lets the aggregated features
 * interact in place of the cross network and feed-forward block.  The residual and the optional output
 * LayerNorm are the stack's ("residual plus LayerNorm between layers" is the reading taken for the
 * stacked workloads).
 * dtype:   element type of the weights and of the MFMA operands (HSTU_BF16: bf16 MFMA with fp32
 *          accumulation; HSTU_F32: fp32 throughout).
 * x:       [T][D] (device), element type x_dtype in {HSTU_F32, dtype}.
 * y:       [T][D] (device), element type y_dtype in {HSTU_F32, dtype}; may not overlap x.
 *          An fp32 residual stream between stacked bf16 layers (x_dtype = y_dtype = HSTU_F32) avoids
 *          rounding the activations to bf16 at every layer boundary.
 * Inside: the projection GEMM fuses bias, SiLU and the U|V|Q|K split into its epilogue (U is kept in
 * fp32, V, Q, K in dtype); the attention writes O in fp32 together with each head row's mean and sum
 * of squared deviations; the output GEMM computes the gate LN(O) * U in fp32 while it loads its A
 * operand (the gate is never stored), adds bias and residual in fp32 and rounds once (or hands the
 * fp32 sum to the output LayerNorm).
 */
hstu_status_t hstu_layer_fwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                             const hstu_layer_weights_t *w, hstu_dtype_t dtype, hstu_dtype_t x_dtype,
                             const void *x, hstu_dtype_t y_dtype, void *y, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Workspace needed by hstu_stack_fwd (bytes).  Depends only on host fields. */
size_t hstu_stack_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *descs,
                                  const hstu_layer_weights_t *weights, int32_t num_layers, hstu_dtype_t dtype);

/*
 * A stack of num_layers layers over rows of an embedding table ("DLRMv4" page, section on the model
 * architecture: the layer input is looked up from embedding tables; the layers are stacked with a
 * residual and a LayerNorm between them):
 *   x_0[t] = table[ids[t]]  (table[t] when ids is NULL)
 *   x_{l+1} = LN(x_l + branch_l(x_l)) for l < num_layers - 1,   y = x_L-1 + branch_L-1(x_L-1),
 * with branch_l the layer of hstu_layer_fwd (weights[l], descs[l]; weights[l].ln_output is not read).
 * Every layer has the same jag, d_model, num_heads, head_dim and mask; tables and weights are per layer.
 * table: [table_rows][D] dtype (device); ids: [T] int64 in [0, table_rows) (device; an id outside is
 * clamped to the nearest row and counted, as in hstu_gather_rows) or NULL (then
 * table_rows >= T); y: [T][D], y_dtype in {HSTU_F32, dtype} (device), may not overlap the table.
 * bf16 with large-tile shapes: the gather is done by layer 0's projection and output GEMMs while they
 * load their operands (x_0 is never stored); each output GEMM before a LayerNorm writes its fp32 sum
 * and per-row statistics of every 256-column tile, and the next layer applies the LayerNorm while its
 * GEMMs load that sum (x_{l+1} is never stored).  Otherwise the call gathers x_0 and runs
 * hstu_layer_fwd per layer with fp32 activations in between.  Both keep the residual stream in fp32.
 * Errors: as hstu_layer_fwd; layers that differ in d_model, num_heads, head_dim or mask are rejected.
 */
hstu_status_t hstu_stack_fwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *descs,
                             const hstu_layer_weights_t *weights, int32_t num_layers, hstu_dtype_t dtype,
                             const void *table, int64_t table_rows, const int64_t *ids, hstu_dtype_t y_dtype,
                             void *y, void *workspace, size_t workspace_bytes, void *stream);

/* Gradients of one layer's parameters: fp32 (device), written, not accumulated into. */
typedef struct {
  float *d_w_uvqk;               /* [4*H*Dh][D]                                                   */
  float *d_b_uvqk;               /* [4*H*Dh], or NULL: not computed                               */
  float *d_w_out;                /* [D][H*Dh]                                                     */
  float *d_b_out;                /* [D], or NULL: not computed                                    */
  float *d_pos_bias;             /* [R][P]                                                        */
  float *d_time_bias;            /* [R][Tb]                                                       */
} hstu_layer_grads_t;

/* Workspace needed by hstu_layer_bwd (bytes).  Depends only on host fields. */
size_t hstu_layer_bwd_workspace_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                      const hstu_layer_weights_t *w, hstu_dtype_t dtype);

/*
 * Backward of hstu_layer_fwd (the layer is trained: "DLRMv4" page, the benchmark is a training
 * benchmark; the layer is the one of its section on the model architecture).  For an upstream
 * gradient dy of y, with r = x + W2 g + b2 (y = LN(r) when ln_output, else y = r), g = LN(o) * U,
 * o = concat_h O and z = W1 x + b1 (U|V|Q|K = SiLU(z)):
 *   dr = LN'(r) dy (or dy);  d_b_out = sum_t dr;  d_w_out = dr^T g;  dg = dr W2
 *   dU = dg * LN(o);  do = LN'(o) (dg * U);  dQ, dK, dV and the bias-table gradients as hstu_attn_bwd
 *   dz = [dU | dV | dQ | dK] * SiLU'(z);  d_b_uvqk = sum_t dz;  d_w_uvqk = dz^T x;  dx = dr + dz W1
 * where LN'(a) b = rstd (b - mean(b) - a_hat mean(b * a_hat)) applies the LayerNorm Jacobian.
 * Nothing is saved from the forward: the call recomputes z, U, V, Q, K, O and g from x (in
 * the forward's numerics, act_split included) and keeps them in the workspace.
 * dtype, x_dtype, x, w, jag, desc: exactly as given to hstu_layer_fwd.
 * dy, dx: [T][D] (device), element type grad_dtype in {HSTU_F32, dtype}; dx may not overlap an input.
 * grads: d_w_uvqk, d_w_out, d_pos_bias, d_time_bias required; the bias gradients may be NULL.
 * bf16: every product runs on bf16 MFMA with fp32 accumulation (its operands rounded to bf16:
 * z, dz, g, dO and the transposed dr and x); the weight gradients are sums over all T tokens, split
 * over workgroups and added in a fixed order.  The result is bitwise deterministic.
 * Errors: as hstu_layer_fwd and hstu_attn_bwd; a NULL required gradient pointer or any overlap of an
 * output with an input, another output or the workspace is HSTU_ERR_INVALID_ARGUMENT.
 */
hstu_status_t hstu_layer_bwd(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                             const hstu_layer_weights_t *w, hstu_dtype_t dtype, hstu_dtype_t x_dtype,
                             const void *x, hstu_dtype_t grad_dtype, const void *dy, void *dx,
                             const hstu_layer_grads_t *grads, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Bytes of the saved activations that hstu_layer_fwd_save keeps for hstu_layer_bwd_saved (the
 * projection's pre-activation z, U, V, Q, K, the attention output O with its row statistics, and with
 * w->ln_output the pre-LayerNorm sum).  Depends only on host fields.
 */
size_t hstu_layer_saved_bytes(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                              const hstu_layer_weights_t *w, hstu_dtype_t dtype);

/*
 * hstu_layer_fwd that also keeps, in the caller's `saved` buffer (device, 16-byte aligned,
 * hstu_layer_saved_bytes long, no overlap with x or y), the activations its backward needs, so that
 * a training step's backward need not recompute the forward (the memory of one GPU holds them for a
 * whole stack of layers at the shipped sizes).  y is bitwise the y of hstu_layer_fwd.  The layout of
 * `saved` is private to the library.  Errors: as hstu_layer_fwd; a short `saved` is
 * HSTU_ERR_WORKSPACE_TOO_SMALL.
 */
hstu_status_t hstu_layer_fwd_save(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                  const hstu_layer_weights_t *w, hstu_dtype_t dtype, hstu_dtype_t x_dtype,
                                  const void *x, hstu_dtype_t y_dtype, void *y, void *saved, size_t saved_bytes,
                                  void *stream);

/*
 * hstu_layer_bwd reading the activations that hstu_layer_fwd_save kept in `saved` (from a call with
 * the same jag, desc, w, dtype, x_dtype and x, not modified since) instead of recomputing them.  The
 * backward works in place on them: `saved` is consumed, its contents are undefined afterwards.  The
 * workspace needs hstu_layer_bwd_workspace_bytes - hstu_layer_saved_bytes bytes.  Results are bitwise
 * those of hstu_layer_bwd.  Errors: as hstu_layer_bwd; a NULL or short `saved`, or one that overlaps
 * an input, an output or the workspace, is an error.
 */
hstu_status_t hstu_layer_bwd_saved(const hstu_jagged_t *jag, const hstu_attn_desc_t *desc,
                                   const hstu_layer_weights_t *w, hstu_dtype_t dtype, hstu_dtype_t x_dtype,
                                   const void *x, hstu_dtype_t grad_dtype, const void *dy, void *dx,
                                   const hstu_layer_grads_t *grads, void *saved, size_t saved_bytes, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * Embedding gather (input staging before the first layer):  out[t][:] = table[ids[t]][:].  Passage:
 * "DLRMv4" page, section "モデルアーキテクチャ：HSTUが従来の特徴インタラクションスタックに取って代わる"
 * -- categorical ids become vectors by an embedding lookup; section "特徴拡張：Embedding Tableが
 * 約560GBへ拡大" -- the tables those ids index (512-wide rows in the benchmark).
 * table: [table_rows][d] (device); ids: [T] int64 (device), each in [0, table_rows);
 * out: [T][d] (device).  Element type `dtype`; d * element size must be a multiple of 16 bytes.
 * An id outside [0, table_rows) reads the nearest row (0 or table_rows - 1) instead of memory past the
 * table, and the read is counted in the device's id-error word (hstu_id_errors).
 */
hstu_status_t hstu_gather_rows(const void *table, int64_t table_rows, int32_t d, hstu_dtype_t dtype,
                               const int64_t *ids, int32_t T, void *out, void *stream);

/*
 * Out-of-range row ids met by the gathers (hstu_gather_rows, and hstu_stack_fwd with ids) on the
 * current device since the library was loaded or last reset.  Not an operation of the method: the
 * gathers run asynchronously and cannot return an error for a bad id, so each read whose id lies
 * outside [0, table_rows) is clamped to the nearest row and adds 1 to a per-device word, which the
 * caller reads here when convenient.  *count (host) receives the word: 0 means no bad id; otherwise
 * the number of clamped reads (one bad id may be read several times).  Waits for `stream` first;
 * with reset != 0 the word is set back to 0.  Calls that gather concurrently on the device add to the
 * same word.  Errors: count NULL -> HSTU_ERR_INVALID_ARGUMENT; a failing HIP call -> HSTU_ERR_DEVICE.
 */
hstu_status_t hstu_id_errors(uint32_t *count, int32_t reset, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
