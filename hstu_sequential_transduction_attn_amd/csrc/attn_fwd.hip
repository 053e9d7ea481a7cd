// Jagged, causally masked pointwise attention of the HSTU layer on gfx950 (CDNA4).
//
//   O_i = c_b * sum_{allowed j} SiLU(q_i . k_j + w_p[bp(i,j)] + w_t[bt(i,j)]) v_j
//   bp = min(|pos_i - pos_j|, P-1),  bt = min(bitlen(|tau_i - tau_j|), Tb-1)
//
// Pointwise attention with a bias from the position and the time distance of two events:
// "DLRMv4：MLPerfの推薦システム訓練ベンチマークがシーケンス化時代へ", section "モデルアーキテクチャ".
// One causal block per user sequence, candidates appended at the end: same page, section
// "1つの訓練サンプルがHSTUでどのように処理されるか".  No softmax, hence no running maximum and no
// normaliser: partial sums over key tiles simply add.
//
// Kernel shape.  A workgroup is 4 waves; each wave owns 32 consecutive queries of one (sequence, head),
// so a workgroup covers 128 queries.  Key tiles of 64 rows are staged through LDS (double buffered,
// one barrier per tile) and shared by the 4 waves.  Both contractions run on 32x32 MFMA tiles in a
// transposed form:
//     S^T[key][query] = K . Q^T        (A = K rows from LDS, B = Q held in registers)
//     O^T[dh][query] += V^T . P^T      (A = V^T read with ds_read_b64_tr_b16, B = P from registers)
// The score accumulator of the first product is already laid out as the B operand of the second:
// lane l always holds query l%32.  K rows are stored in LDS in a permuted order so that the keys a
// lane holds in its 16 accumulator values are two runs of 8 consecutive keys, which is exactly the
// k-order the second MFMA expects.  V stays in its natural [key][dh] layout; the transpose read hands
// each lane 4 consecutive keys of one dh column.
//
// Bias and mask.  Per (wave, key tile) the work is classified from index ranges and from timestamp
// ranges (per-32-token minimum and maximum, computed by a small prologue kernel):
//   none      - no allowed pair: skipped;
//   uniform   - every pair allowed, one position bucket and one time bucket: a single bias constant;
//   two       - every pair allowed, one position bucket, the time bucket is one of two adjacent
//               buckets and the timestamps span less than 2^32: |tau_i - tau_j| from 32-bit offsets
//               (v_sad_u32), one compare and one select per score;
//   general   - per-score mask and bucket lookups in LDS (32-bit offsets when the span allows,
//               exact 64-bit differences otherwise).
// Each class has its own branch-free body; the two score blocks of a tile are ordered so that one
// block's SiLU work overlaps the other's MFMAs.
#include "device_common.hpp"
#include "kernels.h"

namespace hstu {
namespace {

constexpr int kWaves = 4;
constexpr int kQW = 32;                  // queries per wave
constexpr int kBM = kWaves * kQW;        // queries per workgroup
constexpr int kBN = 64;                  // keys per LDS tile
constexpr int kThreads = kWaves * kWave;
constexpr int kTimeTab = 65;             // a 64-bit gap has bit length 0..64
constexpr int kChunk = 32;               // tokens per timestamp-range chunk

enum Mode : int { kUniform = 0, kTwo = 1, kGen32 = 2, kGen64 = 3 };

// Row order of K inside each 32-row block of LDS: row r holds key kperm(r) (an involution swapping
// rows 4..7 with 8..11 and 20..23 with 24..27).  With it, accumulator element e of lane half hf holds
// key 16*(e/8) + 8*hf + e%8.
__device__ __forceinline__ int kperm(int r) {
  const int g = (r >> 2) & 7;
  const int ng = (g == 1) ? 2 : (g == 2) ? 1 : (g == 5) ? 6 : (g == 6) ? 5 : g;
  return (r & ~31) | (ng << 2) | (r & 3);
}

template <typename T, int DH>
struct Layout {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kES = sizeof(T);
  static constexpr int kKStride = kBf16 ? DH * 2 + 16 : (DH + 1) * 4;   // bytes per K row in LDS
  static constexpr int kVStride = kBf16 ? DH * 2 + 32 : DH * 4;         // bytes per V row in LDS
  static constexpr int kChunksPerRow = DH * kES / 16;
  static constexpr int kChunksPerThread = kBN * kChunksPerRow / kThreads;
  static constexpr int kOffK = 0;
  static constexpr int kOffV = kOffK + kBN * kKStride;
  static constexpr int kOffTauLo = (kOffV + kBN * kVStride + 15) & ~15;
  static constexpr int kOffTauHi = kOffTauLo + kBN * 4;
  static constexpr int kStageBytes = kOffTauHi + kBN * 4;
  static constexpr int kKPL = kBf16 ? 8 : 1;                 // operand values per lane per MFMA
  static constexpr int kKStep = kBf16 ? 16 : 2;              // k per MFMA
  static constexpr int kQSteps = DH / kKStep;                // MFMAs per 32x32 score block
  static constexpr int kDB = DH / 32;                        // 32-row dh blocks of O^T
  static_assert(kChunksPerThread >= 1 && kBN * kChunksPerRow % kThreads == 0, "staging split");
  static_assert(kStageBytes % 16 == 0, "stage alignment");
};

// The O^T accumulators of one wave: N blocks of 32 dh rows x 32 queries.
template <int N>
struct OAcc {
  floatx16 d[N];
};

template <typename T> struct QFrag;
template <> struct QFrag<__bf16> { using type = bf16x8; };
template <> struct QFrag<float> { using type = float; };

__device__ __forceinline__ int bitlen_u64(uint64_t d) { return d == 0 ? 0 : 64 - __clzll((long long)d); }
__device__ __forceinline__ int bitlen_u32(uint32_t d) { return 32 - __clz((int)d); }  // __clz(0) = 32

// Per-wave constants of the score pointwise work for one tile.
struct TileCtx {
  int k0;              // first key of the tile (sequence-local)
  int my_q, my_pos;    // this lane's query and its position
  int n, nh;           // sequence length, history length
  bool cand;
  int P, Tb;
  int64_t my_tau;
  uint32_t qoff;       // (uint32)(my_tau - base) for the 32-bit modes
  uint32_t base_lo;    // low word of the tile's timestamp base
  uint32_t thr;        // two-bucket mode: |dt| >= thr selects bias_hi
  float cbias, bias_lo, bias_hi;
  const HSTU_LDS float *wp, *wt;
  const HSTU_LDS uint32_t *tlo, *thi;   // the tile's timestamps, low and high words
};

// SiLU(score + bias) for the 16 scores of one 32-key block kb; element e holds key
// k0 + 32*kb + 16*(e/8) + 8*half + e%8.
template <int MODE, bool MASKED>
__device__ __forceinline__ void pointwise(const floatx16 &s, float (&a)[16], const TileCtx &c, int kb, int half) {
  if constexpr (MODE == kUniform) {
#pragma unroll
    for (int e = 0; e < 16; ++e) a[e] = silu_f32(s[e] + c.cbias);
  } else {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int jl0 = 32 * kb + 16 * g + 8 * half;   // tile-local key of element 8*g
      uint32_t lo[8], hi[8];
      {
        const u32x4 l0 = *(const HSTU_LDS u32x4 *)(c.tlo + jl0), l1 = *(const HSTU_LDS u32x4 *)(c.tlo + jl0 + 4);
        lo[0] = l0.x; lo[1] = l0.y; lo[2] = l0.z; lo[3] = l0.w; lo[4] = l1.x; lo[5] = l1.y; lo[6] = l1.z; lo[7] = l1.w;
      }
      if constexpr (MODE == kGen64) {
        const u32x4 h0 = *(const HSTU_LDS u32x4 *)(c.thi + jl0), h1 = *(const HSTU_LDS u32x4 *)(c.thi + jl0 + 4);
        hi[0] = h0.x; hi[1] = h0.y; hi[2] = h0.z; hi[3] = h0.w; hi[4] = h1.x; hi[5] = h1.y; hi[6] = h1.z; hi[7] = h1.w;
      }
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const int e = 8 * g + e8;
        float bias;
        if constexpr (MODE == kTwo) {
          const uint32_t d = __usad(c.qoff, lo[e8] - c.base_lo, 0u);
          bias = d >= c.thr ? c.bias_hi : c.bias_lo;
        } else {
          const int j = c.k0 + jl0 + e8;
          const int pj = c.cand ? imin(j, c.nh) : j;
          const uint32_t dp = __usad((uint32_t)c.my_pos, (uint32_t)pj, 0u);
          const int bp = (int)(dp < (uint32_t)(c.P - 1) ? dp : (uint32_t)(c.P - 1));
          int bt;
          if constexpr (MODE == kGen32) {
            bt = bitlen_u32(__usad(c.qoff, lo[e8] - c.base_lo, 0u));
          } else {
            const int64_t tj = (int64_t)(((uint64_t)hi[e8] << 32) | lo[e8]);
            bt = bitlen_absdiff(c.my_tau, tj);
          }
          bt = imin(bt, c.Tb - 1);
          bias = c.wp[bp] + c.wt[bt];
        }
        const float v = silu_f32(s[e] + bias);
        if constexpr (MASKED) {
          const int j = c.k0 + jl0 + e8;
          const bool ok = j < c.n && (c.my_q < c.nh ? j <= c.my_q : (j < c.nh || j == c.my_q));
          a[e] = ok ? v : 0.0f;
        } else {
          a[e] = v;
        }
      }
    }
  }
}

template <typename T, int DH>
__device__ __forceinline__ void score_block(floatx16 &s, const HSTU_LDS char *lK, int kb, int l32, int half,
                                            const typename QFrag<T>::type (&qf)[Layout<T, DH>::kQSteps]) {
  using L = Layout<T, DH>;
  s = floatx16{};
#pragma unroll
  for (int st = 0; st < L::kQSteps; ++st) {
    if constexpr (L::kBf16) {
      const bf16x8 kf = *(const HSTU_LDS bf16x8 *)(lK + (32 * kb + l32) * L::kKStride + (16 * st + 8 * half) * 2);
      s = mfma32(kf, qf[st], s);
    } else {
      const float kf = *(const HSTU_LDS float *)(lK + (32 * kb + l32) * L::kKStride + (2 * st + half) * 4);
      s = mfma32(kf, qf[st], s);
    }
  }
}

template <typename T, int DH>
__device__ __forceinline__ void av_block(OAcc<Layout<T, DH>::kDB> &oacc, const float (&a)[16],
                                         const HSTU_LDS char *lV, int kb, int lane) {
  using L = Layout<T, DH>;
  const int l32 = lane & 31, half = lane >> 5;
  if constexpr (L::kBf16) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = f32_to_bf16(a[8 * s2 + e]);
      const int g16 = lane >> 4, i16 = lane & 15;
      const int krow = 32 * kb + 16 * s2 + 8 * half + (i16 >> 2);
#pragma unroll
      for (int db = 0; db < L::kDB; ++db) {
        const int col = 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3);
        const shortx4 v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((HSTU_LDS shortx4 *)(lV + krow * L::kVStride + col * 2));
        const shortx4 v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((HSTU_LDS shortx4 *)(lV + (krow + 4) * L::kVStride + col * 2));
        const bf16x4 w0 = __builtin_bit_cast(bf16x4, v0), w1 = __builtin_bit_cast(bf16x4, v1);
        bf16x8 vf;
        vf[0] = w0[0]; vf[1] = w0[1]; vf[2] = w0[2]; vf[3] = w0[3];
        vf[4] = w1[0]; vf[5] = w1[1]; vf[6] = w1[2]; vf[7] = w1[3];
        oacc.d[db] = mfma32(vf, pf, oacc.d[db]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int krow = 32 * kb + 16 * (e / 8) + 8 * half + (e % 8);
#pragma unroll
      for (int db = 0; db < L::kDB; ++db) {
        const float vf = *(const HSTU_LDS float *)(lV + krow * L::kVStride + (32 * db + l32) * 4);
        oacc.d[db] = mfma32(vf, a[e], oacc.d[db]);
      }
    }
  }
}

// One key tile for one wave: both score blocks, then pointwise and AV for each.
template <typename T, int DH, int MODE, bool MASKED>
__device__ __forceinline__ void tile_body(OAcc<Layout<T, DH>::kDB> &oacc,
                                          const typename QFrag<T>::type (&qf)[Layout<T, DH>::kQSteps],
                                          const HSTU_LDS char *lK, const HSTU_LDS char *lV, const TileCtx &c,
                                          int lane) {
  const int l32 = lane & 31, half = lane >> 5;
  floatx16 s0, s1;
  score_block<T, DH>(s0, lK, 0, l32, half, qf);
  score_block<T, DH>(s1, lK, 1, l32, half, qf);
  float a[16];
  pointwise<MODE, MASKED>(s0, a, c, 0, half);
  av_block<T, DH>(oacc, a, lV, 0, lane);
  pointwise<MODE, MASKED>(s1, a, c, 1, half);
  av_block<T, DH>(oacc, a, lV, 1, lane);
}

// Timestamp minimum and maximum of every 32-token chunk of every sequence.  Chunk c of sequence b is
// stored at index (o_b >> 5) + b + c, which never collides across sequences (at most T/32 + B + 1
// entries).  One workgroup per sequence.
__global__ void __launch_bounds__(256) tau_chunk_stats_kernel(const int32_t *__restrict__ offs,
                                                              const int64_t *__restrict__ tau,
                                                              int64_t *__restrict__ stats) {
  const int b = blockIdx.x;
  const int o0 = offs[b], n = offs[b + 1] - o0;
  const int nc = (n + kChunk - 1) / kChunk;
  const int base = (o0 >> 5) + b;
  for (int c = threadIdx.x; c < nc; c += blockDim.x) {
    int64_t mn = INT64_MAX, mx = INT64_MIN;
    const int e = imin(kChunk, n - kChunk * c);
    for (int i = 0; i < e; ++i) {
      const int64_t t = tau[o0 + kChunk * c + i];
      mn = t < mn ? t : mn;
      mx = t > mx ? t : mx;
    }
    stats[2 * (int64_t)(base + c)] = mn;
    stats[2 * (int64_t)(base + c) + 1] = mx;
  }
}

// Two waves per SIMD (<= 256 registers per lane) so that one wave's MFMAs overlap the other's VALU work.
template <typename T, int DH, typename TO>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const AttnArgs p, const int n_qblocks) {
  using L = Layout<T, DH>;
  using Frag = typename QFrag<T>::type;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  HSTU_LDS char *smem = (HSTU_LDS char *)smem_raw;

  // ---- work item: query block major (longest first), then (sequence, head)
  const int HB = p.num_heads * p.num_seqs;
  const int item = blockIdx.x;
  const int qblk = n_qblocks - 1 - item / HB;
  const int b = (item % HB) / p.num_heads;
  const int h = (item % HB) % p.num_heads;
  const int o0 = p.seq_offsets[b];
  const int n = p.seq_offsets[b + 1] - o0;
  const int q0 = qblk * kBM;
  if (q0 >= n) return;  // uniform over the workgroup
  const bool cand = p.mask == kCausalCandidates;
  const int nh = cand ? n - p.num_candidates[b] : n;
  const float cb = p.attn_scale ? p.attn_scale[b] : 1.0f / (float)n;
  const int P = p.num_pos_buckets;
  const int Tb = p.num_time_buckets;
  const int rr = p.rab_rows == 1 ? 0 : h;
  const int64_t *cstats = p.tau_stats + 2 * (int64_t)((o0 >> 5) + b);   // chunk c at cstats[2c], [2c+1]

  const int tid = threadIdx.x;
  // wave index as a scalar: everything derived from it (query range, tile classes) stays wave-uniform,
  // so the per-tile class selects one body with a scalar branch instead of predicating all of them
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- bias tables into LDS (after the two pipeline stages)
  HSTU_LDS float *wp_lds = (HSTU_LDS float *)(smem + 2 * L::kStageBytes);
  HSTU_LDS float *wt_lds = wp_lds + P;
  for (int i = tid; i < P; i += kThreads) wp_lds[i] = p.pos_bias[(int64_t)rr * P + i];
  const int nt_tab = imin(Tb, kTimeTab);
  for (int i = tid; i < nt_tab; i += kThreads) wt_lds[i] = p.time_bias[(int64_t)rr * Tb + i];

  // ---- this wave's queries
  const int qa = q0 + wave * kQW;                 // first query of the wave (a multiple of 32)
  const int ql = imin(qa + kQW - 1, n - 1);       // last valid query of the wave
  const bool wave_active = qa < n;
  const int my_q = qa + l32;
  const bool my_valid = my_q < n;
  const int64_t my_tau = my_valid ? p.timestamps[o0 + my_q] : 0;
  const int64_t wmin = wave_active ? cstats[2 * (qa >> 5)] : 0;
  const int64_t wmax = wave_active ? cstats[2 * (qa >> 5) + 1] : 0;

  // Q fragments (B operand of S^T = K Q^T): lane holds query l32, dh = kKStep*s + kKPL*half + [0, kKPL)
  Frag qf[L::kQSteps];
  {
    const T *qrow = (const T *)p.q + (int64_t)(o0 + (my_valid ? my_q : 0)) * p.row_stride + h * DH;
#pragma unroll
    for (int s = 0; s < L::kQSteps; ++s) {
      if constexpr (L::kBf16) {
        bf16x8 v = *(const bf16x8 *)(qrow + s * 16 + half * 8);
        if (!my_valid) v = bf16x8{};
        qf[s] = v;
      } else {
        qf[s] = my_valid ? qrow[s * 2 + half] : 0.0f;
      }
    }
  }

  // ---- key tiles needed by the workgroup: [0, r1_end) and, for candidate rows, their own tiles
  const int blast = imin(q0 + kBM - 1, n - 1);
  const int r1_end = (imin(blast + 1, nh) + kBN - 1) / kBN;
  int r2_begin = 0, r2_end = 0;
  if (blast >= nh) {
    r2_begin = imax(imax(q0, nh) / kBN, r1_end);
    r2_end = blast / kBN + 1;
  }
  auto next_tile = [&](int t) -> int {
    ++t;
    if (t < r1_end) return t;
    if (t < r2_begin) t = r2_begin;
    return t < r2_end ? t : -1;
  };
  int tile = r1_end > 0 ? 0 : (r2_begin < r2_end ? r2_begin : -1);

  // ---- staging of one key tile: global -> registers -> LDS
  u32x4 kreg[L::kChunksPerThread], vreg[L::kChunksPerThread];
  int64_t treg = 0;
  auto load_tile = [&](int t) {
    const int k0 = t * kBN;
#pragma unroll
    for (int c = 0; c < L::kChunksPerThread; ++c) {
      const int chunk = tid + c * kThreads;
      const int row = chunk / L::kChunksPerRow, col = chunk % L::kChunksPerRow;
      const bool ok = k0 + row < n;
      const int64_t off = (int64_t)(o0 + (ok ? k0 + row : 0)) * p.row_stride * L::kES + (int64_t)h * DH * L::kES +
                          col * 16;
      const u32x4 kv = *(const u32x4 *)((const char *)p.k + off);
      const u32x4 vv = *(const u32x4 *)((const char *)p.v + off);
      kreg[c] = ok ? kv : u32x4{0u, 0u, 0u, 0u};
      vreg[c] = ok ? vv : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < kBN) treg = (k0 + tid < n) ? p.timestamps[o0 + k0 + tid] : 0;
  };
  auto store_tile = [&](int stage) {
    HSTU_LDS char *base = smem + stage * L::kStageBytes;
#pragma unroll
    for (int c = 0; c < L::kChunksPerThread; ++c) {
      const int chunk = tid + c * kThreads;
      const int row = chunk / L::kChunksPerRow, col = chunk % L::kChunksPerRow;
      HSTU_LDS char *kdst = base + L::kOffK + kperm(row) * L::kKStride + col * 16;
      if constexpr (L::kBf16) {
        *(HSTU_LDS u32x4 *)kdst = kreg[c];
      } else {
        HSTU_LDS uint32_t *d = (HSTU_LDS uint32_t *)kdst;
        d[0] = kreg[c].x; d[1] = kreg[c].y; d[2] = kreg[c].z; d[3] = kreg[c].w;
      }
      *(HSTU_LDS u32x4 *)(base + L::kOffV + row * L::kVStride + col * 16) = vreg[c];
    }
    if (tid < kBN) {
      ((HSTU_LDS uint32_t *)(base + L::kOffTauLo))[tid] = (uint32_t)(uint64_t)treg;
      ((HSTU_LDS uint32_t *)(base + L::kOffTauHi))[tid] = (uint32_t)((uint64_t)treg >> 32);
    }
  };

  OAcc<L::kDB> oacc;
#pragma unroll
  for (int d = 0; d < L::kDB; ++d) oacc.d[d] = floatx16{};

  TileCtx c;
  c.my_q = my_q;
  c.my_pos = cand ? imin(my_q, nh) : my_q;
  c.n = n;
  c.nh = nh;
  c.cand = cand;
  c.P = P;
  c.Tb = Tb;
  c.my_tau = my_tau;
  c.wp = wp_lds;
  c.wt = wt_lds;

  int stage = 0;
  if (tile >= 0) {
    load_tile(tile);
    store_tile(0);
  }
  __syncthreads();

  while (tile >= 0) {
    const int nxt = next_tile(tile);
    if (nxt >= 0) load_tile(nxt);
    const HSTU_LDS char *base = smem + stage * L::kStageBytes;
    const int k0 = tile * kBN;

    const bool none = !wave_active || k0 > ql || (k0 >= nh && (k0 + kBN - 1 < imax(qa, nh)));
    if (!none) {
      // timestamp range of the tile's valid keys
      const int c0 = k0 >> 5;
      int64_t kmin = cstats[2 * c0], kmax = cstats[2 * c0 + 1];
      if (k0 + kChunk < n) {
        const int64_t a = cstats[2 * c0 + 2], bb = cstats[2 * c0 + 3];
        kmin = a < kmin ? a : kmin;
        kmax = bb > kmax ? bb : kmax;
      }
      const int64_t tmin = wmin < kmin ? wmin : kmin;
      const int64_t tmax = wmax > kmax ? wmax : kmax;
      const uint64_t span = (uint64_t)tmax - (uint64_t)tmin;
      c.k0 = k0;
      c.tlo = (const HSTU_LDS uint32_t *)(base + L::kOffTauLo);
      c.thi = (const HSTU_LDS uint32_t *)(base + L::kOffTauHi);
      c.base_lo = (uint32_t)(uint64_t)tmin;
      c.qoff = (uint32_t)(uint64_t)my_tau - c.base_lo;
      const HSTU_LDS char *lK = base + L::kOffK;
      const HSTU_LDS char *lV = base + L::kOffV;

      const bool all = (k0 + kBN - 1 <= qa) && (k0 + kBN - 1 < nh);
      int mode = span < (1ull << 32) ? kGen32 : kGen64;
      if (all && imin(qa, nh) - (k0 + kBN - 1) >= P - 1) {
        uint64_t lo, hi;
        if (wmin >= kmax) {
          lo = (uint64_t)wmin - (uint64_t)kmax;
          hi = (uint64_t)wmax - (uint64_t)kmin;
        } else if (kmin >= wmax) {
          lo = (uint64_t)kmin - (uint64_t)wmax;
          hi = (uint64_t)kmax - (uint64_t)wmin;
        } else {
          lo = 0;
          hi = span;
        }
        const int blo = imin(bitlen_u64(lo), Tb - 1);
        const int bhi = imin(bitlen_u64(hi), Tb - 1);
        const float wpc = wp_lds[P - 1];
        if (blo == bhi) {
          mode = kUniform;
          c.cbias = wpc + wt_lds[blo];
        } else if (bhi == blo + 1 && span < (1ull << 32)) {
          mode = kTwo;
          c.thr = 1u << (bhi - 1);
          c.bias_lo = wpc + wt_lds[blo];
          c.bias_hi = wpc + wt_lds[bhi];
        }
      }
      if (all) {
        if (mode == kUniform) tile_body<T, DH, kUniform, false>(oacc, qf, lK, lV, c, lane);
        else if (mode == kTwo) tile_body<T, DH, kTwo, false>(oacc, qf, lK, lV, c, lane);
        else if (mode == kGen32) tile_body<T, DH, kGen32, false>(oacc, qf, lK, lV, c, lane);
        else tile_body<T, DH, kGen64, false>(oacc, qf, lK, lV, c, lane);
      } else {
        if (mode == kGen32) tile_body<T, DH, kGen32, true>(oacc, qf, lK, lV, c, lane);
        else tile_body<T, DH, kGen64, true>(oacc, qf, lK, lV, c, lane);
      }
    }

    if (nxt >= 0) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    tile = nxt;
  }

  // ---- epilogue: O^T element e of dh block db is dh = 32*db + 8*(e/4) + 4*half + e%4
  if (my_valid) {
    TO *orow = (TO *)p.out + (int64_t)(o0 + my_q) * p.out_row_stride + h * DH;
#pragma unroll
    for (int db = 0; db < L::kDB; ++db) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int dh = 32 * db + 8 * e4 + 4 * half;
        if constexpr (sizeof(TO) == 4) {
          floatx4 w;
          w[0] = oacc.d[db][4 * e4 + 0] * cb; w[1] = oacc.d[db][4 * e4 + 1] * cb;
          w[2] = oacc.d[db][4 * e4 + 2] * cb; w[3] = oacc.d[db][4 * e4 + 3] * cb;
          *(floatx4 *)(orow + dh) = w;
        } else {
          bf16x4 w;
          w[0] = f32_to_bf16(oacc.d[db][4 * e4 + 0] * cb); w[1] = f32_to_bf16(oacc.d[db][4 * e4 + 1] * cb);
          w[2] = f32_to_bf16(oacc.d[db][4 * e4 + 2] * cb); w[3] = f32_to_bf16(oacc.d[db][4 * e4 + 3] * cb);
          *(bf16x4 *)(orow + dh) = w;
        }
      }
    }
  }
}

template <typename T, int DH, typename TO>
hipError_t launch_typed(const AttnArgs &a, hipStream_t stream) {
  using L = Layout<T, DH>;
  const int n_qblocks = (a.max_seq_len + kBM - 1) / kBM;
  const long long grid = (long long)n_qblocks * a.num_heads * a.num_seqs;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = 2 * L::kStageBytes + (size_t)(a.num_pos_buckets + kTimeTab) * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)attn_fwd_kernel<T, DH, TO>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(tau_chunk_stats_kernel, dim3(a.num_seqs), dim3(256), 0, stream, a.seq_offsets, a.timestamps,
                     a.tau_stats);
  hipLaunchKernelGGL((attn_fwd_kernel<T, DH, TO>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a, n_qblocks);
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_dh(const AttnArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 32: return launch_typed<T, 32, TO>(a, stream);
    case 64: return launch_typed<T, 64, TO>(a, stream);
    case 128: return launch_typed<T, 128, TO>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t attn_tau_stats_bytes(int64_t total_tokens, int64_t num_seqs) {
  return (size_t)((total_tokens >> 5) + num_seqs + 1) * 2 * sizeof(int64_t);
}

hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t stream) {
  if (a.in_dtype == kBF16) {
    return a.out_dtype == kBF16 ? launch_dh<__bf16, __bf16>(a, stream) : launch_dh<__bf16, float>(a, stream);
  }
  return launch_dh<float, float>(a, stream);
}

}  // namespace hstu
