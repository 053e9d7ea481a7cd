// Backward of the pointwise attention, key-major pass: dK and dV.
//
// For the forward O_i = c_b sum_j SiLU(s_ij) v_j (s_ij = q_i . k_j + bias, allowed pairs only) and an
// upstream gradient dO:
//   dv_j = c_b sum_i SiLU(s_ij) dO_i,    dk_j = c_b sum_i dP_ij SiLU'(s_ij) q_i,   dP_ij = dO_i . v_j.
// The bias and the masks are those of the forward ("DLRMv4：MLPerfの推薦システム訓練ベンチマークがシー
// ケンス化時代へ", sections "モデルアーキテクチャ" and "1つの訓練サンプルがHSTUでどのように処理されるか").
// No softmax: no row statistics are needed and every pair's gradient is local.
//
// Kernel shape.  A workgroup is 4 waves; wave w owns 32 consecutive keys of one (sequence, head), held
// in registers as the B operands of S = Q K^T and dP = dO V^T, so every product of a query tile lands
// with lane l on key l % 32 and each lane's 16 values per 32-query block on the queries that the next
// MFMA's k order expects (Q and dO rows are read in the kperm order, as K rows are in the forward).
// Query tiles of 64 rows (Q, dO and their timestamps) go global -> LDS with direct-to-LDS loads, both
// in the forward's K layout, so their rows feed S and dP and their transposed reads feed
//   dV^T += dO^T A   and   dK^T += Q^T dS     (A = SiLU(s), dS = dP SiLU'(s)).
// A key sees the queries i >= j (a history key also every candidate; a candidate key only itself), so
// the tiles run from the key block's first row to the end of the sequence.  Each wave classifies each
// tile in scalar code: none, uniform (one bias for every pair), or general (per-score bias and mask).
// bf16 runs two waves per SIMD: the keys' K and V and the dK^T and dV^T accumulators fill most of the
// 256 registers, and the loop keeps nothing else across tiles that can be rebuilt (see KeyCtx), so
// nothing spills (a reload from scratch would also wait for the next tile's direct-to-LDS prefetch).
#include "attn_common.hpp"
#include "work_order.hpp"

namespace hstu {
namespace {

using namespace attn;

// Per-wave constants of the per-score bias and mask of a general tile (roles of the forward's
// TileCtx with queries and keys exchanged: the lane's key is fixed, the tile's queries vary).  The
// lane's own key values (position, allowed queries, timestamp) are rebuilt from the lane index and
// the wave's key timestamps in LDS where a general tile needs them: held in registers for the whole
// loop, they pushed the two-waves-per-SIMD register budget into spills.
struct KeyCtx {
  int q0;              // first query of the tile (sequence-local)
  int ka;              // first key of the wave
  int n, nh;           // sequence length; history length (n without candidates)
  int pos_lim;         // position of query i is min(i, pos_lim)
  int P, Tb;
  const HSTU_LDS int64_t *ktau;    // the wave's 32 key timestamps
  const HSTU_LDS float *wp, *wt;
  const HSTU_LDS char *stage;
  uint32_t base_lo;    // 32-bit mode: low word of the tile's smallest timestamp (all within 2^32 of it)
  uint32_t thr;        // two-bucket tiles: |dt| >= thr takes bias_hi
  float bias_lo, bias_hi;
};

// Bias (and mask) of the 16 scores of 32-query block qb in place; element e holds query
// q0 + 32*qb + 16*(e/8) + 8*half + e%8.
// K32: every timestamp of the tile lies within 2^32 of c.base_lo's full value, so each |dt| is the
// distance of two 32-bit offsets from it (one v_sad_u32) instead of a 64-bit difference.
template <typename T, int DH, bool MASKED, bool K32>
__device__ __forceinline__ void adjust_block_keys(floatx16 &s, const KeyCtx &c, int qb, int lane) {
  using L = Layout<T, DH>;
  const int half = lane >> 5;
  const int my_k = c.ka + (lane & 31);
  const int my_pos = imin(my_k, c.pos_lim);      // a candidate key sits at position nh
  const int q_hi = my_k < c.nh ? c.n - 1 : my_k;  // allowed queries: my_k <= i <= q_hi
  const int64_t my_tau = c.ktau[lane & 31];
  const uint32_t koff = (uint32_t)(uint64_t)my_tau - c.base_lo;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int il0 = 32 * qb + 16 * g + 8 * half;
    int64_t ti[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w = *(const HSTU_LDS u32x4 *)(c.stage + L::tau_at(il0 + 2 * q));
      ti[2 * q] = (int64_t)(((uint64_t)w.y << 32) | w.x);
      ti[2 * q + 1] = (int64_t)(((uint64_t)w.w << 32) | w.z);
    }
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const int e = 8 * g + e8;
      const int i = c.q0 + il0 + e8;
      const int pi = imin(i, c.pos_lim);
      const uint32_t dp = __usad((uint32_t)pi, (uint32_t)my_pos, 0u);
      const int bp = (int)(dp < (uint32_t)(c.P - 1) ? dp : (uint32_t)(c.P - 1));
      const int bt = imin(K32 ? bitlen_u32(__usad(koff, (uint32_t)(uint64_t)ti[e8] - c.base_lo, 0u))
                              : bitlen_absdiff(ti[e8], my_tau), c.Tb - 1);
      const float bias = c.wp[bp] + c.wt[bt];
      if constexpr (MASKED) {
        const bool ok = (i >= my_k) & (i <= q_hi);
        s[e] = ok ? s[e] + bias : kMaskedScore;
      } else {
        s[e] = s[e] + bias;
      }
    }
  }
}

// Bias of the 16 scores of 32-query block qb in a two-bucket tile: every pair is allowed and clamped to
// position bucket P - 1, and |dt| falls in time bucket blo or blo + 1, told apart by |dt| >= 2^blo; the
// gaps come from 32-bit offsets of the tile's smallest timestamp (one v_sad_u32 per score).
template <typename T, int DH>
__device__ __forceinline__ void adjust_block_keys_two(floatx16 &s, const KeyCtx &c, int qb, int lane) {
  using L = Layout<T, DH>;
  const int half = lane >> 5;
  const uint32_t koff = (uint32_t)(uint64_t)c.ktau[lane & 31] - c.base_lo;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int il0 = 32 * qb + 16 * g + 8 * half;
    uint32_t lo[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w = *(const HSTU_LDS u32x4 *)(c.stage + L::tau_at(il0 + 2 * q));
      lo[2 * q] = w.x;
      lo[2 * q + 1] = w.z;
    }
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8)
      s[8 * g + e8] += __usad(koff, lo[e8] - c.base_lo, 0u) >= c.thr ? c.bias_hi : c.bias_lo;
  }
}

// One 32-query block of a tile for one wave.  body: kUniform (bias c1 folded into the exponent), kTwo
// (two time buckets), kGen32/kGen64 (per-score bias), kGen32M/kGen64M (per-score bias and mask).  Every class shares one copy of the MFMA
// code, so the dK^T and dV^T accumulators stay in the same registers whatever the class.
template <typename T, int DH>
__device__ __forceinline__ void dkdv_block(OAcc<Layout<T, DH>::kDB> &dk, OAcc<Layout<T, DH>::kDB> &dv,
                                           const typename QFrag<T>::type (&kf)[Layout<T, DH>::kQSteps],
                                           const typename QFrag<T>::type (&vf)[Layout<T, DH>::kQSteps],
                                           const KeyCtx &c, int body, float c1, int qb, int lane) {
  using L = Layout<T, DH>;
  const int l32 = lane & 31, half = lane >> 5;
  const HSTU_LDS char *lQ = c.stage + L::kOffK;
  const HSTU_LDS char *lG = c.stage + L::kOffV;
  floatx16 s;
  score_block<T, DH>(s, lQ, qb, l32, half, kf);
  if (body == kTwo) adjust_block_keys_two<T, DH>(s, c, qb, lane);
  else if (body == kGen32) adjust_block_keys<T, DH, false, true>(s, c, qb, lane);
  else if (body == kGen32M) adjust_block_keys<T, DH, true, true>(s, c, qb, lane);
  else if (body == kGen64) adjust_block_keys<T, DH, false, false>(s, c, qb, lane);
  else if (body == kGen64M) adjust_block_keys<T, DH, true, false>(s, c, qb, lane);
  // A = SiLU(x) and SiLU'(x) from S, then dV; dP only after that, so that S, A and dP are never all
  // live at once (at two waves per SIMD the registers are the limit)
  float a[16], gd[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float u = fmaf(s[e], kNegLog2e, c1);             // -log2(e) x, x = s + bias
    const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u));
    const float x = u * kNegLn2;
    a[e] = x * sig;                                         // SiLU(x); 0 for a masked score
    gd[e] = sig * fmaf(x, 1.0f - sig, 1.0f);                // SiLU'(x)
  }
  if constexpr (L::kBf16) {
    bf16x8 pa[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) pa[e / 8][e % 8] = f32_to_bf16(a[e]);
    av_block_packed<DH, true>(dv, pa, lG, qb, lane);
  } else {
    av_block_in<T, DH, true>(dv, a, lG, qb, lane);
  }
  floatx16 dp;
  score_block<T, DH>(dp, lG, qb, l32, half, vf);
  float ds[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) ds[e] = dp[e] * gd[e];      // dP SiLU'(x)
  if constexpr (L::kBf16) {
    bf16x8 pd[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) pd[e / 8][e % 8] = f32_to_bf16(ds[e]);
    av_block_packed<DH, true>(dk, pd, lQ, qb, lane);
  } else {
    av_block_in<T, DH, true>(dk, ds, lQ, qb, lane);
  }
}

template <typename T, int DH>
__device__ __forceinline__ void dkdv_tile(OAcc<Layout<T, DH>::kDB> &dk, OAcc<Layout<T, DH>::kDB> &dv,
                                          const typename QFrag<T>::type (&kf)[Layout<T, DH>::kQSteps],
                                          const typename QFrag<T>::type (&vf)[Layout<T, DH>::kQSteps],
                                          const KeyCtx &c, int body, float c1, int lane) {
  dkdv_block<T, DH>(dk, dv, kf, vf, c, body, c1, 0, lane);
  dkdv_block<T, DH>(dk, dv, kf, vf, c, body, c1, 1, lane);
}

__device__ __forceinline__ int64_t smin64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t smax64(int64_t a, int64_t b) { return a > b ? a : b; }

// bf16: two waves per SIMD (<= 256 registers, none spilled at Dh = 128); fp32 operands take twice the
// fragment registers and run one wave per SIMD.
template <typename T, int DH>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, sizeof(T) == 2 ? 2 : 1)))
attn_bwd_dkdv_kernel(const AttnArgs p, const int n_kblocks) {
  using L = Layout<T, DH>;
  using Frag = typename QFrag<T>::type;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  HSTU_LDS char *smem = (HSTU_LDS char *)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  // ---- work item: the XCD-local order of work_order.hpp; rank 0 is the first key block (it sees the
  // most queries)
  const int HB = p.num_heads * p.num_seqs;
  const WorkItem wi = work_item((int)blockIdx.x, HB, n_kblocks);
  const int kblk = wi.rank;
  const int b = wi.pair / p.num_heads;
  const int h = wi.pair % p.num_heads;
  const int o0 = p.seq_offsets[b];
  const int n = p.seq_offsets[b + 1] - o0;
  const int k0 = kblk * kBM;
  if (k0 >= n) return;
  const bool cand = p.mask == kCausalCandidates;
  const int nh = cand ? n - p.num_candidates[b] : n;
  const float cb = p.attn_scale ? p.attn_scale[b] : 1.0f / (float)n;
  const int P = p.num_pos_buckets, Tb = p.num_time_buckets;
  const int rr = p.rab_rows == 1 ? 0 : h;
  const int64_t *stats = p.tau_stats + 2 * (int64_t)((o0 >> 5) + b);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane & 31, half = lane >> 5;

  HSTU_LDS int64_t *ktau_lds = (HSTU_LDS int64_t *)(smem + L::kStages * L::kStageBytes);
  HSTU_LDS float *wp_lds = (HSTU_LDS float *)(ktau_lds + kBM);
  HSTU_LDS float *wt_lds = wp_lds + P;
  for (int i = tid; i < P; i += kThreads) wp_lds[i] = p.pos_bias[(int64_t)rr * P + i];
  const int nt_tab = imin(Tb, kTimeTab);
  for (int i = tid; i < nt_tab; i += kThreads) wt_lds[i] = p.time_bias[(int64_t)rr * Tb + i];

  // ---- this wave's keys
  const int ka = k0 + wave * kQW;                 // first key of the wave (a multiple of 32)
  const int kl = imin(ka + kQW - 1, n - 1);       // last valid key
  const bool wave_active = ka < n;
  const int my_k = ka + l32;
  const bool my_valid = my_k < n;
  ktau_lds[wave * kQW + l32] = my_valid ? p.timestamps[o0 + my_k] : 0;
  const int64_t kmin = wave_active ? stats[2 * (ka >> 5)] : 0;
  const int64_t kmax = wave_active ? stats[2 * (ka >> 5) + 1] : 0;

  // K and V of the lane's key as B operands (dh = kKStep*s + kKPL*half + [0, kKPL))
  Frag kf[L::kQSteps], vf[L::kQSteps];
  {
    const int64_t row = (int64_t)(o0 + (my_valid ? my_k : 0)) * p.row_stride + h * DH;
    const T *krow = (const T *)p.k + row, *vrow = (const T *)p.v + row;
#pragma unroll
    for (int s = 0; s < L::kQSteps; ++s) {
      if constexpr (L::kBf16) {
        bf16x8 x = *(const bf16x8 *)(krow + s * 16 + half * 8), y = *(const bf16x8 *)(vrow + s * 16 + half * 8);
        if (!my_valid) { x = bf16x8{}; y = bf16x8{}; }
        kf[s] = x;
        vf[s] = y;
      } else {
        kf[s] = my_valid ? krow[s * 2 + half] : 0.0f;
        vf[s] = my_valid ? vrow[s * 2 + half] : 0.0f;
      }
    }
  }

  // ---- query tiles: from the block's first row to the end (a block of candidate keys only: its own rows)
  const int q_end = (nh > k0) ? n : imin(k0 + kBM, n);
  const int t0 = k0 / kBN;
  const int ntiles = (q_end - k0 + kBN - 1) / kBN;

  // direct-to-LDS staging of Q and dO rows (both in the K layout) and the queries' timestamps
  const uint32_t rsb = (uint32_t)(p.row_stride * L::kES);
  const char *qbase = (const char *)p.q, *gbase = (const char *)p.d_out;
  auto issue_tile = [&](int i, int stage, int ln) {
    const int lr16 = 16 * wave + (ln >> 2);
    const uint32_t x_add = (uint32_t)(h * L::kRB) + 16u * (uint32_t)((ln & 3) ^ ((ln >> 4) & 3));
    const int tr16 = 16 * wave + ((ln & 31) >> 1);
    const uint32_t t_add = 4u * (uint32_t)(ln & 1);
    const int q0 = (t0 + i) * kBN;
    const int lim = n - 1 - q0;
    const uint32_t r = (uint32_t)imin(lr16, lim);
    const uint32_t off = __umul24(r, rsb) + x_add;
    const uint32_t toff = 8u * (uint32_t)imin(tr16, lim) + t_add;
    const int64_t row0 = (int64_t)(o0 + q0) * rsb;
    const uint32_t sb = smem_addr + stage * L::kStageBytes;
    dma_groups<0, L::kG>(qbase + row0, gbase + row0, off, off, sb + L::kOffK + wave * 1024,
                         sb + L::kOffV + wave * 1024);
    dma4((const char *)(p.timestamps + o0 + q0), toff, sb + L::kOffTau + 256 * wave);
  };

  OAcc<L::kDB> dk, dv;
#pragma unroll
  for (int d = 0; d < L::kDB; ++d) {
    dk.d[d] = floatx16{};
    dv.d[d] = floatx16{};
  }

  KeyCtx c;
  c.ka = ka;
  c.n = n;
  c.nh = nh;
  c.pos_lim = cand ? nh : n;
  c.P = P;
  c.Tb = Tb;
  c.ktau = ktau_lds + wave * kQW;
  c.wp = wp_lds;
  c.wt = wt_lds;
  const int kpl = imin(kl, nh);                    // position of the wave's last key

  constexpr int kAhead = L::kStages - 1;
#pragma unroll
  for (int i = 0; i < kAhead; ++i)
    if (i < ntiles) issue_tile(i, i, lane);
  __syncthreads();

  for (int i = 0; i < ntiles; ++i) {
    const int after = imin(kAhead - 1, ntiles - 1 - i);
    if (after >= 2) wait_vmcnt<2 * L::kLoadsPerTile>();
    else if (after == 1) wait_vmcnt<L::kLoadsPerTile>();
    else wait_vmcnt<0>();
    __syncthreads();
    const int ln = lane_now();
    if (i + kAhead < ntiles) issue_tile(i + kAhead, (i + kAhead) % L::kStages, ln);

    // class of (this wave's keys, tile i), in scalar code
    const int q0 = (t0 + i) * kBN;
    const int ql = imin(q0 + kBN - 1, n - 1);
    int body = kNone;
    float c1 = 0.0f;
    if (wave_active) {
      const bool any = ka < nh ? ql >= ka : (ql >= ka && q0 <= kl);
      if (any) {
        const bool all = kl < nh && q0 >= kl && q0 + kBN - 1 < n;   // a full tile: no repeated rows
        // the tile's timestamp range (rows past the end repeat the last row, inside the last chunk)
        int64_t qmin = stats[2 * (q0 >> 5)], qmax = stats[2 * (q0 >> 5) + 1];
        if (q0 + kChunk < n) {
          qmin = smin64(qmin, stats[2 * (q0 >> 5) + 2]);
          qmax = smax64(qmax, stats[2 * (q0 >> 5) + 3]);
        }
        const int64_t tmin = smin64(qmin, kmin);
        const bool k32 = (uint64_t)smax64(qmax, kmax) - (uint64_t)tmin < (1ull << 32);
        body = k32 ? (all ? kGen32 : kGen32M) : (all ? kGen64 : kGen64M);
        c.base_lo = (uint32_t)(uint64_t)tmin;
        if (all && imin(q0, nh) - kpl >= P - 1) {
          uint64_t lo, hi;
          if (qmin >= kmax) {
            lo = (uint64_t)qmin - (uint64_t)kmax;
            hi = (uint64_t)qmax - (uint64_t)kmin;
          } else if (kmin >= qmax) {
            lo = (uint64_t)kmin - (uint64_t)qmax;
            hi = (uint64_t)kmax - (uint64_t)qmin;
          } else {
            lo = 0;
            hi = (uint64_t)smax64(qmax, kmax) - (uint64_t)smin64(qmin, kmin);
          }
          const int blo = imin(lo == 0 ? 0 : 64 - __clzll((long long)lo), Tb - 1);
          const int bhi = imin(hi == 0 ? 0 : 64 - __clzll((long long)hi), Tb - 1);
          if (blo == bhi) {
            body = kUniform;
            c1 = kNegLog2e * (wp_lds[P - 1] + wt_lds[blo]);
          } else if (bhi == blo + 1 && k32) {
            body = kTwo;
            // wave-uniform values read from LDS: held in scalar registers
            c.thr = 1u << blo;
            c.bias_lo = readlane_f(wp_lds[P - 1] + wt_lds[blo], 0);
            c.bias_hi = readlane_f(wp_lds[P - 1] + wt_lds[bhi], 0);
          }
        }
      }
    }
    body = __builtin_amdgcn_readfirstlane(body);
    if (body != kNone) {
      c.q0 = q0;
      c.stage = smem + (i % L::kStages) * L::kStageBytes;
      dkdv_tile<T, DH>(dk, dv, kf, vf, c, body, c1, ln);
    }
  }

  // ---- epilogue: dK^T / dV^T element e of dh block db is dh = 32*db + 8*(e/4) + 4*half + e%4
  // (the lane's key rebuilt from lane_now(), not held across the loop)
  const int le = lane_now();
  const int e_key = ka + (le & 31), e_half = le >> 5;
  const bool e_valid = e_key < n;
  if (e_valid && p.z_q) {
    T *kz = (T *)p.z_k + (int64_t)(o0 + e_key) * p.z_row_stride + h * DH;
    T *vz = (T *)p.z_v + (int64_t)(o0 + e_key) * p.z_row_stride + h * DH;
#pragma unroll
    for (int db = 0; db < L::kDB; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const float gk[4] = {dk.d[db][4 * e4 + 0] * cb, dk.d[db][4 * e4 + 1] * cb, dk.d[db][4 * e4 + 2] * cb,
                             dk.d[db][4 * e4 + 3] * cb};
        const float gv[4] = {dv.d[db][4 * e4 + 0] * cb, dv.d[db][4 * e4 + 1] * cb, dv.d[db][4 * e4 + 2] * cb,
                             dv.d[db][4 * e4 + 3] * cb};
        silu_grad_store4(kz + 32 * db + 8 * e4 + 4 * e_half, gk);
        silu_grad_store4(vz + 32 * db + 8 * e4 + 4 * e_half, gv);
      }
  } else if (e_valid) {
    float *krow = p.dk + (int64_t)(o0 + e_key) * p.out_row_stride + h * DH;
    float *vrow = p.dv + (int64_t)(o0 + e_key) * p.out_row_stride + h * DH;
#pragma unroll
    for (int db = 0; db < L::kDB; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        floatx4 wk, wv;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          wk[x] = dk.d[db][4 * e4 + x] * cb;
          wv[x] = dv.d[db][4 * e4 + x] * cb;
        }
        *(floatx4 *)(krow + 32 * db + 8 * e4 + 4 * e_half) = wk;
        *(floatx4 *)(vrow + 32 * db + 8 * e4 + 4 * e_half) = wv;
      }
  }
}

template <typename T, int DH>
size_t dkdv_lds_bytes(int num_pos_buckets) {
  using L = Layout<T, DH>;
  return (size_t)L::kStages * L::kStageBytes + (size_t)kBM * sizeof(int64_t) +
         (size_t)(num_pos_buckets + kTimeTab) * sizeof(float);
}

template <typename T, int DH>
hipError_t launch_dkdv_typed(const AttnArgs &a, hipStream_t stream) {
  const int n_kblocks = (a.max_seq_len + kBM - 1) / kBM;
  const long long grid = (long long)n_kblocks * a.num_heads * a.num_seqs;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = dkdv_lds_bytes<T, DH>(a.num_pos_buckets);
  if (lds > 160 * 1024) return hipErrorInvalidConfiguration;
  static LdsLimit lim;
  hipError_t e = lim.raise((const void *)attn_bwd_dkdv_kernel<T, DH>, 160 * 1024);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DH>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a, n_kblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_dkdv(const AttnArgs &a, hipStream_t stream) {
  const bool bf = a.in_dtype == kBF16;
  switch (a.head_dim) {
    case 32: return bf ? launch_dkdv_typed<__bf16, 32>(a, stream) : launch_dkdv_typed<float, 32>(a, stream);
    case 64: return bf ? launch_dkdv_typed<__bf16, 64>(a, stream) : launch_dkdv_typed<float, 64>(a, stream);
    case 128: return bf ? launch_dkdv_typed<__bf16, 128>(a, stream) : launch_dkdv_typed<float, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t attn_bwd_dkdv_lds_bytes(int in_dtype, int head_dim, int num_pos_buckets) {
  const bool bf = in_dtype == kBF16;
  switch (head_dim) {
    case 32: return bf ? dkdv_lds_bytes<__bf16, 32>(num_pos_buckets) : dkdv_lds_bytes<float, 32>(num_pos_buckets);
    case 64: return bf ? dkdv_lds_bytes<__bf16, 64>(num_pos_buckets) : dkdv_lds_bytes<float, 64>(num_pos_buckets);
    default: return bf ? dkdv_lds_bytes<__bf16, 128>(num_pos_buckets) : dkdv_lds_bytes<float, 128>(num_pos_buckets);
  }
}

}  // namespace hstu
