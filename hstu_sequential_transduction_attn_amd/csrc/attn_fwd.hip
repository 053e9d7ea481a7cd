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
// so a workgroup covers 128 queries and shares every key tile among its 4 waves.  Two workgroups share
// a CU (two waves per SIMD, from different workgroups, so that their MFMA and VALU phases drift apart
// instead of running in lock-step behind one barrier).  Key tiles of 64 rows (K, V and their
// timestamps) go global -> LDS with direct-to-LDS loads (global_load_lds_dwordx4: no registers, no
// VALU) into a two-stage LDS ring; one barrier per tile.  Wave w loads rows 16w..16w+15 of every K and
// V column group and the timestamps of those 16 keys, so its per-lane source offsets are three
// registers per tile, clamped at the end of the sequence without a branch.
//
// Both contractions run on 32x32 MFMA tiles in a transposed form:
//     S^T[key][query] = K . Q^T        (A = K rows from LDS, B = Q held in registers)
//     O^T[dh][query] += V^T . P^T      (A = V^T read with ds_read_b64_tr_b16, B = P from registers)
// The score accumulator of the first product is already laid out as the B operand of the second:
// lane l always holds query l%32.  The first product reads its K rows in a permuted order (row m of the
// MFMA is key kperm(m)) so that the keys a lane holds in its 16 accumulator values are two runs of 8
// consecutive keys, which is exactly the k-order the second MFMA expects.  The transpose read hands each
// lane 4 consecutive keys of one dh column of V.
//
// LDS tile layout.  A K or V tile is stored column-group-major: the row's bytes are cut into 64-byte
// groups, and group g of key r sits at ((g * 64 + r) * 64).  One 1 KB direct-to-LDS load fills 16 rows of
// one group (four lanes per 64-byte line of the source); the V transpose reads of 16 lanes cover 4 rows x
// 32 bytes in distinct banks; in K, the four 16-byte pieces of a group are XOR-permuted by bits 2..3 of
// the row, so that the 16 rows one K-operand read touches land in 16 distinct bank groups.
//
// SiLU with the exponent scale folded in.  With u = -log2(e) * x, SiLU(x) = x / (1 + 2^u) =
// -ln(2) * u / (1 + 2^u).  The kernel forms u = fma(s, -log2 e, c1) directly (c1 = -log2(e) * bias for
// a tile with a single bias, else 0 with the bias already added to s), accumulates u / (1 + 2^u) and
// applies -ln(2) once, with c_b, to the output: one FMA, exp2, add, reciprocal and multiply per score.
//
// Bias and mask.  Per (wave, key tile) the work is classified from index ranges and from timestamp
// ranges (per-32-token minimum and maximum, computed by a small prologue kernel).  Each wave classifies
// 64 of its tiles at a time, one per lane, and reads a tile's class with readlane:
//   none      - no allowed pair: skipped;
//   uniform   - every pair allowed, one position bucket and one time bucket: a single bias constant;
//   two       - every pair allowed, one position bucket, the time bucket is one of two adjacent
//               buckets and the timestamps span less than 2^32: |tau_i - tau_j| from 32-bit offsets
//               (v_sad_u32), one compare and one select per score; when every key of the tile is no
//               later than every query of the wave (ordered timestamps) the gap is the plain 32-bit
//               difference of the low words, one instruction fewer;
//   general   - per-score mask and bucket lookups in LDS (32-bit offsets when the span allows,
//               exact 64-bit differences otherwise).
// All classes share one tile body: the MFMA code and the SiLU are common.  The scores of a block are
// taken out of the MFMA accumulator as 16 separate floats before the classes other than uniform add
// their per-score bias (and the mask) in a branch of their own: a branch that rewrote elements of the
// 16-wide accumulator value would make the register allocator copy the whole block at the class merge,
// on every path.  The output accumulators never change registers between classes.
#include "attn_common.hpp"
#include "work_order.hpp"

namespace hstu {
namespace {

using namespace attn;

// Leading zeros of a uint32 in one v_ffbh_u32: 0..31, and -1 (all bits set) for 0, so that a 32-bit gap d
// has bit length 32 - ffbh(d) for d > 0 and 0 for d = 0
__device__ __forceinline__ int ffbh_u32(uint32_t d) {
  int r;
  asm("v_ffbh_u32 %0, %1" : "=v"(r) : "v"(d));
  return r;
}

// |a - b| for uint32 a, b in one v_sad_u32
__device__ __forceinline__ uint32_t absdiff_u32(uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_sad_u32 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Per-score bias and mask of a non-uniform tile, added to the 16 scores of 32-key block kb (held as
// separate floats, so that the adjusted values stay in the scores' registers); element e holds key
// k0 + 32*kb + 16*(e/8) + 8*half + e%8.
// The forward's tables are padded so that no bucket needs a clamp: wp[d] = w_p[min(d, P-1)] for
// d < P + kPosPad and wt[b] = w_t[min(b, Tb-1)] for every bit length b <= 64; a 32-bit gap reads a second
// copy of the time table (wtr) by its leading-zero count, which saves the bit length's two instructions.  In a tile whose keys
// are all allowed, all history and no later than the query's position, the 8 keys of a lane's group
// have position distances d0 - e8 (d0 = my_pos - first key), so their biases are the 8 consecutive
// entries wp[d0 - 7 .. d0]; with d0 capped at P + 6 the window stays in the table and, past P - 1,
// reads w_p[P-1] for every key, as the clamp would.  In a masked tile the same holds for every allowed
// key but a candidate's own (distance 0).
template <typename T, int DH, int MODE>
__device__ __forceinline__ void adjust_scalar(float (&s)[16], const TileCtx &c, int kb, int half) {
  using L = Layout<T, DH>;
  constexpr bool kMasked = MODE == kGen32M || MODE == kGen64M;
  constexpr bool k64 = MODE == kGen64 || MODE == kGen64M;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int jl0 = 32 * kb + 16 * g + 8 * half;   // tile-local key of element 8*g
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w = *(const HSTU_LDS u32x4 *)(c.stage + L::tau_at(jl0 + 2 * q));
      lo[2 * q] = w.x; hi[2 * q] = w.y; lo[2 * q + 1] = w.z; hi[2 * q + 1] = w.w;
    }
    // masked tiles: a group whose keys are all past the position reads its (unused) window from just
    // below the table, inside the stage ring, wherever the position is
    const int d0 = imin(c.my_pos - (c.k0 + jl0), c.P + kPosPad - 2);
    const HSTU_LDS float *wpw = c.wp + (kMasked ? imax(d0, -1) : d0) - 7;
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const int e = 8 * g + e8;
      float bias;
      if constexpr (MODE == kTwoOrd) {
        // every key of the tile is no later than every query and the span is below 2^32: the 32-bit
        // difference of the low words is the exact gap
        bias = c.qlo - lo[e8] >= c.thr ? c.bias_hi : c.bias_lo;
      } else if constexpr (MODE == kTwo) {
        bias = absdiff_u32(c.qoff, lo[e8] - c.base_lo) >= c.thr ? c.bias_hi : c.bias_lo;
      } else {
        float wpv = wpw[7 - e8];
        if constexpr (kMasked) {
          // an allowed key other than the query itself is a history key no later than the query's
          // position, where the window holds; a candidate's own key has distance 0 (both at n_h); the
          // window's value for a masked key is never used
          if (c.k0 + jl0 + e8 == c.my_q) wpv = c.wp[0];
        }
        if constexpr (!k64) {
          // the reversed table takes the leading-zero count directly (no bit length, no clamp)
          bias = wpv + c.wtr[ffbh_u32(absdiff_u32(c.qoff, lo[e8] - c.base_lo))];
        } else {
          const int64_t tj = (int64_t)(((uint64_t)hi[e8] << 32) | lo[e8]);
          bias = wpv + c.wt[bitlen_absdiff(c.my_tau, tj)];
        }
      }
      if constexpr (kMasked) {
        const int j = c.k0 + jl0 + e8;
        const bool ok = (j <= c.key_lim) | (j == c.my_q);
        s[e] = ok ? s[e] + bias : kMaskedScore;
      } else {
        s[e] = s[e] + bias;
      }
    }
  }
}

template <typename T, int DH>
__device__ __forceinline__ void adjust_any(float (&s)[16], const TileCtx &c, int body, int kb, int half) {
  if (body == kTwoOrd) adjust_scalar<T, DH, kTwoOrd>(s, c, kb, half);
  else if (body == kTwo) adjust_scalar<T, DH, kTwo>(s, c, kb, half);
  else if (body == kGen32) adjust_scalar<T, DH, kGen32>(s, c, kb, half);
  else if (body == kGen32M) adjust_scalar<T, DH, kGen32M>(s, c, kb, half);
  else if (body == kGen64) adjust_scalar<T, DH, kGen64>(s, c, kb, half);
  else adjust_scalar<T, DH, kGen64M>(s, c, kb, half);
}

__device__ __forceinline__ void silu_scalar(const float (&s)[16], float (&a)[16], float c1) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float u = __builtin_fmaf(s[e], kNegLog2e, c1);
    a[e] = u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u));
  }
}

// One key tile for one wave.  Each 32-key block: scores (MFMA), for a non-uniform tile the per-score
// bias and mask added to the scores as separate floats (so the class branch changes no register
// assignment), SiLU, then AV.  The second block's score MFMAs are issued before the first block's
// SiLU, so that they run under it.
template <typename T, int DH>
__device__ __forceinline__ void tile_body(OAcc<Layout<T, DH>::kDB> &oacc,
                                          const typename QFrag<T>::type (&qf)[Layout<T, DH>::kQSteps],
                                          const TileCtx &c, int body, int lane) {
  using L = Layout<T, DH>;
  const int l32 = lane & 31, half = lane >> 5;
  const HSTU_LDS char *lK = c.stage + L::kOffK;
  const HSTU_LDS char *lV = c.stage + L::kOffV;
  floatx16 s0, s1;
  float x0[16], x1[16], a0[16], a1[16];
  score_block<T, DH>(s0, lK, 0, l32, half, qf);
#pragma unroll
  for (int e = 0; e < 16; ++e) x0[e] = s0[e];
  if (body != kUniform) adjust_any<T, DH>(x0, c, body, 0, half);
  score_block<T, DH>(s1, lK, 1, l32, half, qf);
  silu_scalar(x0, a0, c.c1);
  av_block<T, DH>(oacc, a0, lV, 0, lane);
#pragma unroll
  for (int e = 0; e < 16; ++e) x1[e] = s1[e];
  if (body != kUniform) adjust_any<T, DH>(x1, c, body, 1, half);
  silu_scalar(x1, a1, c.c1);
  av_block<T, DH>(oacc, a1, lV, 1, lane);
}

// ---- backward (dQ and the bias-table gradients), the same tiles as the forward
//   S^T = K Q^T (+ bias, mask);  dP^T = V dO^T;  dS = dP * SiLU'(s);  dQ^T += K^T dS^T
// (c_b is applied at the end).  V is staged in the K layout, so that its rows feed the A operand of
// dP^T like K's feed S^T, and K is read transposed for dQ^T.

// Bias-table gradient bins of one wave: all uniform and two-bucket tiles have position bucket P-1
// (run_p); consecutive uniform tiles with the same time bucket share run_t.  In the other tiles a
// score of position bucket P-1 also goes to run_p; the other position buckets are summed along
// anti-diagonals first (diag_pos_bins) in waves of history queries, and go score by score into the
// wave's LDS bins in waves of candidates.  The time buckets are run-length summed per lane (lane_t,
// lane_bt): along a query's keys the bucket changes rarely, and a lane adds its run to the LDS bin only
// when it does.  Adding every score to its time bin directly made most lanes of each instruction hit
// the same LDS address.  Per-wave bins, program order and single-lane flushes keep the sums in a fixed
// order.
struct GradBins {
  HSTU_LDS float *hp, *ht;   // this wave's position bins [P] and time bins [kTimeTab]
  float run_p, run_t;        // per-lane running sums
  int cur_bt;                // wave-uniform time bucket of run_t; -1 before the first uniform tile
  float lane_t;              // per-lane run of time bucket lane_bt (general tiles)
  int lane_bt;
  bool diag;                 // wave-uniform: every query of the wave is a history query, so the
                             // position bucket of every unclamped pair is i - j
};

// Lane i takes lane i + 1 (lane 63 takes 0), and lane i takes lane (i + 1) mod 64.
__device__ __forceinline__ float wave_shl1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_rol1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x134, 0xf, 0xf, true));
}

// Position bins of one 32-key block when every unclamped pair's bucket is i - j (history queries).
// w holds the block's dS with clamped pairs already zeroed.  For element e = 8g + m of lane L (query
// i = qa + L%32, key j = kb0 + 16g + 8(L/32) + m), i - j = qk - 16g - 8(L/32) + L%32 - m: along each
// anti-diagonal (lane + 1, element + 1) the bucket is the same.  Chain A shifts by one lane per element
// and sums the anti-diagonals that stay inside their lane half (L%32 >= m) into the lane where they
// start; chain B rotates the others (L%32 < m, whose bucket belongs to the other half's numbering) into
// lanes 25..31 and 57..63.  Two LDS adds per 8 elements replace eight; the order of the sums is fixed.
__device__ __forceinline__ void diag_pos_bins(GradBins &gb, const float (&w)[16], int qk, int lane, int P) {
  const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float a = l32 >= 7 ? w[8 * g + 7] : 0.0f;
    float b = l32 < 7 ? w[8 * g + 7] : 0.0f;
#pragma unroll
    for (int m = 6; m >= 0; --m) {
      a = wave_shl1(a) + (l32 >= m ? w[8 * g + m] : 0.0f);
      b = wave_rol1(b) + (l32 < m ? w[8 * g + m] : 0.0f);
    }
    const int bin_a = qk + l32 - 16 * g - 8 * h;   // bucket of lane L's chain-A sum
    const int bin_b = bin_a + 16 * h - 40;          // bucket of its chain-B sum (lanes 25..31, 57..63)
    if (bin_a >= 0 && bin_a < P - 1) __builtin_amdgcn_ds_faddf(gb.hp + bin_a, a, 0, 0, false);
    if (l32 >= 25 && bin_b >= 0 && bin_b < P - 1) __builtin_amdgcn_ds_faddf(gb.hp + bin_b, b, 0, 0, false);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Lane 0 adds the wave's total of v (its own butterfly order, the same on every run) to an LDS bin.
__device__ __forceinline__ void flush_bin(HSTU_LDS float *bin, float v, int lane) {
  const float t = wave_sum(v);
  if (lane == 0) *bin += t;
}

// SiLU'(x) with x = s + bias recovered from the folded exponent u = -log2(e) x:
// sigma = 1 / (1 + 2^u), SiLU'(x) = sigma (1 + x (1 - sigma)).  A masked score (u = 1.4e30) gives
// sigma = 0 and a derivative of exactly 0.
__device__ __forceinline__ float silu_grad_folded(float u) {
  const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u));
  return sig * fmaf(u * kNegLn2, 1.0f - sig, 1.0f);
}

// One tile for one wave.  As in the forward, every class shares one copy of the MFMA code (so the dQ^T
// accumulators never change registers between classes); only the bias/mask adjustment and the
// bias-gradient binning branch on the class.
template <typename T, int DH>
__device__ __forceinline__ void bwd_tile_body(OAcc<Layout<T, DH>::kDB> &dq,
                                              const typename QFrag<T>::type (&qf)[Layout<T, DH>::kQSteps],
                                              const typename QFrag<T>::type (&gf)[Layout<T, DH>::kQSteps],
                                              const TileCtx &c, int body, int code, int lane, GradBins &gb) {
  using L = Layout<T, DH>;
  const int l32 = lane & 31, half = lane >> 5;
  const HSTU_LDS char *lK = c.stage + L::kOffK;
  const HSTU_LDS char *lV = c.stage + L::kOffV;
  float sa = 0.0f, sb = 0.0f;   // uniform: the tile's sum; two-bucket: the sums of the two buckets
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    floatx16 s, dp;
    score_block<T, DH>(s, lK, kb, l32, half, qf);
    score_block<T, DH>(dp, lV, kb, l32, half, gf);
    int bins[16];
    if (body != kUniform) {
      if (body == kTwo) adjust_block<T, DH, kTwo, true>(s, c, kb, half, bins);
      else if (body == kGen32) adjust_block<T, DH, kGen32, true>(s, c, kb, half, bins);
      else if (body == kGen32M) adjust_block<T, DH, kGen32M, true>(s, c, kb, half, bins);
      else if (body == kGen64) adjust_block<T, DH, kGen64, true>(s, c, kb, half, bins);
      else adjust_block<T, DH, kGen64M, true>(s, c, kb, half, bins);
    }
    float ds[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) ds[e] = dp[e] * silu_grad_folded(fmaf(s[e], kNegLog2e, c.c1));
    if (body == kUniform) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sa += ds[e];
    } else if (body == kTwo) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if ((bins[e] >> 16) == c.blo) sa += ds[e];
        else sb += ds[e];
      }
    } else {
      if (gb.diag) {
        float w[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool clamp = (bins[e] & 0xffff) == c.P - 1;
          gb.run_p += clamp ? ds[e] : 0.0f;
          w[e] = clamp ? 0.0f : ds[e];
        }
        diag_pos_bins(gb, w, c.my_q - l32 - c.k0 - 32 * kb, lane, c.P);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int bp = bins[e] & 0xffff;
          if (bp == c.P - 1) gb.run_p += ds[e];
          else __builtin_amdgcn_ds_faddf(gb.hp + bp, ds[e], 0, 0, false);
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int bt = bins[e] >> 16;
        if (bt != gb.lane_bt) {
          __builtin_amdgcn_ds_faddf(gb.ht + gb.lane_bt, gb.lane_t, 0, 0, false);
          gb.lane_bt = bt;
          gb.lane_t = 0.0f;
        }
        gb.lane_t += ds[e];
      }
    }
    av_block_in<T, DH, true>(dq, ds, lK, kb, lane);
  }
  if (body == kUniform) {
    const int bt = (code >> 8) & 255;
    if (bt != gb.cur_bt) {                     // wave-uniform
      if (gb.cur_bt >= 0) flush_bin(gb.ht + gb.cur_bt, gb.run_t, lane);
      gb.run_t = 0.0f;
      gb.cur_bt = bt;
    }
    gb.run_t += sa;
    gb.run_p += sa;
  } else if (body == kTwo) {
    flush_bin(gb.ht + c.blo, sa, lane);
    flush_bin(gb.ht + c.blo + 1, sb, lane);
    gb.run_p += sa + sb;
  }
}

// Timestamp minimum and maximum of every 32-token chunk of every sequence.  Chunk c of sequence b is
// stored at index first(b) + c with first(b) = (o_b >> 5) + b, which never collides across sequences
// (first(b + 1) >= first(b) + ceil(n_b / 32)) and stays below T/32 + B + 1.  Flat over that index
// space, one lane per token: lanes 32i..32i+31 of the grid own storage index i, find its sequence by a
// binary search of first(b), load one timestamp each and reduce over the 32 lanes.
__global__ void __launch_bounds__(256) tau_chunk_stats_kernel(const int32_t *__restrict__ offs,
                                                              const int64_t *__restrict__ tau,
                                                              int64_t *__restrict__ stats, int num_seqs,
                                                              int num_slots) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int slot = (int)(g >> 5), t = (int)(g & 31);
  int64_t mn = INT64_MAX, mx = INT64_MIN;
  bool owned = false;
  if (slot < num_slots) {
    int lo = 0, hi = num_seqs - 1;                 // last b with first(b) <= slot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((offs[mid] >> 5) + mid <= slot) lo = mid; else hi = mid - 1;
    }
    const int o0 = offs[lo], n = offs[lo + 1] - o0;
    const int c = slot - ((o0 >> 5) + lo);
    owned = c < (n + kChunk - 1) / kChunk;         // false in the gaps between sequences
    if (owned && kChunk * c + t < n) mn = mx = tau[o0 + kChunk * c + t];
  }
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) {
    const int64_t a = __shfl_xor(mn, m, 32), b2 = __shfl_xor(mx, m, 32);
    mn = a < mn ? a : mn;
    mx = b2 > mx ? b2 : mx;
  }
  if (owned && t == 0) {
    stats[2 * (int64_t)slot] = mn;
    stats[2 * (int64_t)slot + 1] = mx;
  }
}

// Sum of the key splits of cached scoring, in split order (deterministic), times c_b * (-ln 2) (the
// folded SiLU's factor).  One thread per 4 consecutive output values of one candidate row; the user of
// the row comes from a binary search of the candidate offsets.
template <typename TO>
__global__ void __launch_bounds__(256) attn_split_reduce_kernel(const AttnArgs p, int row_vals) {
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = i4 * 4 / row_vals;
  if (row >= p.num_rows) return;
  const int col = (int)(i4 * 4 - row * row_vals);
  int lo = 0, hi = p.num_seqs - 1;                 // last b with seq_offsets[b] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.seq_offsets[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int nh = p.hist_offsets[b + 1] - p.hist_offsets[b];
  const int nq = p.seq_offsets[b + 1] - p.seq_offsets[b];
  const int tiles = (nh + kBN - 1) / kBN;
  const int used = imin(p.kv_splits, imax(1, (tiles + p.tiles_per_split - 1) / p.tiles_per_split));
  const float cb = p.attn_scale ? p.attn_scale[b] : 1.0f / (float)(nh + nq);
  const float scale = cb * kNegLn2;
  floatx4 acc = floatx4{};
  for (int sp = 0; sp < used; ++sp) {
    const floatx4 v = *(const floatx4 *)(p.partial + ((int64_t)sp * p.num_rows + row) * row_vals + col);
    acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
  }
  TO *o = (TO *)p.out + row * p.out_row_stride + col;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = from_f32<TO>(acc[e] * scale);
}

// The query-major attention body, shared by the forward, cached scoring (CACHED) and the backward's dQ
// pass (BWD); the kernels that run it are defined after it.
//
// CACHED: candidates scored against a cached history.  The queries are the candidate rows (q,
// seq_offsets, timestamps); user b's keys are its n_h cached history rows (k_hist, v_hist,
// hist_offsets, hist_timestamps), every one of them allowed, and each candidate also sees itself,
// which the epilogue adds as one extra score per row.  A candidate has position n_h and local index
// n_h + c in the virtual sequence [history | candidates], so the tile classes, buckets and masks are
// those of the candidate rows of the one-pass candidate mask.  A user's history tiles may be split over
// kv_splits workgroups (tiles_per_split each, the last one taking the rest): with no softmax the partial
// sums over key ranges simply add, so each split stores its raw sums in `partial` and a reduction kernel
// adds them in split order.
//
// BWD: the dQ pass of the backward (bwd_tile_body); out is dQ (fp32) and each workgroup writes its
// bias-gradient bins (times c_b) to row canonical_item(...) of `partial` (the item's place in query-block-major
// order, whatever order the items run in).
template <typename T, int DH, typename TO, bool CACHED, bool BWD>
__device__ __forceinline__ void attn_query_major(const AttnArgs &p, const int n_qblocks) {
  using L = Layout<T, DH>;
  using Frag = typename QFrag<T>::type;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  HSTU_LDS char *smem = (HSTU_LDS char *)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  // ---- work item: the XCD-local order of work_order.hpp; cached: query block major (longest first),
  // then (sequence, head), key split fastest
  const int HB = p.num_heads * p.num_seqs;
  const int split = CACHED ? (int)(blockIdx.x % (unsigned)p.kv_splits) : 0;
  const int item = CACHED ? (int)(blockIdx.x / (unsigned)p.kv_splits) : (int)blockIdx.x;
  const WorkItem wi = CACHED ? WorkItem{item / HB, item % HB} : work_item(item, HB, n_qblocks);
  const int qblk = n_qblocks - 1 - wi.rank;
  const int b = wi.pair / p.num_heads;
  const int h = wi.pair % p.num_heads;
  [[maybe_unused]] const int64_t bins_row = canonical_item(wi, HB);   // backward: its row of `partial`
  // o0/nq: first row and count of this sequence's query rows; ho/nh: first key row and history length;
  // vq0: local (virtual-sequence) index of query row 0; n: virtual sequence length
  const int o0 = p.seq_offsets[b];
  const int nq = p.seq_offsets[b + 1] - o0;
  const int q0 = qblk * kBM;
  const int nbins = p.num_pos_buckets + kTimeTab;  // backward: bias-gradient bins per wave
  if (q0 >= nq) {        // uniform over the workgroup
    if constexpr (BWD)
      for (int i = threadIdx.x; i < nbins; i += kThreads) p.partial[bins_row * nbins + i] = 0.0f;
    return;
  }
  const bool cand = CACHED || p.mask == kCausalCandidates;
  const int ho = CACHED ? p.hist_offsets[b] : o0;
  const int nh = CACHED ? p.hist_offsets[b + 1] - ho : (cand ? nq - p.num_candidates[b] : nq);
  const int vq0 = CACHED ? nh : 0;
  const int n = vq0 + nq;
  const int nkeys = CACHED ? nh : nq;             // rows of the key buffers of this sequence
  const float cb = p.attn_scale ? p.attn_scale[b] : 1.0f / (float)n;
  const int P = p.num_pos_buckets;
  const int Tb = p.num_time_buckets;
  const int rr = p.rab_rows == 1 ? 0 : h;
  // 32-token timestamp ranges: chunk c at [2c], [2c+1]; of the query rows and of the key rows
  const int64_t *qstats = p.tau_stats + 2 * (int64_t)((o0 >> 5) + b);
  const int64_t *kstats = CACHED ? p.hist_tau_stats + 2 * (int64_t)((ho >> 5) + b) : qstats;
  const int64_t *ktau = CACHED ? p.hist_timestamps : p.timestamps;

  const int tid = threadIdx.x;
  // wave index in a scalar register: the query range and the tile classes derived from it are
  // wave-uniform, so each tile runs exactly one class body, selected by a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- bias tables into LDS (after the stage ring)
  // forward: both tables padded with their last entry (no bucket clamp in the per-score bias, see
  // adjust_scalar); the dQ pass reads entries below P and Tb only
  HSTU_LDS float *wp_lds = (HSTU_LDS float *)(smem + L::kStages * L::kStageBytes);
  HSTU_LDS float *wt_lds = wp_lds + P + (BWD ? 0 : kPosPad);
  for (int i = tid; i < P + (BWD ? 0 : kPosPad); i += kThreads) wp_lds[i] = p.pos_bias[(int64_t)rr * P + imin(i, P - 1)];
  for (int i = tid; i < kTimeTab; i += kThreads) wt_lds[i] = p.time_bias[(int64_t)rr * Tb + imin(i, Tb - 1)];
  // forward: the time table once more, by leading-zero count of a 32-bit gap (entry 0: a gap of 0; entry
  // z + 1: a gap with z leading zeros, bit length 32 - z)
  HSTU_LDS float *wtr_lds = wt_lds + kTimeTab;
  if constexpr (!BWD)
    for (int i = tid; i < kTimeRev; i += kThreads) wtr_lds[i] = p.time_bias[(int64_t)rr * Tb + imin(i == 0 ? 0 : 33 - i, Tb - 1)];

  // ---- this wave's queries
  const int qr = q0 + wave * kQW;                 // first query row of the wave (a multiple of 32)
  const int qa = vq0 + qr;                        // its local index
  const int ql = vq0 + imin(qr + kQW - 1, nq - 1);   // local index of the wave's last valid query
  const bool wave_active = qr < nq;
  const int my_row = qr + l32;                    // this lane's query row (sequence-relative)
  const int my_q = vq0 + my_row;                  // its local index
  const bool my_valid = my_row < nq;
  const int64_t my_tau = my_valid ? p.timestamps[o0 + my_row] : 0;
  const int64_t wmin = wave_active ? qstats[2 * (qr >> 5)] : 0;
  const int64_t wmax = wave_active ? qstats[2 * (qr >> 5) + 1] : 0;

  // Q fragments (B operand of S^T = K Q^T): lane holds query l32, dh = kKStep*s + kKPL*half + [0, kKPL)
  Frag qf[L::kQSteps];
  {
    const T *qrow = (const T *)p.q + (int64_t)(o0 + (my_valid ? my_row : 0)) * p.row_stride + h * DH;
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

  // dO fragments (backward: B operand of dP^T = V dO^T), laid out like the Q fragments
  Frag gf[BWD ? L::kQSteps : 1];
  if constexpr (BWD) {
    const T *grow = (const T *)p.d_out + (int64_t)(o0 + (my_valid ? my_row : 0)) * p.row_stride + h * DH;
#pragma unroll
    for (int s = 0; s < L::kQSteps; ++s) {
      if constexpr (L::kBf16) {
        bf16x8 v = *(const bf16x8 *)(grow + s * 16 + half * 8);
        if (!my_valid) v = bf16x8{};
        gf[s] = v;
      } else {
        gf[s] = my_valid ? grow[s * 2 + half] : 0.0f;
      }
    }
  }

  // ---- key tiles needed by the workgroup: [0, r1_end) and, for candidate rows, their own tiles
  const int blast = vq0 + imin(q0 + kBM - 1, nq - 1);
  const int r1_end = (imin(blast + 1, nh) + kBN - 1) / kBN;
  int r2_begin = 0, r2_end = 0;
  if (!CACHED && blast >= nh) {
    r2_begin = imax(imax(q0, nh) / kBN, r1_end);
    r2_end = blast / kBN + 1;
  }
  int ntiles = r1_end + imax(r2_end - r2_begin, 0);
  int t_first = 0;                                // cached: first history tile of this key split
  if constexpr (CACHED) {
    t_first = split * p.tiles_per_split;
    const int t_end = split == p.kv_splits - 1 ? r1_end : imin(r1_end, t_first + p.tiles_per_split);
    if (split > 0 && t_first >= t_end) return;    // an empty split (split 0 always runs: the self term)
    ntiles = imax(t_end - t_first, 0);
  }
  auto tile_of = [&](int i) -> int { return i < r1_end ? t_first + i : r2_begin + (i - r1_end); };

  // ---- direct-to-LDS staging.  Per tile, wave w loads rows 16w..16w+15 of each 64-byte column group g
  // of K and of V (1 KB each: lane l takes row 16w + l/4 and 16-byte piece l%4 of the group; in K, the
  // piece whose XOR-permuted position is l%4) and the 16 timestamps of those rows (lanes 32..63 repeat
  // lanes 0..31 into an unused half of the wave's 256-byte slot).  Rows past the end of the sequence
  // load its last row instead (finite data that the mask discards).
  const uint32_t rsb = (uint32_t)(p.row_stride * L::kES);        // bytes between tokens (<= 16 KB)
  // (the backward, near the register limit, rebuilds the lane's offsets at each tile from lane_now())
  const char *kbase = (const char *)(CACHED ? p.k_hist : p.k), *vbase = (const char *)(CACHED ? p.v_hist : p.v);
  auto issue_tile = [&](int i, int stage, int ln) {
    const int lr16 = 16 * wave + (ln >> 2);                      // tile-local row this lane loads
    const uint32_t k_add = (uint32_t)(h * L::kRB) + 16u * (uint32_t)((ln & 3) ^ ((ln >> 4) & 3));
    const uint32_t v_add = BWD ? k_add : (uint32_t)(h * L::kRB) + 16u * (uint32_t)(ln & 3);
    const int tr16 = 16 * wave + ((ln & 31) >> 1);               // tile-local key of this lane's tau word
    const uint32_t t_add = 4u * (uint32_t)(ln & 1);
    const int k0 = tile_of(i) * kBN;
    const int lim = nkeys - 1 - k0;                              // >= 0: every tile starts inside the keys
    const uint32_t r = (uint32_t)imin(lr16, lim);
    const uint32_t koff = __umul24(r, rsb) + k_add;
    const uint32_t voff = __umul24(r, rsb) + v_add;
    const uint32_t toff = 8u * (uint32_t)imin(tr16, lim) + t_add;
    const int64_t row0 = (int64_t)(ho + k0) * rsb;
    const uint32_t sb = smem_addr + stage * L::kStageBytes;
    dma_groups<0, L::kG>(kbase + row0, vbase + row0, koff, voff, sb + L::kOffK + wave * 1024,
                         sb + L::kOffV + wave * 1024);
    dma4((const char *)(ktau + ho + k0), toff, sb + L::kOffTau + 256 * wave);
  };

  // ---- tile classes, one tile per lane, 64 tiles at a time (vector code, once per 64 tiles)
  int cls_code = 0;
  float cls_lo = 0.0f, cls_hi = 0.0f;
  uint32_t cls_base = 0;
  auto classify = [&](int t0) {
    const int t = t0 + lane;
    int code = kNone;
    float clo = 0.0f, chi = 0.0f;
    uint32_t base = 0;
    if (t < ntiles && wave_active) {
      const int k0 = tile_of(t) * kBN;
      const bool none = k0 > ql || (k0 >= nh && k0 + kBN - 1 < imax(qa, nh));
      if (!none) {
        const int c0 = k0 >> 5;
        int64_t kmin = kstats[2 * c0], kmax = kstats[2 * c0 + 1];
        if (k0 + kChunk < nkeys) {
          const int64_t a = kstats[2 * c0 + 2], bb = kstats[2 * c0 + 3];
          kmin = a < kmin ? a : kmin;
          kmax = bb > kmax ? bb : kmax;
        }
        const int64_t tmin = wmin < kmin ? wmin : kmin;
        const int64_t tmax = wmax > kmax ? wmax : kmax;
        const uint64_t span = (uint64_t)tmax - (uint64_t)tmin;
        base = (uint32_t)(uint64_t)tmin;
        const bool all = (k0 + kBN - 1 <= qa) && (k0 + kBN - 1 < nh);
        code = span < (1ull << 32) ? (all ? kGen32 : kGen32M) : (all ? kGen64 : kGen64M);
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
          const int blo = imin(lo == 0 ? 0 : 64 - __clzll((long long)lo), Tb - 1);
          const int bhi = imin(hi == 0 ? 0 : 64 - __clzll((long long)hi), Tb - 1);
          const float wpc = wp_lds[P - 1];
          if (blo == bhi) {
            code = kUniform | (blo << 8);   // the bucket is read only by the backward
            clo = kNegLog2e * (wpc + wt_lds[blo]);
          } else if (bhi == blo + 1 && span < (1ull << 32)) {
            // threshold 2^blo: |dt| >= 2^blo has bit length > blo
            code = (!BWD && kmax <= wmin ? kTwoOrd : kTwo) | (blo << 8);
            clo = wpc + wt_lds[blo];
            chi = wpc + wt_lds[bhi];
          }
        }
      }
    }
    cls_code = code; cls_lo = clo; cls_hi = chi; cls_base = base;
  };

  OAcc<L::kDB> oacc;
#pragma unroll
  for (int d = 0; d < L::kDB; ++d) oacc.d[d] = floatx16{};

  TileCtx c;
  // cached mode: the tiles hold history keys only (rows past the history repeat its last row), and the
  // candidate's score against itself is added in the epilogue, so no tile key may match it
  c.my_q = CACHED ? -1 : my_q;
  c.my_pos = cand ? imin(my_q, nh) : my_q;
  c.pos_lim = cand ? nh : n;
  // a history query sees keys 0..my_q, a candidate the whole history and itself (every allowed key is
  // < n for a query < n; lanes past the end are never stored)
  c.key_lim = my_q < nh ? my_q : nh - 1;
  c.nh = nh;
  c.P = P;
  c.Tb = Tb;
  c.my_tau = my_tau;
  c.wp = wp_lds;
  c.wt = wt_lds;
  c.wtr = wtr_lds + 1;

  // backward: this wave's bias-gradient bins (after the bias tables), cleared by the wave itself
  GradBins gb{};
  if constexpr (BWD) {
    gb.hp = wt_lds + kTimeTab + wave * nbins;
    gb.ht = gb.hp + P;
    gb.cur_bt = -1;
    gb.lane_bt = 0;   // an empty run (lane_t = 0) of bucket 0
    gb.diag = !cand || qa + kQW - 1 < nh;
    for (int i = lane; i < nbins; i += kWave) gb.hp[i] = 0.0f;
  }

  constexpr int kAhead = L::kStages - 1;      // tiles in flight beyond the one being computed
#pragma unroll
  for (int i = 0; i < kAhead; ++i)
    if (i < ntiles) issue_tile(i, i, lane);
  __syncthreads();                            // bias tables visible to the classification

  for (int i = 0; i < ntiles; ++i) {
    if ((i & 63) == 0) classify(i);
    // tile i has landed once at most (tiles issued after it) x (loads per tile) loads are outstanding
    const int after = imin(kAhead - 1, ntiles - 1 - i);
    if (after >= 2) wait_vmcnt<2 * L::kLoadsPerTile>();
    else if (after == 1) wait_vmcnt<L::kLoadsPerTile>();
    else wait_vmcnt<0>();
    __syncthreads();  // tile i visible to all waves; every wave is done with tile i - 1
    const int ln = BWD ? lane_now() : lane;
    if (i + kAhead < ntiles) issue_tile(i + kAhead, (i + kAhead) % L::kStages, ln);

    const int li = i & 63;
    const int code = readlane_i(cls_code, li);
    const int body = code & 7;
    if (body != kNone) {
      c.k0 = tile_of(i) * kBN;
      c.stage = smem + (i % L::kStages) * L::kStageBytes;
      const float lo_v = readlane_f(cls_lo, li);
      c.c1 = body == kUniform ? lo_v : 0.0f;
      c.bias_lo = lo_v;
      c.bias_hi = readlane_f(cls_hi, li);
      c.thr = 1u << ((code >> 8) & 31);
      c.blo = (code >> 8) & 255;
      c.base_lo = (uint32_t)readlane_i((int)cls_base, li);
      c.qoff = (uint32_t)(uint64_t)my_tau - c.base_lo;
      c.qlo = (uint32_t)(uint64_t)my_tau;
      if constexpr (BWD) bwd_tile_body<T, DH>(oacc, qf, gf, c, body, code, ln, gb);
      else tile_body<T, DH>(oacc, qf, c, body, lane);
    }
  }

  // ---- epilogue: O^T element e of dh block db is dh = 32*db + 8*(e/4) + 4*half + e%4; the sums carry
  // the factor -log2(e) of the folded SiLU, removed here together with c_b
  if (CACHED && split == 0) {
    // the candidate's score against itself: both distances are 0, so the bias is w_p[0] + w_t[0]
    const int64_t crow = (int64_t)(o0 + (my_valid ? my_row : 0));
    const T *krow = (const T *)p.k + crow * p.row_stride + h * DH;
    const T *vrow = (const T *)p.v + crow * p.row_stride + h * DH;
    float dot = 0.0f;
#pragma unroll
    for (int st = 0; st < L::kQSteps; ++st) {
      if constexpr (L::kBf16) {
        const bf16x8 kv = *(const bf16x8 *)(krow + st * 16 + half * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(bf16_to_f32(qf[st][e]), bf16_to_f32(kv[e]), dot);
      } else {
        dot = fmaf(qf[st], krow[st * 2 + half], dot);
      }
    }
    dot += __shfl_xor(dot, 32, kWave);
    const float u = (dot + wp_lds[0] + wt_lds[0]) * kNegLog2e;
    const float a = my_valid ? u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u)) : 0.0f;
#pragma unroll
    for (int db = 0; db < L::kDB; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int dh = 32 * db + 8 * e4 + 4 * half;
#pragma unroll
        for (int x = 0; x < 4; ++x) oacc.d[db][4 * e4 + x] = fmaf(a, to_f32(vrow[dh + x]), oacc.d[db][4 * e4 + x]);
      }
  }
  if constexpr (BWD) {
    // dQ = c_b * sum dS k (the accumulators hold true dS values); then the bias-gradient bins
    if (gb.cur_bt >= 0) flush_bin(gb.ht + gb.cur_bt, gb.run_t, lane);
    flush_bin(gb.hp + (P - 1), gb.run_p, lane);
    __builtin_amdgcn_ds_faddf(gb.ht + gb.lane_bt, gb.lane_t, 0, 0, false);
    if (my_valid && p.z_q) {
      T *zrow = (T *)p.z_q + (int64_t)(o0 + my_row) * p.z_row_stride + h * DH;
#pragma unroll
      for (int db = 0; db < L::kDB; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const float g[4] = {oacc.d[db][4 * e4 + 0] * cb, oacc.d[db][4 * e4 + 1] * cb,
                              oacc.d[db][4 * e4 + 2] * cb, oacc.d[db][4 * e4 + 3] * cb};
          silu_grad_store4(zrow + 32 * db + 8 * e4 + 4 * half, g);
        }
    } else if (my_valid) {
      float *drow = (float *)p.out + (int64_t)(o0 + my_row) * p.out_row_stride + h * DH;
#pragma unroll
      for (int db = 0; db < L::kDB; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          floatx4 w;
          w[0] = oacc.d[db][4 * e4 + 0] * cb; w[1] = oacc.d[db][4 * e4 + 1] * cb;
          w[2] = oacc.d[db][4 * e4 + 2] * cb; w[3] = oacc.d[db][4 * e4 + 3] * cb;
          *(floatx4 *)(drow + 32 * db + 8 * e4 + 4 * half) = w;
        }
    }
    __syncthreads();   // every wave's bins complete
    const HSTU_LDS float *h0 = wt_lds + kTimeTab;
    for (int i = tid; i < nbins; i += kThreads) {
      const float v = ((h0[i] + h0[nbins + i]) + h0[2 * nbins + i]) + h0[3 * nbins + i];
      p.partial[bins_row * nbins + i] = v * cb;
    }
    return;
  }
  if (CACHED && p.kv_splits > 1) {
    // raw sums of this key split; attn_split_reduce_kernel adds the splits and applies the scale
    if (my_valid) {
      float *prow = p.partial + (((int64_t)split * p.num_rows + o0 + my_row) * p.num_heads + h) * DH;
#pragma unroll
      for (int db = 0; db < L::kDB; ++db)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          floatx4 w;
          w[0] = oacc.d[db][4 * e4 + 0]; w[1] = oacc.d[db][4 * e4 + 1];
          w[2] = oacc.d[db][4 * e4 + 2]; w[3] = oacc.d[db][4 * e4 + 3];
          *(floatx4 *)(prow + 32 * db + 8 * e4 + 4 * half) = w;
        }
    }
    return;
  }
  const float scale = cb * kNegLn2;
  if (p.row_stats) {
    // mean and sum of squared deviations of the stored head row: each lane holds 16*kDB of its query's
    // values, lane ^ 32 the others; the two halves combine exactly (equal counts)
    constexpr float kN = 16.0f * L::kDB;
    float sum = 0.0f;
#pragma unroll
    for (int db = 0; db < L::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += oacc.d[db][e] * scale;
    const float mean_l = sum / kN;
    float m2_l = 0.0f;
#pragma unroll
    for (int db = 0; db < L::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float d = oacc.d[db][e] * scale - mean_l;
        m2_l += d * d;
      }
    const float mean_o = __shfl_xor(mean_l, 32, kWave), m2_o = __shfl_xor(m2_l, 32, kWave);
    const float dm = mean_l - mean_o;
    if (my_valid && half == 0) {
      float *st = p.row_stats + 2 * ((int64_t)(o0 + my_row) * p.num_heads + h);
      st[0] = 0.5f * (mean_l + mean_o);
      st[1] = m2_l + m2_o + dm * dm * (0.5f * kN);
    }
  }
  if (my_valid) {
    TO *orow = (TO *)p.out + (int64_t)(o0 + my_row) * p.out_row_stride + h * DH;
#pragma unroll
    for (int db = 0; db < L::kDB; ++db) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int dh = 32 * db + 8 * e4 + 4 * half;
        if constexpr (sizeof(TO) == 4) {
          floatx4 w;
          w[0] = oacc.d[db][4 * e4 + 0] * scale; w[1] = oacc.d[db][4 * e4 + 1] * scale;
          w[2] = oacc.d[db][4 * e4 + 2] * scale; w[3] = oacc.d[db][4 * e4 + 3] * scale;
          *(floatx4 *)(orow + dh) = w;
        } else {
          bf16x4 w;
          w[0] = f32_to_bf16(oacc.d[db][4 * e4 + 0] * scale); w[1] = f32_to_bf16(oacc.d[db][4 * e4 + 1] * scale);
          w[2] = f32_to_bf16(oacc.d[db][4 * e4 + 2] * scale); w[3] = f32_to_bf16(oacc.d[db][4 * e4 + 3] * scale);
          *(bf16x4 *)(orow + dh) = w;
        }
      }
    }
  }
}

void launch_tau_stats(const int32_t *offs, const int64_t *tau, int64_t *stats, int num_seqs, int64_t total_tokens,
                      hipStream_t stream) {
  if (num_seqs <= 0) return;
  const int64_t slots = (total_tokens >> 5) + num_seqs + 1;
  hipLaunchKernelGGL(tau_chunk_stats_kernel, dim3((unsigned)((slots * 32 + 255) / 256)), dim3(256), 0, stream, offs,
                     tau, stats, num_seqs, (int)slots);
}

// The forward and cached scoring: two waves per SIMD (<= 256 registers per lane), so that one wave's
// MFMAs overlap the other's VALU work.
template <typename T, int DH, typename TO, bool CACHED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const AttnArgs p, const int n_qblocks) {
  attn_query_major<T, DH, TO, CACHED, false>(p, n_qblocks);
}

// The backward's dQ pass carries dO fragments and bucket indices as well.  It too runs two waves per
// SIMD; at Dh = 128 (bf16) it fits the 256 registers without spilling because its lane offsets are
// rebuilt at each tile from lane_now() rather than held across the loop.
template <typename T, int DH>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(const AttnArgs p, const int n_qblocks) {
  attn_query_major<T, DH, float, false, true>(p, n_qblocks);
}

// Dynamic LDS of the query-major kernel: the stage ring, the bias tables and (backward) four waves'
// bias-gradient bins.
template <typename T, int DH, bool BWD>
size_t attn_lds_bytes(int num_pos_buckets) {
  using L = Layout<T, DH>;
  const size_t tables = (size_t)(num_pos_buckets + (BWD ? 0 : kPosPad + kTimeRev) + kTimeTab) * sizeof(float);
  return (size_t)L::kStages * L::kStageBytes + tables * (BWD ? 1 + kWaves : 1);
}

// Bias-table gradients: the workgroups' bins (already times c_b) added over the workgroups, one
// 256-thread block per table entry: thread t adds rows t, t + 256, ... in order, then the block adds
// its 256 partial sums in a fixed tree (so the result is the same on every run).  Time buckets past
// the largest possible bit length (64) get 0.
__global__ void __launch_bounds__(256) attn_bias_grad_reduce_kernel(const AttnArgs p, int nwg) {
  const int P = p.num_pos_buckets, Tb = p.num_time_buckets, nbins = P + kTimeTab;
  const int idx = blockIdx.x;                      // < rab_rows * (P + Tb)
  const int r = idx / (P + Tb), i = idx % (P + Tb);
  const int bin = i < P ? i : (i - P < kTimeTab ? i : -1);
  const int HB = p.num_heads * p.num_seqs;
  float sum = 0.0f;
  if (bin >= 0)
    for (int w = threadIdx.x; w < nwg; w += 256)
      if (p.rab_rows == 1 || (w % HB) % p.num_heads == r) sum += p.partial[(int64_t)w * nbins + bin];
  __shared__ float part[256];
  part[threadIdx.x] = sum;
  __syncthreads();
#pragma unroll
  for (int h = 128; h >= 1; h >>= 1) {
    if ((int)threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (i < P) p.d_pos_bias[(int64_t)r * P + i] = part[0];
    else p.d_time_bias[(int64_t)r * Tb + (i - P)] = part[0];
  }
}

template <typename T, int DH, typename TO, bool CACHED, bool BWD>
hipError_t launch_typed(const AttnArgs &a, hipStream_t stream) {
  const int n_qblocks = (a.max_seq_len + kBM - 1) / kBM;
  const long long grid = (long long)n_qblocks * a.num_heads * a.num_seqs * (CACHED ? a.kv_splits : 1);
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = attn_lds_bytes<T, DH, BWD>(a.num_pos_buckets);
  if (lds > 160 * 1024) return hipErrorInvalidConfiguration;
  if (grid == 0) {
    if constexpr (BWD) {   // no tokens: the bias-table gradients are 0
      const unsigned entries = (unsigned)(a.rab_rows * (a.num_pos_buckets + a.num_time_buckets));
      hipLaunchKernelGGL(attn_bias_grad_reduce_kernel, dim3(entries), dim3(256), 0, stream, a, 0);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  static LdsLimit lim;
  {
    const void *fn = BWD ? (const void *)attn_bwd_dq_kernel<T, DH> : (const void *)attn_fwd_kernel<T, DH, TO, CACHED>;
    hipError_t e = lim.raise(fn, 160 * 1024);
    if (e != hipSuccess) return e;
  }
  launch_tau_stats(a.seq_offsets, a.timestamps, a.tau_stats, a.num_seqs, a.num_rows_total, stream);
  if constexpr (CACHED)
    launch_tau_stats(a.hist_offsets, a.hist_timestamps, a.hist_tau_stats, a.num_seqs, a.num_hist_rows, stream);
  if constexpr (BWD)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DH>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a, n_qblocks);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, DH, TO, CACHED>), dim3((unsigned)grid), dim3(kThreads), lds, stream, a,
                       n_qblocks);
  if (CACHED && a.kv_splits > 1) {
    const long long n4 = (long long)a.num_rows * a.num_heads * DH / 4;
    hipLaunchKernelGGL(attn_split_reduce_kernel<TO>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, a,
                       a.num_heads * DH);
  }
  if constexpr (BWD) {
    const unsigned entries = (unsigned)(a.rab_rows * (a.num_pos_buckets + a.num_time_buckets));
    hipLaunchKernelGGL(attn_bias_grad_reduce_kernel, dim3(entries), dim3(256), 0, stream, a, (int)grid);
  }
  return hipGetLastError();
}

template <typename T, typename TO, bool CACHED, bool BWD = false>
hipError_t launch_dh(const AttnArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 32: return launch_typed<T, 32, TO, CACHED, BWD>(a, stream);
    case 64: return launch_typed<T, 64, TO, CACHED, BWD>(a, stream);
    case 128: return launch_typed<T, 128, TO, CACHED, BWD>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int attn_cached_splits(int64_t num_seqs, int64_t num_heads, int64_t max_candidates, int64_t max_history,
                       int32_t *tiles_per_split) {
  // about 1024 workgroups (two resident per CU, two rounds), at least 8 tiles per split so that the
  // partial sums (written once, read once) stay small against the tile work
  constexpr int64_t kTarget = 1024, kMinTiles = 8;
  const int64_t base = (max_candidates + kBM - 1) / kBM * num_heads * num_seqs;
  const int64_t tiles = (max_history + kBN - 1) / kBN;
  int64_t splits = 1;
  if (base > 0 && tiles >= 2 * kMinTiles) {
    splits = (kTarget + base - 1) / base;
    const int64_t cap = tiles / kMinTiles;
    splits = splits < cap ? splits : cap;
    splits = splits < 1 ? 1 : splits;
  }
  int64_t tps = splits > 1 ? (tiles + splits - 1) / splits : (tiles > 1 ? tiles : 1);
  if (splits > 1) splits = (tiles + tps - 1) / tps;   // no trailing empty split
  *tiles_per_split = (int32_t)tps;
  return (int)splits;
}

size_t attn_tau_stats_bytes(int64_t total_tokens, int64_t num_seqs) {
  return (size_t)((total_tokens >> 5) + num_seqs + 1) * 2 * sizeof(int64_t);
}

hipError_t launch_attn_fwd(const AttnArgs &a, hipStream_t stream) {
  if (a.in_dtype == kBF16) {
    return a.out_dtype == kBF16 ? launch_dh<__bf16, __bf16, false>(a, stream)
                                : launch_dh<__bf16, float, false>(a, stream);
  }
  return launch_dh<float, float, false>(a, stream);
}

hipError_t launch_attn_bwd_dq(const AttnArgs &a, hipStream_t stream) {
  if (a.in_dtype == kBF16) return launch_dh<__bf16, float, false, true>(a, stream);
  return launch_dh<float, float, false, true>(a, stream);
}

size_t attn_bwd_dq_lds_bytes(int in_dtype, int head_dim, int num_pos_buckets) {
  const bool bf = in_dtype == kBF16;
  const int P = num_pos_buckets;
  switch (head_dim) {
    case 32: return bf ? attn_lds_bytes<__bf16, 32, true>(P) : attn_lds_bytes<float, 32, true>(P);
    case 64: return bf ? attn_lds_bytes<__bf16, 64, true>(P) : attn_lds_bytes<float, 64, true>(P);
    default: return bf ? attn_lds_bytes<__bf16, 128, true>(P) : attn_lds_bytes<float, 128, true>(P);
  }
}

hipError_t launch_attn_cached(const AttnArgs &a, hipStream_t stream) {
  if (a.in_dtype == kBF16) {
    return a.out_dtype == kBF16 ? launch_dh<__bf16, __bf16, true>(a, stream)
                                : launch_dh<__bf16, float, true>(a, stream);
  }
  return launch_dh<float, float, true>(a, stream);
}

}  // namespace hstu
