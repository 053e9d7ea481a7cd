// Device pieces shared by the attention kernels of libhstu (forward, cached-history scoring and
// backward): tile shapes and LDS layouts, the score MFMA block, the per-score bias and mask, the
// folded SiLU and the transposed-operand MFMA block.  Included by attn_fwd.hip and attn_bwd.hip only.
#pragma once

#include "device_common.hpp"
#include "kernels.h"

namespace hstu {
namespace attn {

constexpr int kWaves = 4;
constexpr int kQW = 32;                  // queries per wave
constexpr int kBM = kWaves * kQW;        // queries per workgroup
constexpr int kBN = 64;                  // keys per LDS tile
constexpr int kThreads = kWaves * kWave;
constexpr int kTimeTab = 65;             // a 64-bit gap has bit length 0..64
constexpr int kTimeRev = 34;             // forward: the time table by leading-zero count of a 32-bit gap
constexpr int kPosPad = 8;               // forward: position-table entries past P - 1 (copies of w_p[P-1])
constexpr int kChunk = 32;               // tokens per timestamp-range chunk
constexpr int kRingBudget = 68 * 1024;   // LDS for the stage ring: two workgroups per CU
constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;
static_assert(kWaves * 16 == kBN, "each wave stages 16 rows of a tile");

// Tile classes.  A class code is body | (low time bucket << 8).
enum Body : int { kNone = 0, kUniform = 1, kTwo = 2, kGen32 = 3, kGen64 = 4, kGen32M = 5, kGen64M = 6, kTwoOrd = 7 };

// Row order of K inside each 32-row block of LDS: row r holds key kperm(r) (an involution swapping
// rows 4..7 with 8..11 and 20..23 with 24..27, i.e. bits 2 and 3 of r).  With it, accumulator element e
// of lane half hf holds key 16*(e/8) + 8*hf + e%8.
__device__ __forceinline__ int kperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <typename T, int DH>
struct Layout {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kES = sizeof(T);
  static constexpr int kRB = DH * kES;                 // bytes of one K or V row
  static constexpr int kG = kRB / 64;                  // 64-byte column groups per row
  static constexpr int kTileBytes = kBN * kRB;
  static constexpr int kOffK = 0;
  static constexpr int kOffV = kTileBytes;
  static constexpr int kOffTau = 2 * kTileBytes;       // wave w's 16 timestamps at 256*w (+128 B unused)
  static constexpr int kStageBytes = 2 * kTileBytes + kWaves * 256;
  static constexpr int kFit = kRingBudget / kStageBytes;
  static constexpr int kStages = kFit >= 4 ? 4 : (kFit >= 2 ? kFit : 2);   // at least double-buffered
  static constexpr int kLoadsPerTile = 2 * kG + 1;     // per wave: K and V column groups, timestamps
  static constexpr int kKPL = kBf16 ? 8 : 1;           // operand values per lane per MFMA
  static constexpr int kKStep = kBf16 ? 16 : 2;        // k per MFMA
  static constexpr int kQSteps = DH / kKStep;          // MFMAs per 32x32 score block
  static constexpr int kDB = DH / 32;                  // 32-row dh blocks of O^T
  static_assert(kStages >= 2, "ring");
  static_assert(kRB % 64 == 0, "rows of whole 64-byte groups");
  static_assert(kStageBytes % 16 == 0, "stage alignment");
  // LDS byte offset of byte b of row r in a V tile, and in a K tile (16-byte pieces XOR-permuted)
  __device__ static int v_at(int r, int b) { return (((b >> 6) * 64 + r) << 6) + (b & 63); }
  __device__ static int k_at(int r, int b) {
    return (((b >> 6) * 64 + r) << 6) + ((((b >> 4) & 3) ^ ((r >> 2) & 3)) << 4) + (b & 15);
  }
  // LDS byte offset (from the stage) of the timestamp of tile-local key j
  __device__ static int tau_at(int j) { return kOffTau + 256 * (j >> 4) + 8 * (j & 15); }
};

// The lane's index in its wave, recomputed at each use.  The volatile read is never hoisted or
// merged, so addresses derived from it are rebuilt in the loop body (a few VALU instructions) rather
// than held across the loop; near the register limit the compiler would spill them, and a reload from
// scratch waits on the vector-memory counter that also tracks the direct-to-LDS prefetch of the next
// tile, so every reload would wait for that prefetch.
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The O^T accumulators of one wave: N blocks of 32 dh rows x 32 queries.
template <int N>
struct OAcc {
  floatx16 d[N];
};

template <typename T> struct QFrag;
template <> struct QFrag<__bf16> { using type = bf16x8; };
template <> struct QFrag<float> { using type = float; };

__device__ __forceinline__ int bitlen_u32(uint32_t d) { return 32 - __clz((int)d); }  // __clz(0) = 32

// Column groups G..NG-1 of one row group of K and V: LDS group g sits at m + 4096*g; the immediate 64*g
// selects the source column group and is taken back out of M0.
template <int G, int NG>
__device__ __forceinline__ void dma_groups(const char *kb, const char *vb, uint32_t koff, uint32_t voff, uint32_t mk,
                                           uint32_t mv) {
  if constexpr (G < NG) {
    dma16<64 * G>(kb, koff, mk + (uint32_t)G * (4096u - 64u));
    dma16<64 * G>(vb, voff, mv + (uint32_t)G * (4096u - 64u));
    dma_groups<G + 1, NG>(kb, vb, koff, voff, mk, mv);
  }
}
__device__ __forceinline__ int readlane_i(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Per-wave constants of the score pointwise work for one tile.
struct TileCtx {
  int k0;              // first key of the tile (sequence-local)
  int my_q, my_pos;    // this lane's query and its position
  int pos_lim;         // position of key j is min(j, pos_lim): n_h with candidates, else n
  int key_lim;         // allowed keys of this lane's query: j <= key_lim, or j == my_q
  int nh;              // history length
  int P, Tb;
  int64_t my_tau;
  uint32_t qoff;       // (uint32)(my_tau - base) for the 32-bit modes
  uint32_t qlo;        // low word of my_tau (two-bucket tiles whose keys are no later than their queries)
  uint32_t base_lo;    // low word of the tile's timestamp base
  uint32_t thr;        // two-bucket mode: |dt| >= thr selects bias_hi
  int blo;             // two-bucket mode: the lower time bucket (the upper one is blo + 1)
  float c1;            // -log2(e) * bias of a uniform tile, 0 otherwise
  float bias_lo, bias_hi;          // two-bucket mode: the two biases
  const HSTU_LDS float *wp, *wt;   // bias tables
  const HSTU_LDS float *wtr;       // forward: wtr[z] = time bias of a 32-bit gap with v_ffbh_u32 = z (-1 for 0)
  const HSTU_LDS char *stage;      // the tile's LDS stage
};

// Score of a pair outside the mask: its folded SiLU u / (1 + 2^u) is exactly 0 (u = 1.4e30 is finite, 2^u
// overflows to +inf, the reciprocal of 1 + inf is 0 and u * 0 = 0), and adding a finite q.k keeps it there.
constexpr float kMaskedScore = -1.0e30f;

// Per-score bias and mask of a non-uniform tile, added to the 16 scores of 32-key block kb in place;
// element e holds key k0 + 32*kb + 16*(e/8) + 8*half + e%8.
// BINS: also return each score's position and time bucket for the bias-table gradients, packed as
// bp | (bt << 16) (bp < 4096, bt <= 64).
template <typename T, int DH, int MODE, bool BINS = false>
__device__ __forceinline__ void adjust_block(floatx16 &s, const TileCtx &c, int kb, int half,
                                             int *bins_out = nullptr) {
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
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const int e = 8 * g + e8;
      float bias;
      if constexpr (MODE == kTwo) {
        const uint32_t d = __usad(c.qoff, lo[e8] - c.base_lo, 0u);
        bias = d >= c.thr ? c.bias_hi : c.bias_lo;
        if constexpr (BINS) bins_out[e] = (c.P - 1) | ((d >= c.thr ? c.blo + 1 : c.blo) << 16);
      } else {
        const int j = c.k0 + jl0 + e8;
        const int pj = imin(j, c.pos_lim);
        const uint32_t dp = __usad((uint32_t)c.my_pos, (uint32_t)pj, 0u);
        const int bp = (int)(dp < (uint32_t)(c.P - 1) ? dp : (uint32_t)(c.P - 1));
        int bt;
        if constexpr (!k64) {
          bt = bitlen_u32(__usad(c.qoff, lo[e8] - c.base_lo, 0u));
        } else {
          const int64_t tj = (int64_t)(((uint64_t)hi[e8] << 32) | lo[e8]);
          bt = bitlen_absdiff(c.my_tau, tj);
        }
        bt = imin(bt, c.Tb - 1);
        bias = c.wp[bp] + c.wt[bt];
        if constexpr (BINS) bins_out[e] = bp | (bt << 16);
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

// LDS offsets of the A operand of k step st of score_block in a K-layout tile (bf16): row
// r = 32*kb + kperm(l32), byte 32*st + 16*half.  The XOR of the layout sees bits 2-3 of the row (kb
// never changes them) and the piece index 2*(st&1) + half, so every step is one of two lane parts
// plus 2048*kb + 4096*(st/2).
struct ScoreAddr {
  int even, odd;
};
template <int DH>
__device__ __forceinline__ ScoreAddr score_addr(int l32, int half) {
  using L = Layout<__bf16, DH>;
  return {L::k_at(kperm(l32), 16 * half), L::k_at(kperm(l32), 32 + 16 * half)};
}

template <typename T, int DH>
__device__ __forceinline__ void score_block(floatx16 &s, const HSTU_LDS char *lK, int kb, int l32, int half,
                                            const typename QFrag<T>::type (&qf)[Layout<T, DH>::kQSteps]) {
  using L = Layout<T, DH>;
  const int r = 32 * kb + kperm(l32);   // MFMA row l32 takes key kperm(l32) of this 32-key block
  s = floatx16{};
#pragma unroll
  for (int st = 0; st < L::kQSteps; ++st) {
    if constexpr (L::kBf16) {
      const ScoreAddr sa = score_addr<DH>(l32, half);
      const int off = ((st & 1) ? sa.odd : sa.even) + 2048 * kb + 4096 * (st >> 1);
      const bf16x8 kf = *(const HSTU_LDS bf16x8 *)(lK + off);
      s = mfma32(kf, qf[st], s);
    } else {
      const float kf = *(const HSTU_LDS float *)(lK + L::k_at(r, (2 * st + half) * 4));
      s = mfma32(kf, qf[st], s);
    }
  }
}

// O^T += X^T a^T for one 32-key block: X^T read transposed from a tile in the V layout, or (XL) in the
// K layout (the backward's dQ^T += K^T dS^T reads the K tile this way).
template <int DH, bool XL>
__device__ __forceinline__ void av_block_packed(OAcc<Layout<__bf16, DH>::kDB> &oacc, const bf16x8 (&pf)[2],
                                                const HSTU_LDS char *lV, int kb, int lane);

template <typename T, int DH, bool XL>
__device__ __forceinline__ void av_block_in(OAcc<Layout<T, DH>::kDB> &oacc, const float (&a)[16],
                                            const HSTU_LDS char *lV, int kb, int lane) {
  using L = Layout<T, DH>;
  const auto at = [](int r, int b) { return XL ? L::k_at(r, b) : L::v_at(r, b); };
  const int l32 = lane & 31, half = lane >> 5;
  if constexpr (L::kBf16 && XL) {
    bf16x8 pf[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) pf[e / 8][e % 8] = f32_to_bf16(a[e]);
    av_block_packed<DH, XL>(oacc, pf, lV, kb, lane);
  } else if constexpr (L::kBf16) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = f32_to_bf16(a[8 * s2 + e]);
      const int g16 = lane >> 4, i16 = lane & 15;
      const int r0 = 32 * kb + 16 * s2 + 8 * half + (i16 >> 2);
#pragma unroll
      for (int db = 0; db < L::kDB; ++db) {
        const int b = (32 * db + 16 * (g16 & 1) + 4 * (i16 & 3)) * 2;
        const shortx4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HSTU_LDS shortx4 *)(lV + at(r0, b)));
        const shortx4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HSTU_LDS shortx4 *)(lV + at(r0 + 4, b)));
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
      const int r = 32 * kb + 16 * (e / 8) + 8 * half + (e % 8);
#pragma unroll
      for (int db = 0; db < L::kDB; ++db) {
        const float vf = *(const HSTU_LDS float *)(lV + at(r, (32 * db + l32) * 4));
        oacc.d[db] = mfma32(vf, a[e], oacc.d[db]);
      }
    }
  }
}

// av_block_in with the bf16 operand already packed (pf[s2] holds a[8*s2 .. 8*s2+7], rounded).
template <int DH, bool XL>
__device__ __forceinline__ void av_block_packed(OAcc<Layout<__bf16, DH>::kDB> &oacc, const bf16x8 (&pf)[2],
                                                const HSTU_LDS char *lV, int kb, int lane) {
  using L = Layout<__bf16, DH>;
  const auto at = [](int r, int b) { return XL ? L::k_at(r, b) : L::v_at(r, b); };
  // Row r0 + 16*s2 + 32*kb and byte b0 + 64*db of either layout lie at a lane part plus
  // 64*(16*s2 + 32*kb) + 4096*db: the XOR of the K layout reads only bits 2-3 of the row and bits 4-5
  // of the byte, which those steps never change.  Two lane parts serve every read of the block.
  const int half = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
  const int r0 = 8 * half + (i16 >> 2), b0 = (16 * (g16 & 1) + 4 * (i16 & 3)) * 2;
  const HSTU_LDS char *p0 = lV + at(r0, b0) + 2048 * kb;
  const HSTU_LDS char *p1 = lV + at(r0 + 4, b0) + 2048 * kb;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
    for (int db = 0; db < L::kDB; ++db) {
      const int step = 1024 * s2 + 4096 * db;
      const shortx4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HSTU_LDS shortx4 *)(p0 + step));
      const shortx4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HSTU_LDS shortx4 *)(p1 + step));
      const bf16x4 w0 = __builtin_bit_cast(bf16x4, v0), w1 = __builtin_bit_cast(bf16x4, v1);
      bf16x8 vf;
      vf[0] = w0[0]; vf[1] = w0[1]; vf[2] = w0[2]; vf[3] = w0[3];
      vf[4] = w1[0]; vf[5] = w1[1]; vf[6] = w1[2]; vf[7] = w1[3];
      oacc.d[db] = mfma32(vf, pf[s2], oacc.d[db]);
    }
  }
}

template <typename T, int DH>
__device__ __forceinline__ void av_block(OAcc<Layout<T, DH>::kDB> &oacc, const float (&a)[16],
                                         const HSTU_LDS char *lV, int kb, int lane) {
  av_block_in<T, DH, false>(oacc, a, lV, kb, lane);
}

// dz = g * SiLU'(z) for four consecutive elements, in place over z (the layer backward's gradient of
// the projection's pre-activation); SiLU'(z) = sigma (1 + z (1 - sigma)), sigma = 1 / (1 + 2^(-z log2 e)).
template <typename T>
__device__ __forceinline__ void silu_grad_store4(T *z, const float (&g)[4]) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float zz = to_f32(z[x]);
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(zz * kNegLog2e));
    z[x] = from_f32<T>(g[x] * sg * fmaf(zz, 1.0f - sg, 1.0f));
  }
}

}  // namespace attn
}  // namespace hstu
