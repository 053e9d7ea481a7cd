// MFMA GEMMs of the HSTU layer on gfx950: C[M][N] = A[M][K] . B[N][K]^T with fused epilogues.
//
//  * projection:  U|V|Q|K = SiLU(X W1^T + b1), the four H*Dh column slices written to four buffers
//    (one projection makes every internal representation of the layer: "DLRMv4：MLPerfの推薦システム
//    訓練ベンチマークがシーケンス化時代へ", section "モデルアーキテクチャ").  U, used only by the
//    elementwise gate, is kept in fp32; V, Q, K are stored in the MFMA operand type.
//  * output:      y = x + G W2^T + b2 (residual added in fp32, one rounding), or the fp32 sum for a
//    following LayerNorm pass, with the gate G = LN(O) * U (the gated transformation of the same
//    section) computed while the A operand is loaded: the rows' LayerNorm statistics are combined
//    from the per-head partial statistics the attention kernel stored next to O, and each A element
//    is (o - mean) * rstd * u.  G is never stored.
//  * stack:       the projection and output GEMMs of a layer stack over embedding-table rows (the layer
//    input is looked up from embedding tables, same section): layer 0 reads its operand and residual
//    rows through the row ids (the gather is never stored); a layer followed by a LayerNorm writes its
//    fp32 sum with per-row statistics of each 256-column tile, and the next layer normalises those rows
//    while loading them (the LayerNorm output is never stored).
//  * plain:       c = A B^T (+ residual), optionally split over K into fp32 partial products that are
//    summed in split order (the weight gradients of the layer backward, whose K is the token count).
//
// Both operands are K-contiguous (row-major activations, torch-Linear [out][in] weights), which is the
// native operand form of the 32x32 MFMAs.  Two kernels:
//  * gemm_big_kernel (bf16 weights, K a whole number of k-tiles, at least 256 tiles): large tiles,
//    direct-to-LDS staging, fp32 activations converted while fragments are read, XCD-aware tile order;
//    described where it is defined.
//  * gemm_kernel (everything else: fp32 weights, small or odd shapes): workgroup tile 128x128, k-tile 32,
//    4 waves in a 2x2 grid, each wave 64x64 (2x2 MFMA tiles); register staging, LDS double-buffered
//    with one barrier per k-tile.
//
// Activation operand precision.  With bf16 weights the activation A may be stored in fp32; it is then
// rounded to bf16 on the way into LDS, or (SPLIT = 2) split into hi = bf16(a) and lo = bf16(a - hi),
// and both halves are multiplied with the same weight fragment.  The pair carries ~16 significant
// bits, so the product is as accurate as fp32 activations times bf16 weights, at two MFMAs per step.
#include "device_common.hpp"
#include "kernels.h"

namespace hstu {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kThreads = 256;

// Epilogues: the projection's SiLU + U|V|Q|K split; the output's bias + residual (plain rows); the
// stack's output (residual rows gathered or LayerNorm-ed, per-row tile statistics for the next LN).
enum Epi : int { kEpiUvqk = 0, kEpiOut = 1, kEpiOutStack = 2 };

// TM: MFMA operand / weight type.  TA: storage type of the activation A.  SPLIT: 1 or 2 A terms.
template <typename TM, typename TA, int SPLIT>
struct GLayout {
  static constexpr bool kBf16 = sizeof(TM) == 2;
  static constexpr bool kConvA = kBf16 && sizeof(TA) == 4;       // fp32 A rounded/split to bf16
  static constexpr int kMS = sizeof(TM);
  static constexpr int kRowBytes = kBK * kMS;                    // LDS bytes of one row of one k-tile
  static constexpr int kStride = kBf16 ? kRowBytes + 16 : kRowBytes + 4;
  static constexpr int kElemsPerChunk = 16 / kMS;                // elements per 16-byte LDS chunk
  static constexpr int kChunksPerRow = kBK / kElemsPerChunk;
  static constexpr int kCPT = kBM * kChunksPerRow / kThreads;    // chunks per thread per operand
  static constexpr int kOpBytes = kBM * kStride;
  static constexpr int kATerms = kConvA ? SPLIT : 1;
  static constexpr int kStageBytes = ((kATerms + 1) * kOpBytes + 15) & ~15;
  static constexpr int kKStep = kBf16 ? 16 : 2;
  static constexpr int kSteps = kBK / kKStep;
  static_assert(kBM * kChunksPerRow % kThreads == 0, "staging split");
  static_assert(SPLIT == 1 || kConvA, "a split A needs fp32 storage and bf16 MFMA");
};

template <typename T> struct Frag;
template <> struct Frag<__bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = float; };

struct GemmParams {
  const void *a;       // [M][K] (TA); with the fused gate: O, fp32
  const void *b;       // [N][K] (TM)
  const void *bias;    // [N] (TM) or null
  const void *resid;   // [M][N] residual (output epilogue), fp32 if resid_f32 else TM
  void *out0, *out1, *out2, *out3;  // projection: U (fp32), V, Q, K (TM), [M][HD]; output: y or null
  void *zout;          // projection: the pre-activation x W1^T + b1, [M][N] (TM), or null
  float *out32;        // output epilogue: fp32 result (pre-LayerNorm; per split with split-K) or null
  int M, N, K, HD;
  int splits, kt_per_split;  // split-K (large-tile kernel only): k-tiles [s * kt_per_split, ...) per split
  int resid_f32, y_f32;
  const float *gate_u;     // fused gate: U [M][K] fp32
  const float *row_stats;  // fused gate: [M][heads][2] per-head mean and sum of squared deviations of O
  int heads, head_dim;
  float eps;
  // large-tile kernel only:
  const int64_t *ids;      // gathered rows: A row m (kAkGather) and residual row m (resid_mode 1) are row
                           // ids[m] of a [rows][K] (A) or [rows][N] (residual) bf16 table
  int64_t id_rows;         // the table's row count: ids are clamped into [0, id_rows)
  unsigned int *id_err;    // id-error word: +1 per clamped read
  const float *a_rowstat;  // kAkLn: [M][2] (mean, rstd) of A's rows
  int resid_mode;          // 0: resid [M][N]; 1: bf16 table rows resid[ids[m]]; 2: LN of fp32 resid rows
  const float *resid_rowstat;  // resid_mode 2: [M][2] (mean, rstd)
  float *out_stats;        // output epilogue with out32: [M][ceil(N/BN)][2] per-row (mean, M2) of each column tile
};

// Staging registers of one 16-byte LDS chunk of A: the global source is 16 bytes (TA == TM) or
// 32 bytes (fp32 A converted to bf16).
template <typename TM, typename TA>
struct AChunk;
template <typename T>
struct AChunk<T, T> {
  u32x4 v;
};
template <>
struct AChunk<__bf16, float> {
  floatx4 lo, hi;  // 8 consecutive fp32 values
};

template <typename TM, typename TA, int SPLIT, int EPI, bool GATE>
__global__ void __launch_bounds__(kThreads) gemm_kernel(const GemmParams p) {
  using L = GLayout<TM, TA, SPLIT>;
  using F = typename Frag<TM>::type;
  static_assert(!GATE || sizeof(TA) == 4, "the fused gate reads fp32 O and U");
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * L::kStageBytes];
  __shared__ float row_norm[GATE ? 2 * kBM : 2];   // fused gate: (mean, rstd) of the tile's rows
  HSTU_LDS char *smem = (HSTU_LDS char *)smem_raw;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, l32 = lane & 31, half = lane >> 5;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  if constexpr (GATE) {
    // LayerNorm statistics of the row from its heads' (mean, M2): equal counts per head, so the row
    // mean is the mean of the head means and M2 = sum(M2_h + Dh (mean_h - mean)^2)
    if (tid < kBM) {
      const int m = m0 + tid;
      float mean = 0.0f, rstd = 0.0f;
      if (m < p.M) {
        const float *st = p.row_stats + (int64_t)m * p.heads * 2;
        float s = 0.0f;
        for (int hh = 0; hh < p.heads; ++hh) s += st[2 * hh];
        mean = s / (float)p.heads;
        float m2 = 0.0f;
        for (int hh = 0; hh < p.heads; ++hh) {
          const float d = st[2 * hh] - mean;
          m2 += st[2 * hh + 1] + (float)p.head_dim * d * d;
        }
        rstd = 1.0f / sqrtf(m2 / (float)(p.heads * p.head_dim) + p.eps);
      }
      row_norm[2 * tid] = mean;
      row_norm[2 * tid + 1] = rstd;
    }
    __syncthreads();
  }

  AChunk<TM, TA> areg[L::kCPT];
  u32x4 breg[L::kCPT];
  auto load = [&](int k0) {
#pragma unroll
    for (int c = 0; c < L::kCPT; ++c) {
      const int chunk = tid + c * kThreads;
      const int row = chunk / L::kChunksPerRow, col = chunk % L::kChunksPerRow;
      const int kk = k0 + col * L::kElemsPerChunk;
      const bool kok = kk < p.K;
      {
        const int m = m0 + row;
        const bool ok = kok && m < p.M;
        const int64_t aoff = (int64_t)(ok ? m : 0) * p.K + (ok ? kk : 0);
        const TA *src = (const TA *)p.a + aoff;
        if constexpr (GATE) {
          // g = (o - mean) * rstd * u for the chunk's 8 (bf16 operand) or 4 (fp32 operand) columns
          const float mean = row_norm[2 * row], rstd = row_norm[2 * row + 1];
          const float *usrc = p.gate_u + aoff;
          floatx4 g0 = (*(const floatx4 *)src - mean) * rstd * *(const floatx4 *)usrc;
          if constexpr (L::kConvA) {
            floatx4 g1 = (*(const floatx4 *)(src + 4) - mean) * rstd * *(const floatx4 *)(usrc + 4);
            areg[c].lo = ok ? g0 : floatx4{};
            areg[c].hi = ok ? g1 : floatx4{};
          } else {
            if (!ok) g0 = floatx4{};
            areg[c].v = __builtin_bit_cast(u32x4, g0);
          }
        } else if constexpr (L::kConvA) {
          const floatx4 a0 = *(const floatx4 *)src, a1 = *(const floatx4 *)(src + 4);
          areg[c].lo = ok ? a0 : floatx4{};
          areg[c].hi = ok ? a1 : floatx4{};
        } else {
          const u32x4 v = *(const u32x4 *)src;
          areg[c].v = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
      }
      {
        const int nn = n0 + row;
        const bool ok = kok && nn < p.N;
        const TM *src = (const TM *)p.b + (int64_t)(ok ? nn : 0) * p.K + (ok ? kk : 0);
        const u32x4 v = *(const u32x4 *)src;
        breg[c] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store = [&](int stage) {
    HSTU_LDS char *base = smem + stage * L::kStageBytes;
#pragma unroll
    for (int c = 0; c < L::kCPT; ++c) {
      const int chunk = tid + c * kThreads;
      const int row = chunk / L::kChunksPerRow, col = chunk % L::kChunksPerRow;
      const int off = row * L::kStride + col * 16;
      HSTU_LDS char *db = base + L::kATerms * L::kOpBytes + off;
      if constexpr (L::kConvA) {
        bf16x8 h8, l8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = e < 4 ? areg[c].lo[e] : areg[c].hi[e - 4];
          const __bf16 h = f32_to_bf16(a);
          h8[e] = h;
          if constexpr (SPLIT == 2) l8[e] = f32_to_bf16(a - bf16_to_f32(h));
        }
        *(HSTU_LDS bf16x8 *)(base + off) = h8;
        if constexpr (SPLIT == 2) *(HSTU_LDS bf16x8 *)(base + L::kOpBytes + off) = l8;
        *(HSTU_LDS u32x4 *)db = breg[c];
      } else if constexpr (L::kBf16) {
        *(HSTU_LDS u32x4 *)(base + off) = areg[c].v;
        *(HSTU_LDS u32x4 *)db = breg[c];
      } else {
        HSTU_LDS uint32_t *x = (HSTU_LDS uint32_t *)(base + off);
        x[0] = areg[c].v.x; x[1] = areg[c].v.y; x[2] = areg[c].v.z; x[3] = areg[c].v.w;
        HSTU_LDS uint32_t *y = (HSTU_LDS uint32_t *)db;
        y[0] = breg[c].x; y[1] = breg[c].y; y[2] = breg[c].z; y[3] = breg[c].w;
      }
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  const int nk = (p.K + kBK - 1) / kBK;
  load(0);
  store(0);
  __syncthreads();
  int stage = 0;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load((kt + 1) * kBK);
    const HSTU_LDS char *base = smem + stage * L::kStageBytes;
    const HSTU_LDS char *bbase = base + L::kATerms * L::kOpBytes;
#pragma unroll
    for (int st = 0; st < L::kSteps; ++st) {
      F af[L::kATerms][2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = wm + 32 * i + l32, rb = wn + 32 * i + l32;
        if constexpr (L::kBf16) {
#pragma unroll
          for (int t = 0; t < L::kATerms; ++t)
            af[t][i] = *(const HSTU_LDS bf16x8 *)(base + t * L::kOpBytes + ra * L::kStride + (16 * st + 8 * half) * 2);
          bfr[i] = *(const HSTU_LDS bf16x8 *)(bbase + rb * L::kStride + (16 * st + 8 * half) * 2);
        } else {
          af[0][i] = *(const HSTU_LDS float *)(base + ra * L::kStride + (2 * st + half) * 4);
          bfr[i] = *(const HSTU_LDS float *)(bbase + rb * L::kStride + (2 * st + half) * 4);
        }
      }
#pragma unroll
      for (int t = 0; t < L::kATerms; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[t][i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) store(stage ^ 1);
    __syncthreads();
    stage ^= 1;
  }

  // epilogue: acc[i][j] element e -> row m = m0 + wm + 32i + 8*(e/4) + 4*half + e%4, col n = n0 + wn + 32j + l32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn + 32 * j + l32;
    if (n >= p.N) continue;
    const float bias = p.bias ? to_f32(((const TM *)p.bias)[n]) : 0.0f;
    if constexpr (EPI == kEpiUvqk) {
      const int part = n / p.HD, col = n % p.HD;
      void *dst = part == 0 ? p.out0 : part == 1 ? p.out1 : part == 2 ? p.out2 : p.out3;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4);
          if (m < p.M) {
            const float z = acc[i][j][e] + bias;
            const float s = silu_f32(z);
            const int64_t idx = (int64_t)m * p.HD + col;
            if (part == 0) ((float *)dst)[idx] = s;
            else ((TM *)dst)[idx] = from_f32<TM>(s);
            if (p.zout) ((TM *)p.zout)[(int64_t)m * p.N + n] = from_f32<TM>(z);
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // the 16 residuals of the fragment are loaded (rows clamped into the matrix) before any is used
        float r[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = imin(m0 + wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4), p.M - 1);
          const int64_t idx = (int64_t)m * p.N + n;
          if (!p.resid) r[e] = 0.0f;
          else r[e] = p.resid_f32 ? ((const float *)p.resid)[idx] : to_f32(((const TM *)p.resid)[idx]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4);
          if (m < p.M) {
            const int64_t idx = (int64_t)m * p.N + n;
            const float y = acc[i][j][e] + bias + r[e];
            if (p.out32) p.out32[idx] = y;
            else if (p.y_f32) ((float *)p.out0)[idx] = y;
            else ((TM *)p.out0)[idx] = from_f32<TM>(y);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------------
// Large-tile kernel for bf16 weights and K a multiple of BK.
//
// Workgroup tile BM x BN in 4 waves of (BM/WM) x (BN/WN), two workgroups per CU; every operand goes
// global -> LDS with direct-to-LDS loads into an S-stage ring, one barrier per k-tile.  LDS holds each
// operand tile column-group-major: the BK-wide slice of a row is cut into 64-byte groups, and group g of
// row r sits at (g * R + r) * 64 with its four 16-byte pieces XOR-permuted by bits 2..3 of r, so that one
// 1 KB direct-to-LDS load fills 16 rows of one group and the 16 rows one fragment read touches land in
// 16 distinct bank groups.  An fp32 activation (AK = kAkF32) or the gate's O and U (AK = kAkGate) are
// staged as fp32 and turned into the bf16 operand (rounded, or split into hi + lo) while the fragment
// is read, so no VALU work or registers are spent on staging.  Workgroups are dealt to the 8 XCDs
// round-robin; the tile order gives each XCD a contiguous range of tiles, walked in groups of GM row
// blocks, so that the workgroups resident on one XCD share A and B slices in its L2.
//
// The configurations below use 128 x 256 tiles (64 x 256 for the gate, whose A operand is 8 bytes per
// element) with 2 x 2 waves and two workgroups per CU: one workgroup's barrier waits, prologue and
// epilogue overlap the other's MFMA work, which single-workgroup 256 x 256 tiles cannot hide.
// A operand kinds: bf16 rows; fp32 rows; the gate LN(O) * U from fp32 O and U; bf16 rows gathered
// through a row-index array (an embedding table); fp32 rows normalised per row with precomputed
// (mean, rstd) (a LayerNorm applied while the operand is read).
enum AKind : int { kAkBf16 = 0, kAkF32 = 1, kAkGate = 2, kAkGather = 3, kAkLn = 4 };

template <int BM_, int BN_, int BK_, int S_, int WM_, int WN_, int AK_, int SPLIT_, int GM_, int OCC_ = 1>
struct BigCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_, WM = WM_, WN = WN_, AK = AK_, GM = GM_;
  static constexpr int kOcc = OCC_;                                 // workgroups per CU
  static constexpr bool kA16 = AK == kAkBf16 || AK == kAkGather;   // A staged as bf16
  static constexpr int kTerms = (!kA16 && SPLIT_ == 2) ? 2 : 1;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  static constexpr int kEA = kA16 ? 2 : 4;                          // A element bytes (global and LDS)
  static constexpr int kABytes = BM * BK * kEA;
  static constexpr int kUBytes = AK == kAkGate ? BM * BK * 4 : 0;
  static constexpr int kBBytes = BN * BK * 2;
  static constexpr int kStage = kABytes + kUBytes + kBBytes;
  static constexpr int kDA = kABytes / 1024 / kWaves, kDU = kUBytes / 1024 / kWaves, kDB = kBBytes / 1024 / kWaves;
  static constexpr int kD = kDA + kDU + kDB;                        // direct-to-LDS loads per wave per stage
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  static constexpr int kSteps = BK / 16;
  static constexpr int kLds = S * kStage;
  static_assert((BK * kEA) % 64 == 0 && (BK * 2) % 64 == 0, "whole 64-byte column groups");
  static_assert(kABytes % (1024 * kWaves) == 0 && kUBytes % (1024 * kWaves) == 0 &&
                kBBytes % (1024 * kWaves) == 0, "loads split evenly over the waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32x32 fragments");
  static_assert(S >= 2 && S <= 4 && (S - 2) * kD < 64, "ring depth");
  static_assert(kLds * kOcc <= 160 * 1024, "LDS");
};

// LDS byte offset of 16-byte piece p (0..3) of column group g of row r, in a tile of R rows
template <int R>
__device__ __forceinline__ int cg_at(int r, int g, int p) {
  return ((g * R + r) << 6) + ((p ^ ((r >> 2) & 3)) << 4);
}

// Eight fp32 values to bf16 (round to nearest even, two values per v_cvt_pk_bf16_f32), and the bf16
// residuals x - hi, read back from the packed words without a second conversion.
__device__ __forceinline__ u32x4 to_bf16x8(floatx4 x0, floatx4 x1) {
  u32x4 h;
  h.x = __builtin_bit_cast(uint32_t, bf16x2{f32_to_bf16(x0[0]), f32_to_bf16(x0[1])});
  h.y = __builtin_bit_cast(uint32_t, bf16x2{f32_to_bf16(x0[2]), f32_to_bf16(x0[3])});
  h.z = __builtin_bit_cast(uint32_t, bf16x2{f32_to_bf16(x1[0]), f32_to_bf16(x1[1])});
  h.w = __builtin_bit_cast(uint32_t, bf16x2{f32_to_bf16(x1[2]), f32_to_bf16(x1[3])});
  return h;
}
__device__ __forceinline__ float lo_half_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_half_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ u32x4 residual_bf16x8(floatx4 x0, floatx4 x1, u32x4 h) {
  floatx4 r0, r1;
  r0[0] = x0[0] - lo_half_f32(h.x); r0[1] = x0[1] - hi_half_f32(h.x);
  r0[2] = x0[2] - lo_half_f32(h.y); r0[3] = x0[3] - hi_half_f32(h.y);
  r1[0] = x1[0] - lo_half_f32(h.z); r1[1] = x1[1] - hi_half_f32(h.z);
  r1[2] = x1[2] - lo_half_f32(h.w); r1[3] = x1[3] - hi_half_f32(h.w);
  return to_bf16x8(r0, r1);
}

// A workgroup-uniform pointer, moved into scalar registers
__device__ __forceinline__ const char *uniform_ptr(const char *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <class C, int EPI>
__global__ void __launch_bounds__(C::kThreads, C::kOcc) gemm_big_kernel(const GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  HSTU_LDS char *smem = (HSTU_LDS char *)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, FM = C::FM, FN = C::FN;

  // ---- tile: XCD-contiguous ranges, groups of GM row blocks, row block fastest inside a group
  const int nN = (p.N + BN - 1) / BN, nM = (p.M + BM - 1) / BM, tiles = nN * nM, total = tiles * p.splits;
  const int per = (total + 7) / 8;
  const int ws = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (ws >= total) return;
  const int split = ws / tiles, w = ws % tiles;      // split-K: each split is a full set of tiles
  const int kt0 = split * p.kt_per_split;
  float *const out32 = p.out32 ? p.out32 + (int64_t)split * p.M * p.N : nullptr;
  const int grp = w / (C::GM * nN), gi = w % (C::GM * nN);
  const int gm = imin(C::GM, nM - grp * C::GM);
  const int m0 = (grp * C::GM + gi % gm) * BM, n0 = (gi / gm) * BN;

  const int tid = threadIdx.x, lane = tid % 64, l32 = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // wave-uniform: LDS addresses go to M0
  const int wm = (wave / C::WN) * C::TM, wn = (wave % C::WN) * C::TN;

  // ---- per-lane source offsets of this wave's direct-to-LDS blocks (rows clamped into the matrix)
  const int lrow = lane >> 2;
  const uint32_t lpiece = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  const int a_rows = imin(BM, p.M - m0), b_rows = imin(BN, p.N - n0);
  const uint32_t a_rb = (uint32_t)p.K * C::kEA, b_rb = (uint32_t)p.K * 2u;
  uint32_t aoff[C::kDA], boff[C::kDB];
#pragma unroll
  for (int t = 0; t < C::kDA; ++t) {
    const int q = wave + t * C::kWaves, g = q / (BM / 16), r = (q % (BM / 16)) * 16 + lrow;
    aoff[t] = (uint32_t)imin(r, a_rows - 1) * a_rb + (uint32_t)g * 64u + lpiece;
  }
#pragma unroll
  for (int t = 0; t < C::kDB; ++t) {
    const int q = wave + t * C::kWaves, g = q / (BN / 16), r = (q % (BN / 16)) * 16 + lrow;
    boff[t] = (uint32_t)imin(r, b_rows - 1) * b_rb + (uint32_t)g * 64u + lpiece;
  }
  // workgroup-uniform operand bases (scalar registers: the direct-to-LDS loads take them as SGPR pairs)
  const char *abase = uniform_ptr((const char *)p.a + (int64_t)m0 * a_rb + (int64_t)kt0 * BK * C::kEA);
  // gathered A rows: per-lane 64-bit source addresses (the table can exceed 4 GB)
  const char *aptr[C::AK == kAkGather ? C::kDA : 1];
  if constexpr (C::AK == kAkGather) {
#pragma unroll
    for (int t = 0; t < C::kDA; ++t) {
      const int q = wave + t * C::kWaves, g = q / (BM / 16), r = (q % (BM / 16)) * 16 + lrow;
      const int64_t row = checked_row_id(p.ids[m0 + imin(r, a_rows - 1)], p.id_rows, p.id_err);
      aptr[t] = (const char *)p.a + row * (int64_t)a_rb + (int64_t)kt0 * BK * 2 + g * 64 + lpiece;
    }
  }
  const char *ubase = uniform_ptr((const char *)p.gate_u + (int64_t)m0 * a_rb + (int64_t)kt0 * BK * 4);
  const char *bbase = uniform_ptr((const char *)p.b + (int64_t)n0 * b_rb + (int64_t)kt0 * BK * 2);

  auto issue = [&](int kt, int slot) {
    const uint32_t st = smem_addr + (uint32_t)(slot * C::kStage);
    if constexpr (C::AK == kAkGather) {
#pragma unroll
      for (int t = 0; t < C::kDA; ++t)
        dma16_at(aptr[t] + (int64_t)kt * BK * 2, st + (uint32_t)((wave + t * C::kWaves) * 1024));
    } else {
      const char *ab = abase + (int64_t)kt * BK * C::kEA;
#pragma unroll
      for (int t = 0; t < C::kDA; ++t) dma16<0>(ab, aoff[t], st + (uint32_t)((wave + t * C::kWaves) * 1024));
    }
    if constexpr (C::AK == kAkGate) {
      const char *ub = ubase + (int64_t)kt * BK * 4;
#pragma unroll
      for (int t = 0; t < C::kDU; ++t)
        dma16<0>(ub, aoff[t], st + (uint32_t)(C::kABytes + (wave + t * C::kWaves) * 1024));
    }
    const char *bb = bbase + (int64_t)kt * BK * 2;
#pragma unroll
    for (int t = 0; t < C::kDB; ++t)
      dma16<0>(bb, boff[t], st + (uint32_t)(C::kABytes + C::kUBytes + (wave + t * C::kWaves) * 1024));
  };

  // ---- gate: LayerNorm statistics of this lane's A rows, from the per-head (mean, M2) pairs
  constexpr bool kNorm = C::AK == kAkGate || C::AK == kAkLn;
  float rstd[kNorm ? FM : 1], nmr[kNorm ? FM : 1];
  if constexpr (C::AK == kAkLn) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = imin(m0 + wm + 32 * i + l32, p.M - 1);
      const float mean = p.a_rowstat[2 * (int64_t)m], rs = p.a_rowstat[2 * (int64_t)m + 1];
      rstd[i] = rs;
      nmr[i] = -mean * rs;
    }
  }
  if constexpr (C::AK == kAkGate) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = imin(m0 + wm + 32 * i + l32, p.M - 1);
      const float *st = p.row_stats + (int64_t)m * p.heads * 2;
      float s = 0.0f;
      for (int hh = 0; hh < p.heads; ++hh) s += st[2 * hh];
      const float mean = s / (float)p.heads;
      float m2 = 0.0f;
      for (int hh = 0; hh < p.heads; ++hh) {
        const float d = st[2 * hh] - mean;
        m2 += st[2 * hh + 1] + (float)p.head_dim * d * d;
      }
      rstd[i] = 1.0f / sqrtf(m2 / (float)(p.heads * p.head_dim) + p.eps);
      nmr[i] = -mean * rstd[i];
    }
  }

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

  auto compute = [&](int slot) {
    const HSTU_LDS char *As = smem + slot * C::kStage;
    const HSTU_LDS char *Us = As + C::kABytes;
    const HSTU_LDS char *Bs = As + C::kABytes + C::kUBytes;
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      bf16x8 bfr[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const HSTU_LDS bf16x8 *)(Bs + cg_at<BN>(wn + 32 * j + l32, st >> 1, 2 * (st & 1) + half));
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm + 32 * i + l32;
        bf16x8 ahi, alo;
        if constexpr (C::kA16) {
          ahi = *(const HSTU_LDS bf16x8 *)(As + cg_at<BM>(r, st >> 1, 2 * (st & 1) + half));
        } else {
          u32x4 h, l;
          floatx4 x0 = *(const HSTU_LDS floatx4 *)(As + cg_at<BM>(r, st, 2 * half));
          floatx4 x1 = *(const HSTU_LDS floatx4 *)(As + cg_at<BM>(r, st, 2 * half + 1));
          if constexpr (C::AK == kAkGate) {
            const floatx4 u0 = *(const HSTU_LDS floatx4 *)(Us + cg_at<BM>(r, st, 2 * half));
            const floatx4 u1 = *(const HSTU_LDS floatx4 *)(Us + cg_at<BM>(r, st, 2 * half + 1));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x0[e] = fmaf(x0[e], rstd[i], nmr[i]) * u0[e];
              x1[e] = fmaf(x1[e], rstd[i], nmr[i]) * u1[e];
            }
          } else if constexpr (C::AK == kAkLn) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x0[e] = fmaf(x0[e], rstd[i], nmr[i]);
              x1[e] = fmaf(x1[e], rstd[i], nmr[i]);
            }
          }
          h = to_bf16x8(x0, x1);
          ahi = __builtin_bit_cast(bf16x8, h);
          if constexpr (C::kTerms == 2) {
            l = residual_bf16x8(x0, x1, h);
            alo = __builtin_bit_cast(bf16x8, l);
          }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = mfma32(ahi, bfr[j], acc[i][j]);
          if constexpr (C::kTerms == 2) acc[i][j] = mfma32(alo, bfr[j], acc[i][j]);
        }
      }
    }
  };

  // ---- k loop over an S-stage ring
  const int nk = imax(imin(p.K / BK - kt0, p.kt_per_split), 0);
  constexpr int kAhead = C::S - 1;
  for (int t = 0; t < kAhead; ++t)
    if (t < nk) issue(t, t);
  for (int kt = 0; kt < nk; ++kt) {
    const int after = imin(kAhead - 1, nk - 1 - kt);   // stages issued after this one
    if constexpr (C::S >= 4) {
      if (after >= 2) wait_vmcnt<2 * C::kD>();
      else if (after == 1) wait_vmcnt<C::kD>();
      else wait_vmcnt<0>();
    } else if constexpr (C::S == 3) {
      if (after >= 1) wait_vmcnt<C::kD>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();   // stage kt visible to every wave; every wave is done with stage kt - 1
    if (kt + kAhead < nk) issue(kt + kAhead, (kt + kAhead) % C::S);
    compute(kt % C::S);
  }

  // ---- epilogue: acc[i][j] element e -> row m0 + wm + 32i + 8(e/4) + 4 half + e%4, column n0 + wn + 32j + l32
  // stack output: the residual's per-row parameters, loaded once per row (resid_mode 1: the table row as
  // two 32-bit halves; 2: mean and rstd as bits)
  uint32_t rp0[EPI == kEpiOutStack ? FM : 1][16], rp1[EPI == kEpiOutStack ? FM : 1][16];
  if constexpr (EPI == kEpiOutStack) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = imin(m0 + wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4), p.M - 1);
        if (p.resid_mode == 1) {
          const uint64_t row = (uint64_t)checked_row_id(p.ids[m], p.id_rows, p.id_err);
          rp0[i][e] = (uint32_t)row;
          rp1[i][e] = (uint32_t)(row >> 32);
        } else if (p.resid_mode == 2) {
          const float2 st = *(const float2 *)(p.resid_rowstat + 2 * (int64_t)m);
          rp0[i][e] = __builtin_bit_cast(uint32_t, st.x);
          rp1[i][e] = __builtin_bit_cast(uint32_t, st.y);
        } else {
          rp0[i][e] = rp1[i][e] = 0u;
        }
      }
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn + 32 * j + l32;
    if (n >= p.N) continue;
    const float bias = p.bias ? to_f32(((const __bf16 *)p.bias)[n]) : 0.0f;
    if constexpr (EPI == kEpiUvqk) {
      const int part = n / p.HD, col = n % p.HD;
      void *dst = part == 0 ? p.out0 : part == 1 ? p.out1 : part == 2 ? p.out2 : p.out3;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4);
          if (m < p.M) {
            const float z = acc[i][j][e] + bias;
            const float s = silu_f32(z);
            const int64_t idx = (int64_t)m * p.HD + col;
            if (part == 0) ((float *)dst)[idx] = s;
            else ((__bf16 *)dst)[idx] = f32_to_bf16(s);
            if (p.zout) ((__bf16 *)p.zout)[(int64_t)m * p.N + n] = f32_to_bf16(z);
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        // the 16 residuals of the fragment are loaded (rows clamped into the matrix) before any is used:
        // the residual kind is decided once per fragment, so each branch issues its 16 loads back to back
        float r[16];
        auto idx_of = [&](int e) {
          return (int64_t)imin(m0 + wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4), p.M - 1) * p.N + n;
        };
        const float *rf = (const float *)p.resid;
        const __bf16 *rb = (const __bf16 *)p.resid;
        if constexpr (EPI == kEpiOutStack) {
          if (p.resid_mode == 1) {               // gathered bf16 rows
#pragma unroll
            for (int e = 0; e < 16; ++e) r[e] = to_f32(rb[(((int64_t)rp1[i][e] << 32) | rp0[i][e]) * p.N + n]);
          } else if (p.resid_mode == 2) {        // LayerNorm of fp32 rows
#pragma unroll
            for (int e = 0; e < 16; ++e) r[e] = rf[idx_of(e)];
#pragma unroll
            for (int e = 0; e < 16; ++e)
              r[e] = (r[e] - __builtin_bit_cast(float, rp0[i][e])) * __builtin_bit_cast(float, rp1[i][e]);
          } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) r[e] = to_f32(rb[idx_of(e)]);
          }
        } else {
          if (!p.resid) {
#pragma unroll
            for (int e = 0; e < 16; ++e) r[e] = 0.0f;
          } else if (p.resid_f32) {
#pragma unroll
            for (int e = 0; e < 16; ++e) r[e] = rf[idx_of(e)];
          } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) r[e] = to_f32(rb[idx_of(e)]);
          }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4);
          const float y = acc[i][j][e] + bias + r[e];
          if constexpr (EPI == kEpiOutStack) acc[i][j][e] = y;   // kept for the row statistics below
          if (m < p.M) {
            const int64_t idx = (int64_t)m * p.N + n;
            if (out32) out32[idx] = y;
            else if (p.y_f32) ((float *)p.out0)[idx] = y;
            else ((__bf16 *)p.out0)[idx] = f32_to_bf16(y);
          }
        }
      }
    }
  }

  // ---- per-row (mean, M2) of this tile's columns, for a LayerNorm applied by the next consumer.
  // Two passes over the values in registers (mean, then squared deviations); each pass sums a lane's
  // columns, then every lane's partial goes to LDS and one thread per row adds the WN x 32 partials in
  // order.  The LDS ring is idle by now (the barrier below waits for the last stage's readers).
  if constexpr (EPI == kEpiOutStack) {
    if (p.out_stats) {
      constexpr int kParts = C::WN * 32;
      constexpr int kStride = kParts + 1;   // a padded row: the per-row sums below read down a column
      static_assert(BM * (kStride + 1) * 4 <= C::kLds, "row statistics fit in the LDS ring");
      HSTU_LDS float *red = (HSTU_LDS float *)smem;    // [BM][kStride]
      HSTU_LDS float *rmean = red + BM * kStride;      // [BM]
      const int cnt = imin(BN, p.N - n0);
      const int wn_i = wave % C::WN;
      float mean_r[FM][16];
      for (int pass = 0; pass < 2; ++pass) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4);
            float v = 0.0f;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const bool ok = n0 + wn + 32 * j + l32 < p.N;
              const float d = pass == 0 ? acc[i][j][e] : acc[i][j][e] - mean_r[i][e];
              v += ok ? (pass == 0 ? d : d * d) : 0.0f;
            }
            red[row * kStride + wn_i * 32 + l32] = v;
          }
        __syncthreads();
        if (tid < BM) {
          float sum = 0.0f;
          for (int q = 0; q < kParts; ++q) sum += red[tid * kStride + q];
          if (pass == 0) {
            rmean[tid] = sum / (float)cnt;
          } else {
            const int m = m0 + tid;
            if (m < p.M) {
              const int nN = (p.N + BN - 1) / BN;
              float *st = p.out_stats + 2 * ((int64_t)m * nN + n0 / BN);
              st[0] = rmean[tid];
              st[1] = sum;
            }
          }
        }
        if (pass == 0) {
          __syncthreads();
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) mean_r[i][e] = rmean[wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4)];
        }
      }
    }
  }
}

template <class C, int EPI>
hipError_t launch_big(const GemmParams &p0, hipStream_t s) {
  if (p0.M == 0 || p0.N == 0) return hipSuccess;
  static LdsLimit lim;
  {
    hipError_t e = lim.raise((const void *)gemm_big_kernel<C, EPI>, C::kLds);
    if (e != hipSuccess) return e;
  }
  GemmParams p = p0;
  p.splits = p.splits > 1 ? p.splits : 1;
  const int nkt = p.K / C::BK;
  p.kt_per_split = (nkt + p.splits - 1) / p.splits;
  const long long nt = (long long)((p.N + C::BN - 1) / C::BN) * ((p.M + C::BM - 1) / C::BM) * p.splits;
  hipLaunchKernelGGL((gemm_big_kernel<C, EPI>), dim3((unsigned)((nt + 7) / 8 * 8)), dim3(C::kThreads), C::kLds, s, p);
  return hipGetLastError();
}

// out[i] = sum over s of part[s][i], s in increasing order (deterministic split-K reduction)
__global__ void __launch_bounds__(256) split_sum_kernel(const float *__restrict__ part, float *__restrict__ out,
                                                        int64_t n, int splits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (4 * i + 3 < n) {
    floatx4 acc = *(const floatx4 *)(part + 4 * i);
    for (int sp = 1; sp < splits; ++sp) acc += *(const floatx4 *)(part + (int64_t)sp * n + 4 * i);
    *(floatx4 *)(out + 4 * i) = acc;
  } else {
    for (int64_t j = 4 * i; j < n; ++j) {
      float acc = part[j];
      for (int sp = 1; sp < splits; ++sp) acc += part[(int64_t)sp * n + j];
      out[j] = acc;
    }
  }
}

template <typename TM, typename TA, int SPLIT, int EPI, bool GATE>
hipError_t launch(const GemmParams &p, hipStream_t s) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  dim3 grid((p.N + kBN - 1) / kBN, (p.M + kBM - 1) / kBM);
  hipLaunchKernelGGL((gemm_kernel<TM, TA, SPLIT, EPI, GATE>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// Large-tile configurations: <BM, BN, BK, stages, waves along M, waves along N, A kind, A terms, GM,
// workgroups per CU>
using CfgBf16 = BigCfg<128, 256, 32, 2, 2, 2, kAkBf16, 1, 4, 2>;
using CfgF32 = BigCfg<128, 256, 32, 2, 2, 2, kAkF32, 1, 8, 2>;
using CfgF32Split = BigCfg<128, 256, 32, 2, 2, 2, kAkF32, 2, 8, 2>;
using CfgGate = BigCfg<64, 256, 32, 2, 2, 2, kAkGate, 1, 4, 2>;
using CfgGateSplit = BigCfg<64, 256, 32, 2, 2, 2, kAkGate, 2, 4, 2>;
using CfgGather = BigCfg<128, 256, 32, 2, 2, 2, kAkGather, 1, 4, 2>;
using CfgLn = BigCfg<128, 256, 32, 2, 2, 2, kAkLn, 1, 8, 2>;
using CfgLnSplit = BigCfg<128, 256, 32, 2, 2, 2, kAkLn, 2, 8, 2>;
// bf16 operands on a small problem (fewer than 1024 tiles of 128 x 256, about two rounds of the 512
// workgroup slots): narrower tiles, twice as many workgroups (config-2 projection: 60 -> 49 us)
using CfgBf16N = BigCfg<128, 128, 32, 2, 2, 2, kAkBf16, 1, 4, 2>;

// The large-tile kernel needs K to be a whole number of k-tiles, per-lane source offsets (row within
// the tile times the row's bytes) that fit 32 bits, and enough tiles to fill the chip.
template <class C>
bool offsets_fit(int64_t K) {
  const int64_t rows = C::BM > C::BN ? C::BM : C::BN;
  return K * 4 * rows < (int64_t(1) << 32);
}
template <class C>
bool big_fits(const GemmParams &p) {
  const long long tiles = (long long)((p.N + C::BN - 1) / C::BN) * ((p.M + C::BM - 1) / C::BM);
  return p.K % C::BK == 0 && tiles >= 256 && offsets_fit<C>(p.K);
}

template <class C>
long long big_tiles(const GemmParams &p) {
  return (long long)((p.N + C::BN - 1) / C::BN) * ((p.M + C::BM - 1) / C::BM);
}

template <int EPI, bool GATE>
hipError_t dispatch(const GemmParams &p, int dtype, int a_f32, int split, hipStream_t s) {
  if (dtype == kF32) return launch<float, float, 1, EPI, GATE>(p, s);
  if constexpr (GATE) {
    if (split && big_fits<CfgGateSplit>(p)) return launch_big<CfgGateSplit, EPI>(p, s);
    if (!split && big_fits<CfgGate>(p)) return launch_big<CfgGate, EPI>(p, s);
  } else {
    if (a_f32 && split && big_fits<CfgF32Split>(p)) return launch_big<CfgF32Split, EPI>(p, s);
    if (a_f32 && !split && big_fits<CfgF32>(p)) return launch_big<CfgF32, EPI>(p, s);
    if (!a_f32 && big_tiles<CfgBf16>(p) < 1024 && big_fits<CfgBf16N>(p)) return launch_big<CfgBf16N, EPI>(p, s);
    if (!a_f32 && big_fits<CfgBf16>(p)) return launch_big<CfgBf16, EPI>(p, s);
  }
  if constexpr (!GATE) {
    if (!a_f32) return launch<__bf16, __bf16, 1, EPI, false>(p, s);
  }
  return split ? launch<__bf16, float, 2, EPI, GATE>(p, s) : launch<__bf16, float, 1, EPI, GATE>(p, s);
}

}  // namespace

hipError_t launch_gemm_uvqk(const GemmUvqkArgs &a, hipStream_t s) {
  GemmParams p{};
  p.a = a.x; p.b = a.w; p.bias = a.bias; p.resid = nullptr;
  p.out0 = a.u; p.out1 = a.v; p.out2 = a.q; p.out3 = a.k; p.out32 = nullptr; p.zout = a.z;
  p.M = a.M; p.N = 4 * a.HD; p.K = a.K; p.HD = a.HD;
  p.splits = 1;
  return dispatch<kEpiUvqk, false>(p, a.dtype, a.x_f32, a.split, s);
}

hipError_t launch_gemm_out(const GemmOutArgs &a, hipStream_t s) {
  GemmParams p{};
  p.a = a.o; p.b = a.w; p.bias = a.bias; p.resid = a.x;
  p.out0 = a.y; p.out1 = p.out2 = p.out3 = nullptr; p.out32 = a.y32;
  p.M = a.M; p.N = a.N; p.K = a.K; p.HD = 0;
  p.resid_f32 = a.x_f32; p.y_f32 = a.y_f32;
  p.gate_u = a.u; p.row_stats = a.row_stats; p.heads = a.heads; p.head_dim = a.head_dim; p.eps = a.eps;
  p.splits = 1;
  return dispatch<kEpiOut, true>(p, a.dtype, 1, a.split, s);
}

int gemm_plain_splits(int64_t M, int64_t N, int64_t K, int dtype, int a_f32) {
  if (dtype != kBF16 || a_f32 || K % CfgBf16::BK != 0 || M <= 0 || N <= 0 || !offsets_fit<CfgBf16>(K)) return 1;
  const int64_t tiles = ((N + CfgBf16::BN - 1) / CfgBf16::BN) * ((M + CfgBf16::BM - 1) / CfgBf16::BM);
  if (tiles >= 512) return 1;
  const int64_t by_fill = (1024 + tiles - 1) / tiles;     // about four workgroups per CU
  const int64_t by_depth = K / CfgBf16::BK / 16;           // at least 16 k-tiles per split
  const int64_t sp = by_fill < by_depth ? by_fill : by_depth;
  return sp > 1 ? (int)(sp < 64 ? sp : 64) : 1;
}

bool stack_gemms_fit(int64_t M, int64_t D, int64_t HD) {
  GemmParams p{};
  p.M = (int)M; p.N = (int)(4 * HD); p.K = (int)D;
  if (!big_fits<CfgGather>(p) || !big_fits<CfgLn>(p)) return false;
  p.N = (int)D; p.K = (int)HD;
  return big_fits<CfgGate>(p);
}

int stack_out_col_tiles(int64_t N) { return (int)((N + CfgGate::BN - 1) / CfgGate::BN); }

hipError_t launch_gemm_stack_proj(const GemmStackProjArgs &a, hipStream_t s) {
  GemmParams p{};
  p.a = a.a; p.b = a.w; p.bias = a.bias; p.resid = nullptr;
  p.out0 = a.u; p.out1 = a.v; p.out2 = a.q; p.out3 = a.k; p.out32 = nullptr; p.zout = nullptr;
  p.M = a.M; p.N = 4 * a.HD; p.K = a.K; p.HD = a.HD;
  p.splits = 1;
  p.ids = a.ids; p.id_rows = a.id_rows; p.id_err = a.id_err; p.a_rowstat = a.a_rowstat;
  if (a.a_mode == 1) return launch_big<CfgGather, kEpiUvqk>(p, s);
  if (a.a_mode == 2) return a.split ? launch_big<CfgLnSplit, kEpiUvqk>(p, s) : launch_big<CfgLn, kEpiUvqk>(p, s);
  return launch_big<CfgBf16, kEpiUvqk>(p, s);
}

hipError_t launch_gemm_stack_out(const GemmStackOutArgs &a, hipStream_t s) {
  GemmParams p{};
  p.a = a.o; p.b = a.w; p.bias = a.bias; p.resid = a.resid;
  p.out0 = a.y; p.out1 = p.out2 = p.out3 = nullptr; p.out32 = a.y32;
  p.M = a.M; p.N = a.N; p.K = a.K; p.HD = 0;
  p.resid_f32 = 0; p.y_f32 = a.y_f32;
  p.gate_u = a.u; p.row_stats = a.row_stats; p.heads = a.heads; p.head_dim = a.head_dim; p.eps = a.eps;
  p.splits = 1;
  p.resid_mode = a.resid_mode; p.ids = a.ids; p.id_rows = a.id_rows; p.id_err = a.id_err;
  p.resid_rowstat = a.resid_rowstat;
  p.out_stats = a.y32 ? a.out_stats : nullptr;
  return a.split ? launch_big<CfgGateSplit, kEpiOutStack>(p, s) : launch_big<CfgGate, kEpiOutStack>(p, s);
}

hipError_t launch_gemm_plain(const GemmPlainArgs &a, hipStream_t s) {
  GemmParams p{};
  p.a = a.a; p.b = a.b; p.bias = nullptr; p.resid = a.resid;
  p.out0 = a.c; p.out1 = p.out2 = p.out3 = nullptr;
  p.M = a.M; p.N = a.N; p.K = a.K; p.HD = 0;
  p.resid_f32 = a.resid_f32; p.y_f32 = a.c_f32;
  p.splits = 1;
  if (a.splits > 1) {
    // split-K: fp32 partial products per split, then a fixed-order sum into c
    if (a.dtype != kBF16 || a.a_f32 || a.resid || !a.c_f32 || !a.partial || a.K % CfgBf16::BK != 0 ||
        !offsets_fit<CfgBf16>(a.K) || ((int64_t)a.M * a.N) % 4 != 0)
      return hipErrorInvalidValue;
    if (a.M == 0 || a.N == 0) return hipSuccess;
    p.splits = a.splits;
    p.out32 = a.partial;
    hipError_t e = launch_big<CfgBf16, kEpiOut>(p, s);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)a.M * a.N;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, a.partial,
                       (float *)a.c, n, a.splits);
    return hipGetLastError();
  }
  return dispatch<kEpiOut, false>(p, a.dtype, a.a_f32, 0, s);
}

}  // namespace hstu
