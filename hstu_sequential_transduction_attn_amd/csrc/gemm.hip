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
//
// Both operands are K-contiguous (row-major activations, torch-Linear [out][in] weights), which is the
// native operand form of the 32x32 MFMAs.  Workgroup tile 128x128, k-tile 32, 4 waves in a 2x2 grid,
// each wave 64x64 (2x2 MFMA tiles); LDS double-buffered with one barrier per k-tile.
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

enum Epi : int { kEpiUvqk = 0, kEpiOut = 1 };

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
  float *out32;        // output epilogue: fp32 result (pre-LayerNorm) or null
  int M, N, K, HD;
  int resid_f32, y_f32;
  const float *gate_u;     // fused gate: U [M][K] fp32
  const float *row_stats;  // fused gate: [M][heads][2] per-head mean and sum of squared deviations of O
  int heads, head_dim;
  float eps;
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
            const float s = silu_f32(acc[i][j][e] + bias);
            const int64_t idx = (int64_t)m * p.HD + col;
            if (part == 0) ((float *)dst)[idx] = s;
            else ((TM *)dst)[idx] = from_f32<TM>(s);
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm + 32 * i + 8 * (e / 4) + 4 * half + (e % 4);
          if (m < p.M) {
            const int64_t idx = (int64_t)m * p.N + n;
            const float r = p.resid_f32 ? ((const float *)p.resid)[idx] : to_f32(((const TM *)p.resid)[idx]);
            const float y = acc[i][j][e] + bias + r;
            if (p.out32) p.out32[idx] = y;
            else if (p.y_f32) ((float *)p.out0)[idx] = y;
            else ((TM *)p.out0)[idx] = from_f32<TM>(y);
          }
        }
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

template <int EPI, bool GATE>
hipError_t dispatch(const GemmParams &p, int dtype, int a_f32, int split, hipStream_t s) {
  if (dtype == kF32) return launch<float, float, 1, EPI, GATE>(p, s);
  if constexpr (!GATE) {
    if (!a_f32) return launch<__bf16, __bf16, 1, EPI, false>(p, s);
  }
  return split ? launch<__bf16, float, 2, EPI, GATE>(p, s) : launch<__bf16, float, 1, EPI, GATE>(p, s);
}

}  // namespace

hipError_t launch_gemm_uvqk(const GemmUvqkArgs &a, hipStream_t s) {
  GemmParams p{};
  p.a = a.x; p.b = a.w; p.bias = a.bias; p.resid = nullptr;
  p.out0 = a.u; p.out1 = a.v; p.out2 = a.q; p.out3 = a.k; p.out32 = nullptr;
  p.M = a.M; p.N = 4 * a.HD; p.K = a.K; p.HD = a.HD;
  return dispatch<kEpiUvqk, false>(p, a.dtype, a.x_f32, a.split, s);
}

hipError_t launch_gemm_out(const GemmOutArgs &a, hipStream_t s) {
  GemmParams p{};
  p.a = a.o; p.b = a.w; p.bias = a.bias; p.resid = a.x;
  p.out0 = a.y; p.out1 = p.out2 = p.out3 = nullptr; p.out32 = a.y32;
  p.M = a.M; p.N = a.N; p.K = a.K; p.HD = 0;
  p.resid_f32 = a.x_f32; p.y_f32 = a.y_f32;
  p.gate_u = a.u; p.row_stats = a.row_stats; p.heads = a.heads; p.head_dim = a.head_dim; p.eps = a.eps;
  return dispatch<kEpiOut, true>(p, a.dtype, 1, a.split, s);
}

}  // namespace hstu
