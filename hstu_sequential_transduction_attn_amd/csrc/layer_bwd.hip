// HBM-bound kernels of the HSTU layer backward on gfx950 (the layer is trained: "DLRMv4：MLPerfの推薦
// システム訓練ベンチマークがシーケンス化時代へ" describes a training benchmark; its section
// "モデルアーキテクチャ" gives the layer: one projection, pointwise attention, a gated transformation).
//
// With r = x + g W2^T + b2 (y = LN(r) between stacked layers), g = LN(o) * U, o = concat_h O and
// z = x W1^T + b1 (U|V|Q|K = SiLU(z)), the backward is
//   dr = LN'(r) dy  (or dy)            -> ln_bwd_rows_kernel
//   dg = dr W2                         -> plain GEMM
//   dU = dg * LN(o),  do = LN'(o)(dg * U),  g recomputed for dW2      -> norm_gate_bwd_kernel
//   dQ, dK, dV = attention backward(do)
//   dz = [dU | dV | dQ | dK] * SiLU'(z)                               -> norm_gate_bwd / the attention
//                                                                        backward's epilogues
//   dx = dr + dz W1;  dW1 = dz^T x;  dW2 = dr^T g                      -> GEMMs (the weight gradients on
//                                                                        token-contiguous transposes)
//   db1 = sum_t dz,  db2 = sum_t dr                                   -> column sums per 64-row tile in
//                                                                        the transposes, then added
// where LN'(a) b = rstd (b - mean(b) - a_hat mean(b a_hat)) is the LayerNorm Jacobian applied to b.
//
// Row kernels use one wave per row with the row in registers (two passes over registers for the
// statistics); the transpose goes through a padded LDS tile so both sides are coalesced.
#include "device_common.hpp"
#include "kernels.h"

namespace hstu {
namespace {

constexpr int kRowsPerBlock = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// SiLU'(z) = sigma(z) (1 + z (1 - sigma(z))), sigma(z) = 1 / (1 + 2^(-z log2 e)); z << 0 gives
// sigma = 0 (the exponential overflows, its reciprocal is 0) and the derivative's limit 0.
__device__ __forceinline__ float silu_grad_f32(float z) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
  return sg * (1.0f + z * (1.0f - sg));
}

// Four consecutive elements as fp32, and back.
__device__ __forceinline__ floatx4 load4(const float *p) { return *(const floatx4 *)p; }
__device__ __forceinline__ floatx4 load4(const __bf16 *p) {
  const bf16x4 v = *(const bf16x4 *)p;
  return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void store4(float *p, floatx4 v) { *(floatx4 *)p = v; }
__device__ __forceinline__ void store4(__bf16 *p, floatx4 v) {
  *(bf16x4 *)p = bf16x4{f32_to_bf16(v[0]), f32_to_bf16(v[1]), f32_to_bf16(v[2]), f32_to_bf16(v[3])};
}

// ---- dr = LN'(r) dy, in place over r (fp32 [M][N]); dy [M][N] in TG.  N <= 256 * MAXC, N % 4 == 0.
template <typename TG, int MAXC>
__global__ void __launch_bounds__(256) ln_bwd_rows_kernel(float *__restrict__ r, const TG *__restrict__ dy, int M,
                                                          int N, float eps) {
  const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= M) return;
  float *rr = r + (int64_t)row * N;
  const TG *gr = dy + (int64_t)row * N;
  floatx4 x[MAXC], g[MAXC];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int col = 256 * c + 4 * lane;
    x[c] = col < N ? load4(rr + col) : floatx4{};
    g[c] = col < N ? load4(gr + col) : floatx4{};
    s += x[c][0] + x[c][1] + x[c][2] + x[c][3];
  }
  const float mean = wave_sum(s) / (float)N;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    if (256 * c + 4 * lane < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = x[c][i] - mean;
        q += d * d;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)N + eps);
  float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[c][i] = (x[c][i] - mean) * rstd;   // x_hat; padding lanes add nothing below (their g is 0)
      s1 += g[c][i];
      s2 += g[c][i] * x[c][i];
    }
  }
  const float m1 = wave_sum(s1) / (float)N, m2 = wave_sum(s2) / (float)N;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int col = 256 * c + 4 * lane;
    if (col < N) {
      floatx4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = rstd * (g[c][i] - m1 - x[c][i] * m2);
      store4(rr + col, d);
    }
  }
}

// ---- norm-gate backward, one wave per token.  o, u, dg: fp32 [M][N] (N = H*Dh); z: TM [M][4N], its
// first N columns (the U slice) are replaced by dz_U = dg * LN(o) * SiLU'(z_U); g = LN(o) * U and
// d_o = LN'(o)(dg * U) go to [M][N] TM buffers.
template <typename TM, int MAXC>
__global__ void __launch_bounds__(256) norm_gate_bwd_kernel(const float *__restrict__ o, const float *__restrict__ u,
                                                            const float *__restrict__ dg, TM *__restrict__ z,
                                                            TM *__restrict__ g_out, TM *__restrict__ d_o, int M,
                                                            int N, float eps) {
  const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= M) return;
  const int64_t base = (int64_t)row * N;
  floatx4 xh[MAXC], dxh[MAXC];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int col = 256 * c + 4 * lane;
    xh[c] = col < N ? load4(o + base + col) : floatx4{};
    s += xh[c][0] + xh[c][1] + xh[c][2] + xh[c][3];
  }
  const float mean = wave_sum(s) / (float)N;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    if (256 * c + 4 * lane < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = xh[c][i] - mean;
        q += d * d;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)N + eps);
  TM *zr = z + (int64_t)row * 4 * N;
  float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int col = 256 * c + 4 * lane;
    if (col < N) {
      const floatx4 uu = load4(u + base + col), gg = load4(dg + base + col), zz = load4(zr + col);
      floatx4 gv, dz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = (xh[c][i] - mean) * rstd;
        xh[c][i] = x;
        gv[i] = x * uu[i];
        dz[i] = gg[i] * x * silu_grad_f32(zz[i]);
        dxh[c][i] = gg[i] * uu[i];
        s1 += dxh[c][i];
        s2 += dxh[c][i] * x;
      }
      store4(g_out + base + col, gv);
      store4(zr + col, dz);
    } else {
      xh[c] = floatx4{};
      dxh[c] = floatx4{};
    }
  }
  const float m1 = wave_sum(s1) / (float)N, m2 = wave_sum(s2) / (float)N;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int col = 256 * c + 4 * lane;
    if (col < N) {
      floatx4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = rstd * (dxh[c][i] - m1 - xh[c][i] * m2);
      store4(d_o + base + col, d);
    }
  }
}

// ---- dst[c][r] = src[r][c] for r < R, 0 for R <= r < Rp (TI -> TO, rounded when TO is bf16).
// 64 x 64 tiles through a padded LDS tile; C % 4 == 0, Rp % 4 == 0.  With colsum, each tile also writes
// its 64 column sums (of the source values) to colsum[c * ldp + blockIdx.y]: four lanes per column add
// 16 rows each, then a fixed butterfly over the four.  Tiles past the rows write zeros.
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) transpose_kernel(const TI *__restrict__ src, TO *__restrict__ dst, int R, int C,
                                                        int Rp, float *__restrict__ colsum, int ldp) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  {
    const int cc = 4 * (tid % 16), rr = tid / 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = r0 + rr + 16 * p, c = c0 + cc;
      floatx4 v{};
      if (r < R && c < C) v = load4(src + (int64_t)r * C + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[rr + 16 * p][cc + e] = v[e];
    }
  }
  __syncthreads();
  if (colsum) {
    const int cc = tid / 4, q = tid % 4;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += tile[16 * q + r][cc];
    sum += __shfl_xor(sum, 1, 4);
    sum += __shfl_xor(sum, 2, 4);
    if (q == 0 && c0 + cc < C) colsum[(int64_t)(c0 + cc) * ldp + blockIdx.y] = sum;
  }
  {
    const int rr = 4 * (tid % 16), cc = tid / 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c = c0 + cc + 16 * p, r = r0 + rr;
      if (c < C && r < Rp) {
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = tile[rr + e][cc + 16 * p];
        store4(dst + (int64_t)c * Rp + r, v);
      }
    }
  }
}

// ---- out[c] = sum_r src[c][r] over a row of Rp elements (Rp % 4 == 0), one workgroup per row: each
// thread sums a strided set of 4-element groups in increasing order, then a fixed LDS tree.
template <typename T>
__global__ void __launch_bounds__(256) row_sum_kernel(const T *__restrict__ src, float *__restrict__ out, int Rp) {
  __shared__ float part[256];
  const T *row = src + (int64_t)blockIdx.x * Rp;
  float s = 0.0f;
  for (int r = 4 * threadIdx.x; r < Rp; r += 4 * 256) {
    const floatx4 v = load4(row + r);
    s += (v[0] + v[1]) + (v[2] + v[3]);
  }
  part[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = part[0];
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

template <typename TG>
hipError_t launch_ln_bwd_t(const LnBwdArgs &a, hipStream_t s) {
  const dim3 grid((a.M + kRowsPerBlock - 1) / kRowsPerBlock);
  const TG *dy = (const TG *)a.dy;
  if (a.N <= 256) hipLaunchKernelGGL((ln_bwd_rows_kernel<TG, 1>), grid, dim3(256), 0, s, a.r, dy, a.M, a.N, a.eps);
  else if (a.N <= 1024) hipLaunchKernelGGL((ln_bwd_rows_kernel<TG, 4>), grid, dim3(256), 0, s, a.r, dy, a.M, a.N, a.eps);
  else hipLaunchKernelGGL((ln_bwd_rows_kernel<TG, 16>), grid, dim3(256), 0, s, a.r, dy, a.M, a.N, a.eps);
  return hipGetLastError();
}

template <typename TM>
hipError_t launch_norm_gate_bwd_t(const NormGateBwdArgs &a, hipStream_t s) {
  const dim3 grid((a.M + kRowsPerBlock - 1) / kRowsPerBlock);
  TM *z = (TM *)a.z, *g = (TM *)a.g, *d_o = (TM *)a.d_o;
  if (a.N <= 256)
    hipLaunchKernelGGL((norm_gate_bwd_kernel<TM, 1>), grid, dim3(256), 0, s, a.o, a.u, a.dg, z, g, d_o, a.M, a.N, a.eps);
  else if (a.N <= 1024)
    hipLaunchKernelGGL((norm_gate_bwd_kernel<TM, 4>), grid, dim3(256), 0, s, a.o, a.u, a.dg, z, g, d_o, a.M, a.N, a.eps);
  else
    hipLaunchKernelGGL((norm_gate_bwd_kernel<TM, 16>), grid, dim3(256), 0, s, a.o, a.u, a.dg, z, g, d_o, a.M, a.N,
                       a.eps);
  return hipGetLastError();
}

template <typename TI, typename TO>
hipError_t launch_transpose_t(const void *src, void *dst, int R, int C, int Rp, float *colsum, hipStream_t s) {
  const int ldp = transpose_colsum_ld(Rp);
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)(colsum ? ldp : (Rp + 63) / 64));
  hipLaunchKernelGGL((transpose_kernel<TI, TO>), grid, dim3(256), 0, s, (const TI *)src, (TO *)dst, R, C, Rp, colsum,
                     ldp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ln_bwd_rows(const LnBwdArgs &a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  return a.dy_f32 ? launch_ln_bwd_t<float>(a, s) : launch_ln_bwd_t<__bf16>(a, s);
}

hipError_t launch_norm_gate_bwd(const NormGateBwdArgs &a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  return a.dtype == kF32 ? launch_norm_gate_bwd_t<float>(a, s) : launch_norm_gate_bwd_t<__bf16>(a, s);
}

int transpose_colsum_ld(int Rp) { return ((Rp + 63) / 64 + 3) / 4 * 4; }

hipError_t launch_transpose(const void *src, int src_f32, void *dst, int dst_f32, int R, int C, int Rp, hipStream_t s,
                            float *colsum) {
  if (C == 0 || Rp == 0) return hipSuccess;
  if (src_f32 && dst_f32) return launch_transpose_t<float, float>(src, dst, R, C, Rp, colsum, s);
  if (src_f32) return launch_transpose_t<float, __bf16>(src, dst, R, C, Rp, colsum, s);
  if (dst_f32) return launch_transpose_t<__bf16, float>(src, dst, R, C, Rp, colsum, s);
  return launch_transpose_t<__bf16, __bf16>(src, dst, R, C, Rp, colsum, s);
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
  if (n == 0 || !p) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_row_sum(const void *src, int src_f32, float *out, int rows, int Rp, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (src_f32)
    hipLaunchKernelGGL((row_sum_kernel<float>), dim3((unsigned)rows), dim3(256), 0, s, (const float *)src, out, Rp);
  else
    hipLaunchKernelGGL((row_sum_kernel<__bf16>), dim3((unsigned)rows), dim3(256), 0, s, (const __bf16 *)src, out, Rp);
  return hipGetLastError();
}

}  // namespace hstu
