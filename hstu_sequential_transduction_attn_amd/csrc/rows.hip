// Row-wise, HBM-bound kernels of the HSTU layer on gfx950.
//
//  * row_layernorm:  y_t = LN(y32_t) between stacked layers (LayerNorm with biased variance, no affine).
//  * gather_rows:    x_t = E[id_t], the embedding lookup that stages the first layer's input.  An id
//                    outside [0, table_rows) is clamped to the nearest row and counted in the
//                    per-device id-error word (read back through hstu_id_errors).
//
// One wave per row; each lane keeps its slice of the row in registers, so the row is read from HBM
// exactly once and the statistics take two passes over registers (mean, then centred squares).
#include <mutex>

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

template <typename TO, int MAXC>
__global__ void __launch_bounds__(256) row_ln_kernel(const float *__restrict__ in, TO *__restrict__ out, int M, int N,
                                                     float eps) {
  const int row = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= M) return;
  const float *irow = in + (int64_t)row * N;
  float x[MAXC][4];
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int col = 256 * c + 4 * lane;
    if (col < N) {
      const floatx4 v = *(const floatx4 *)(irow + col);
      x[c][0] = v[0]; x[c][1] = v[1]; x[c][2] = v[2]; x[c][3] = v[3];
      s += v[0] + v[1] + v[2] + v[3];
    } else {
      x[c][0] = x[c][1] = x[c][2] = x[c][3] = 0.0f;
    }
  }
  const float mean = wave_sum(s) / (float)N;
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int col = 256 * c + 4 * lane;
    if (col < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = x[c][i] - mean;
        q += d * d;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)N + eps);
  TO *orow = out + (int64_t)row * N;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int col = 256 * c + 4 * lane;
    if (col < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[col + i] = from_f32<TO>((x[c][i] - mean) * rstd);
    }
  }
}

__global__ void __launch_bounds__(256) gather_kernel(const u32x4 *__restrict__ table, const int64_t *__restrict__ ids,
                                                     u32x4 *__restrict__ out, int T, int chunks_per_row, int64_t rows,
                                                     unsigned int *__restrict__ err) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)T * chunks_per_row;
  if (i >= total) return;
  const int64_t t = i / chunks_per_row;
  const int c = (int)(i % chunks_per_row);
  out[i] = table[checked_row_id(ids[t], rows, err) * chunks_per_row + c];
}

// Chan's pairwise combination of per-tile (mean, M2) in tile order; one thread per row.
__global__ void __launch_bounds__(256) row_stats_combine_kernel(const float *__restrict__ ts, float *__restrict__ rs,
                                                                int M, int N, int tiles, float eps) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const float *t = ts + (int64_t)m * tiles * 2;
  float n = 0.0f, mean = 0.0f, m2 = 0.0f;
  for (int c = 0; c < tiles; ++c) {
    const float nc = (float)min(256, N - 256 * c);
    const float d = t[2 * c] - mean;
    const float tot = n + nc;
    mean += d * (nc / tot);
    m2 += t[2 * c + 1] + d * d * (n * nc / tot);
    n = tot;
  }
  rs[2 * (int64_t)m] = mean;
  rs[2 * (int64_t)m + 1] = 1.0f / sqrtf(m2 / (float)N + eps);
}

// Row width is bounded by 256 * MAXC (checked on the host: width <= 4096, width % 4 == 0).
template <typename TO>
hipError_t launch_ln(const RowLnArgs &a, hipStream_t s) {
  const dim3 grid((a.M + kRowsPerBlock - 1) / kRowsPerBlock);
  TO *out = (TO *)a.out;
  if (a.N <= 256) hipLaunchKernelGGL((row_ln_kernel<TO, 1>), grid, dim3(256), 0, s, a.in, out, a.M, a.N, a.eps);
  else if (a.N <= 1024) hipLaunchKernelGGL((row_ln_kernel<TO, 4>), grid, dim3(256), 0, s, a.in, out, a.M, a.N, a.eps);
  else hipLaunchKernelGGL((row_ln_kernel<TO, 16>), grid, dim3(256), 0, s, a.in, out, a.M, a.N, a.eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_row_layernorm(const RowLnArgs &a, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  return a.out_f32 ? launch_ln<float>(a, s) : launch_ln<__bf16>(a, s);
}

hipError_t launch_row_stats_combine(const float *tile_stats, float *rowstat, int M, int N, float eps, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int tiles = (N + 255) / 256;
  hipLaunchKernelGGL(row_stats_combine_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, tile_stats,
                     rowstat, M, N, tiles, eps);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *table, int64_t table_rows, int32_t row_bytes, const int64_t *ids, int32_t T,
                              void *out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  unsigned int *err = nullptr;
  hipError_t e = id_error_word(&err);
  if (e != hipSuccess) return e;
  const int cpr = row_bytes / 16;
  const int64_t total = (int64_t)T * cpr;
  const dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, (const u32x4 *)table, ids, (u32x4 *)out, T, cpr,
                     table_rows, err);
  return hipGetLastError();
}

// The per-device id-error word: a file-scope device variable whose device address is looked up once
// per device (with that device current) and kept; host code never passes the variable's own name.
namespace {
static __device__ __align__(256) unsigned int id_errors;
constexpr int kMaxIdDevices = 64;
std::once_flag g_id_once[kMaxIdDevices];
unsigned int *g_id_ptr[kMaxIdDevices];
hipError_t g_id_err[kMaxIdDevices];
}  // namespace

hipError_t id_error_word(unsigned int **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxIdDevices) return hipErrorInvalidDevice;
  std::call_once(g_id_once[dev], [dev] {
    void *p = nullptr;
    g_id_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(id_errors));
    g_id_ptr[dev] = g_id_err[dev] == hipSuccess ? (unsigned int *)p : nullptr;
  });
  if (g_id_err[dev] != hipSuccess) return g_id_err[dev];
  if (!g_id_ptr[dev]) return hipErrorInvalidSymbol;
  *ptr = g_id_ptr[dev];
  return hipSuccess;
}

}  // namespace hstu
