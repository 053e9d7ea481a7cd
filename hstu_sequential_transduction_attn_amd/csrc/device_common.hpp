// Device-side helpers shared by the gfx950 kernels of libhstu: vector types, MFMA wrappers,
// bf16 conversion, LDS pointer qualifiers.  CDNA4 only (wave64, MFMA, LDS transpose reads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "row_ids.hpp"

namespace hstu {

// Host side: a kernel's dynamic-LDS limit, raised once per device (function attributes are kept per
// device) and safely when several host threads launch at once.  One static instance per kernel.
struct LdsLimit {
  static constexpr int kMaxDevices = 64;
  std::once_flag once[kMaxDevices];
  hipError_t err[kMaxDevices] = {};
  hipError_t raise(const void *fn, int bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] { err[dev] = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); });
    return err[dev];
  }
};

#define HSTU_LDS __attribute__((address_space(3)))

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

// 32x32 MFMA over one k-step.  bf16: k = 16 per instruction, 8 values per lane; f32: k = 2, 1 value.
// Operand layouts (lane l): A[m][k] at lane m + 32*(k/KPL), B[k][n] at lane n + 32*(k/KPL);
// D[m][n] at lane n + 32*((m/4)%2), element 4*(m/8) + m%4.
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// SiLU(s) = s * sigmoid(s) = s / (1 + 2^(-s*log2(e))), with the hardware exp2 and reciprocal.
// For s << 0 the exponential overflows to +inf and the reciprocal gives 0, the right limit.
__device__ __forceinline__ float silu_f32(float s) {
  const float e = __builtin_amdgcn_exp2f(s * -1.4426950408889634f);
  return s * __builtin_amdgcn_rcpf(1.0f + e);
}

// A gathered row id clamped into [0, rows); each clamped read adds 1 to *err, the library's
// per-device id-error word (a vector atomic: the branch is taken only for a bad id).
__device__ __forceinline__ int64_t checked_row_id(int64_t id, int64_t rows, unsigned int *err) {
  if (!row_id_in_range(id, rows)) {
    atomicAdd(err, 1u);
    id = clamp_row_id(id, rows);
  }
  return id;
}

// Number of significant bits of |a - b| for int64 a, b (exact; the difference fits in uint64).
__device__ __forceinline__ int bitlen_absdiff(int64_t a, int64_t b) {
  const uint64_t d = a >= b ? (uint64_t)a - (uint64_t)b : (uint64_t)b - (uint64_t)a;
  return d == 0 ? 0 : 64 - __clzll((long long)d);
}

// 16 bytes (or 4 bytes) from global memory at base + lane_off + IMM straight into LDS at
// m0 + IMM + 16 * lane (4 * lane): the immediate offset moves both addresses.  base is a wave-uniform
// 64-bit address, lane_off a 32-bit per-lane offset.  Issued as inline assembly so that the waits for
// these loads are exactly the explicit vmcnt waits of a kernel's LDS ring (a wait the compiler inserted
// itself before LDS reads would not know that they read another stage); the s_nop is the one wait state
// an LDS DMA needs after an SALU write of M0.
template <int IMM>
__device__ __forceinline__ void dma16(const void *base, uint32_t lane_off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3"
               : : "s"(m0), "v"(lane_off), "s"(base), "i"(IMM) : "memory");
}
// The same 16-byte load from a per-lane 64-bit address (rows gathered from anywhere in memory).
__device__ __forceinline__ void dma16_at(const void *addr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m0), "v"(addr) : "memory");
}
__device__ __forceinline__ void dma4(const void *base, uint32_t lane_off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" : : "s"(m0), "v"(lane_off), "s"(base)
               : "memory");
}
// s_waitcnt with only the vector-memory counter constrained (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

}  // namespace hstu
