// Causal softmax attention over the same jagged batch, bf16 with Dh = 128: the comparison point the
// HSTU abstract measures against ("Actions Speak Louder than Words: Trillion-Parameter Sequential
// Transducers for Generative Recommendations", abstract: HSTU against FlashAttention2-based
// Transformers at sequence length 8192).  It is here to time pointwise and softmax attention on the
// same shapes and hardware; it is not part of the HSTU layer.
//
//   O_i = sum_{j <= i} softmax_j(q_i . k_j / sqrt(Dh)) v_j
//
// Same tiling, staging and MFMA forms as the pointwise forward (attn_fwd.hip): 4 waves of 32 queries
// per workgroup, 64-key K/V tiles staged global -> LDS with direct-to-LDS loads in a two-stage ring,
// S^T = K Q^T and O^T += V^T P^T on 32x32x16 bf16 MFMAs.  The softmax is the online form: per query a
// running maximum m (in the log2 domain, t = s * log2(e) / sqrt(Dh)) and a running sum l of
// 2^(t - m); a tile that raises m rescales O and l by 2^(m_old - m_new), and a tile that raises no
// query's maximum (a scalar vote over the wave) skips the rescale, which is then exact.  Each lane
// holds one query and 16 of the 32 keys of a block (the other 16 are in lane ^ 32), so the tile
// maximum takes one cross-half exchange and each half keeps its own l until the epilogue.
#include "attn_common.hpp"

namespace hstu {
namespace {

using namespace attn;

constexpr float kLog2eOverSqrt128 = 0.12751743082459868f;   // log2(e) / sqrt(128)
constexpr float kNegInf = -__builtin_huge_valf();

template <typename TO>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
softmax_attn_kernel(const AttnArgs p, const int n_qblocks) {
  using L = Layout<__bf16, 128>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  HSTU_LDS char *smem = (HSTU_LDS char *)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  // ---- work item: query block major (longest first), then (sequence, head)
  const int HB = p.num_heads * p.num_seqs;
  const int item = (int)blockIdx.x;
  const int qblk = n_qblocks - 1 - item / HB;
  const int b = (item % HB) / p.num_heads;
  const int h = (item % HB) % p.num_heads;
  const int o0 = p.seq_offsets[b];
  const int nq = p.seq_offsets[b + 1] - o0;
  const int q0 = qblk * kBM;
  if (q0 >= nq) return;   // uniform over the workgroup

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int qr = q0 + wave * kQW;                  // the wave's first query (a multiple of 32)
  const int ql = imin(qr + kQW - 1, nq - 1);       // and its last valid one
  const int my_q = qr + l32;
  const bool my_valid = my_q < nq;

  bf16x8 qf[8];
  {
    const __bf16 *qrow = (const __bf16 *)p.q + (int64_t)(o0 + (my_valid ? my_q : 0)) * p.row_stride + h * 128;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 v = *(const bf16x8 *)(qrow + s * 16 + half * 8);
      if (!my_valid) v = bf16x8{};
      qf[s] = v;
    }
  }

  const int blast = imin(q0 + kBM - 1, nq - 1);
  const int ntiles = (blast + kBN) / kBN;          // tiles 0 .. blast / 64
  const uint32_t rsb = (uint32_t)(p.row_stride * L::kES);
  auto issue_tile = [&](int i, int stage) {
    const int lr16 = 16 * wave + (lane >> 2);
    const uint32_t k_add = (uint32_t)(h * L::kRB) + 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t v_add = (uint32_t)(h * L::kRB) + 16u * (uint32_t)(lane & 3);
    const int k0 = i * kBN;
    const uint32_t r = (uint32_t)imin(lr16, nq - 1 - k0);   // rows past the end repeat the last row
    const int64_t row0 = (int64_t)(o0 + k0) * rsb;
    const uint32_t sb = smem_addr + stage * L::kStageBytes;
    dma_groups<0, L::kG>((const char *)p.k + row0, (const char *)p.v + row0, __umul24(r, rsb) + k_add,
                         __umul24(r, rsb) + v_add, sb + L::kOffK + wave * 1024, sb + L::kOffV + wave * 1024);
  };

  OAcc<4> oacc;
#pragma unroll
  for (int d = 0; d < 4; ++d) oacc.d[d] = floatx16{};
  float m = kNegInf, lsum = 0.0f;

  if (0 < ntiles) issue_tile(0, 0);
  for (int i = 0; i < ntiles; ++i) {
    wait_vmcnt<0>();   // tile i landed (no later tile has been issued yet)
    __syncthreads();   // tile i visible; every wave is done with tile i - 1
    if (i + 1 < ntiles) issue_tile(i + 1, (i + 1) & 1);
    const int k0 = i * kBN;
    if (k0 > ql) continue;   // wave-uniform: no key of this tile is allowed for this wave
    const HSTU_LDS char *stage = smem + (i & 1) * L::kStageBytes;
    floatx16 s0, s1;
    score_block<__bf16, 128>(s0, stage + L::kOffK, 0, l32, half, qf);
    score_block<__bf16, 128>(s1, stage + L::kOffK, 1, l32, half, qf);
    float x[32];
#pragma unroll
    for (int e = 0; e < 16; ++e) { x[e] = s0[e]; x[16 + e] = s1[e]; }
    if (k0 + kBN - 1 > qr) {   // the diagonal tile: keys after the query are masked
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int j = k0 + 32 * (e / 16) + 16 * ((e % 16) / 8) + 8 * half + e % 8;
        x[e] = j <= my_q ? x[e] : kNegInf;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m, mx * kLog2eOverSqrt128);
    if (__any(m_new != m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);   // 2^-inf = 0 on the first tile
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc.d[d][e] *= alpha;
      m = m_new;
    }
    bf16x8 pf[2][2];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], kLog2eOverSqrt128, -m));
      lsum += pe;
      pf[e / 16][(e % 16) / 8][e % 8] = f32_to_bf16(pe);
    }
    av_block_packed<128, false>(oacc, pf[0], stage + L::kOffV, 0, lane);
    av_block_packed<128, false>(oacc, pf[1], stage + L::kOffV, 1, lane);
  }

  // ---- epilogue: divide by the row sum (each lane half summed its own keys)
  const float ltot = lsum + __shfl_xor(lsum, 32, kWave);
  const float rl = 1.0f / ltot;
  if (my_valid) {
    TO *orow = (TO *)p.out + (int64_t)(o0 + my_q) * p.out_row_stride + h * 128;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int dh = 32 * db + 8 * e4 + 4 * half;
        if constexpr (sizeof(TO) == 4) {
          floatx4 w;
          w[0] = oacc.d[db][4 * e4 + 0] * rl; w[1] = oacc.d[db][4 * e4 + 1] * rl;
          w[2] = oacc.d[db][4 * e4 + 2] * rl; w[3] = oacc.d[db][4 * e4 + 3] * rl;
          *(floatx4 *)(orow + dh) = w;
        } else {
          bf16x4 w;
          w[0] = f32_to_bf16(oacc.d[db][4 * e4 + 0] * rl); w[1] = f32_to_bf16(oacc.d[db][4 * e4 + 1] * rl);
          w[2] = f32_to_bf16(oacc.d[db][4 * e4 + 2] * rl); w[3] = f32_to_bf16(oacc.d[db][4 * e4 + 3] * rl);
          *(bf16x4 *)(orow + dh) = w;
        }
      }
  }
}

template <typename TO>
hipError_t launch_softmax_typed(const AttnArgs &a, hipStream_t stream) {
  const int n_qblocks = (a.max_seq_len + kBM - 1) / kBM;
  const long long grid = (long long)n_qblocks * a.num_heads * a.num_seqs;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (grid == 0) return hipSuccess;
  const size_t lds = 2 * (size_t)Layout<__bf16, 128>::kStageBytes;
  static LdsLimit lim;
  {
    hipError_t e = lim.raise((const void *)softmax_attn_kernel<TO>, 160 * 1024);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(softmax_attn_kernel<TO>, dim3((unsigned)grid), dim3(kThreads), lds, stream, a, n_qblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_attn(const AttnArgs &a, hipStream_t stream) {
  return a.out_dtype == kBF16 ? launch_softmax_typed<__bf16>(a, stream) : launch_softmax_typed<float>(a, stream);
}

}  // namespace hstu
