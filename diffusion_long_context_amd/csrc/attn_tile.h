// One wavefront's share of an attention step on gfx950: 32 query rows attend
// to a block of kv rows whose K (row-major) and V (transposed) sit in LDS.
// Shared by the split-KV decode kernel and the chunk prefill kernel.
//
// Layout (v_mfma_f32_16x16x32_bf16; lane = 16 lj + lr):
//   S^T = K Q^T : lane holds S^T[kv = 16 kb + 4 lj + e][q = 16 b + lr]
//   O^T += V^T P^T : lane holds O^T[d = 16 db + 4 lj + e][q = 16 b + lr]
// so every lane owns whole query columns and the probabilities it computes
// are directly the PV product's B operand.  For a 32-row kv chunk kc the B
// operand's elements 0..3 are kv 32 kc + 4 lj + e and 4..7 are
// kv 32 kc + 16 + 4 lj + e; the V^T A operand is read in the same order.
//
// Online softmax in base 2 (scale * log2 e folded into one FMA before
// v_exp_f32).  A row's reference max only moves when a block's max exceeds
// it by more than 2^kRescaleLog2, so the accumulators are rescaled rarely and
// probabilities stay below 2^8.  The row sums come from the PV MFMA with an
// all-ones A operand, i.e. they are sums of the same bf16 probabilities the
// PV product uses.
#pragma once

#include "device_common.h"

namespace pdllm {

constexpr float kRescaleLog2 = 8.0f;


template <int D, int KP, int VP>
struct WaveAttn {
  static constexpr int DC = D / 32;   // 32-wide d chunks of QK^T
  static constexpr int DB = D / 16;   // 16-row d blocks of O^T

  f32x4 acc[DB][2];
  f32x4 lacc[2];
  float m_run[2];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][0] = acc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    lacc[0] = lacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[0] = m_run[1] = -INFINITY;
  }

  // Attend to kv rows [0, 16 NK) of an LDS block; only rows in
  // [valid_lo, valid_hi) count, the rest are masked (a wave-uniform branch,
  // taken only by a partial block).  k_lane = &K[lr][8 lj] (pitch KP) and vt_lane = &V^T[lr][4 lj]
  // (pitch VP) are the lane's base addresses, so every fragment read below is
  // the base plus a compile-time offset.
  template <int NK>
  __device__ __forceinline__ void step(const uint16_t* __restrict__ k_lane,
                                       const uint16_t* __restrict__ vt_lane,
                                       const bf16x8 (&qf)[2][DC], float sl2, int valid_hi, int lj,
                                       int valid_lo = 0) {
    static_assert(NK % 2 == 0, "kv blocks come in 32-row pairs");
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 sc[NK][2];
    __builtin_amdgcn_s_setprio(1);          // MFMA phases win issue over softmax phases
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(k_lane + 16 * kb * KP);
      sc[kb][0] = mfma16x16x32(ka, qf[0][0], zero);
      sc[kb][1] = mfma16x16x32(ka, qf[1][0], zero);
    }
#pragma unroll
    for (int dc = 1; dc < DC; ++dc) {
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(k_lane + 16 * kb * KP + 32 * dc);
        sc[kb][0] = mfma16x16x32(ka, qf[0][dc], sc[kb][0]);
        sc[kb][1] = mfma16x16x32(ka, qf[1][dc], sc[kb][1]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (valid_hi < 16 * NK || valid_lo > 0) {
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * kb + 4 * lj + e;
          if (r >= valid_hi || r < valid_lo) sc[kb][0][e] = sc[kb][1][e] = -INFINITY;
        }
    }
    bf16x8 pf[NK / 2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float mx = fmaxf(fmaxf(sc[0][b][0], sc[0][b][1]), fmaxf(sc[0][b][2], sc[0][b][3]));
#pragma unroll
      for (int kb = 1; kb < NK; ++kb) {
        mx = fmaxf(fmaxf(mx, sc[kb][b][0]), sc[kb][b][1]);
        mx = fmaxf(fmaxf(mx, sc[kb][b][2]), sc[kb][b][3]);
      }
      mx = wave_xor_max(mx, 16);
      mx = wave_xor_max(mx, 32);
      const float ms = mx * sl2;
      const bool need = ms > m_run[b] + kRescaleLog2;
      if (__ballot(need)) {
        const float m_new = need ? ms : m_run[b];
        const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_new);
        m_run[b] = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][b] *= alpha;
        lacc[b] *= alpha;
      }
      const float neg_m = -m_run[b];
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[kb][b][e] = __builtin_amdgcn_exp2f(fmaf(sc[kb][b][e], sl2, neg_m));
#pragma unroll
      for (int kc = 0; kc < NK / 2; ++kc)
        pf[kc][b] = bf16x8{(__bf16)sc[2 * kc][b][0], (__bf16)sc[2 * kc][b][1],
                           (__bf16)sc[2 * kc][b][2], (__bf16)sc[2 * kc][b][3],
                           (__bf16)sc[2 * kc + 1][b][0], (__bf16)sc[2 * kc + 1][b][1],
                           (__bf16)sc[2 * kc + 1][b][2], (__bf16)sc[2 * kc + 1][b][3]};
    }
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kc = 0; kc < NK / 2; ++kc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vp = vt_lane + 16 * db * VP + 32 * kc;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 16);
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        acc[db][0] = mfma16x16x32(va, pf[kc][0], acc[db][0]);
        acc[db][1] = mfma16x16x32(va, pf[kc][1], acc[db][1]);
      }
      lacc[0] = mfma16x16x32(ones, pf[kc][0], lacc[0]);
      lacc[1] = mfma16x16x32(ones, pf[kc][1], lacc[1]);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // Row sum and natural-log normaliser of column block b.
  __device__ __forceinline__ float row_sum(int b) const { return lacc[b][0]; }
  __device__ __forceinline__ float lse(int b) const { return m_run[b] * kLn2 + logf(lacc[b][0]); }
};

// Query fragments (B operand of S^T): lane column lr of block b, d = 32 dc + 8 lj ...
template <int DC>
__device__ __forceinline__ void zero_q(bf16x8 (&qf)[DC]) {
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qf[dc] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
}

template <int DC>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[DC], const uint16_t* row_plus_8lj) {
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qf[dc] = *reinterpret_cast<const bf16x8*>(row_plus_8lj + 32 * dc);
}

// Store a wavefront's O^T column (query column lr of block b) as 4 bf16 per d block.
template <int DB>
__device__ __forceinline__ void store_o_bf16(uint16_t* row_plus_4lj, const f32x4 (&acc)[DB][2], int b,
                                             float inv) {
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const f32x4 x = acc[db][b] * inv;
    *reinterpret_cast<u32x2*>(row_plus_4lj + 16 * db) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  }
}

}  // namespace pdllm
