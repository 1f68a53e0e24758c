// One wavefront's share of an attention step on gfx950: 32 query rows attend
// to a block of kv rows whose K (row-major) and V (transposed) sit in LDS.
// Shared by the split-KV decode kernel and the chunk prefill kernel.
//
// The contractions run on v_mfma_f32_32x32x16_bf16 (the 16x16x32 variant
// reaches only about half the dense bf16 rate on this chip).  Lane l = 32 j + c
// (c = l % 32, j = l / 32):
//   S^T = K Q^T : lane holds S^T[kv = 32 kb + 8 m + 4 j + t][q = c], i = 4 m + t
//   O^T += V^T P^T : lane holds O^T[d = 32 db + 8 m + 4 j + t][q = c]
// so every lane owns one query column; the row max needs one exchange with
// lane l ^ 32 (v_permlane32_swap).  For the 16-row kv chunk h of block kb, the PV B operand is the
// lane's accumulator registers 8 h .. 8 h + 7 (kv 32 kb + 16 h + 8 u + 4 j + t,
// element 4 u + t).  V stays row-major in LDS like K; its A operand (V^T rows)
// comes from two ds_read_b64_tr_b16: inside each 16-lane group, lane 4 a + b
// receives element e of the 8-byte row addressed by lane a + 4 e (offset b),
// so lane s = a + 4 e of group g points at kv row 4 j + e (+ 8 for the second
// read) and d column 16 (g % 2) + 4 a (see v_lane_offset).
//
// Online softmax in base 2 (scale * log2 e folded into one FMA before
// v_exp_f32).  A row's reference max only moves when a block's max exceeds it
// by more than 2^kRescaleLog2, so the accumulators are rescaled rarely and
// probabilities stay below 2^8.  Row sums are float32 sums of the unrounded
// probabilities.
#pragma once

#include "device_common.h"

namespace pdllm {

constexpr float kRescaleLog2 = 8.0f;
// Starting reference max: finite, so that a block with every row masked
// (scores -inf) gives p = 2^(-inf - kNoMax) = 0 rather than NaN, and below
// any score, so that the first block with a counted row replaces it
// (its rescale factor 2^(kNoMax - m) is 0 on the still-empty sums).
constexpr float kNoMax = -1e30f;

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16) on one wavefront: lane l
// supplies A row l % 32 and B column l % 32 with the eight k values
// 8 (l / 32) .. 8 (l / 32) + 7, and receives D column l % 32, rows
// 8 (i / 4) + 4 (l / 32) + i % 4 for i = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum of a value and its copy in lane l ^ 32.  v_permlane32_swap with
// the same register as both operands leaves one output holding lanes 0..31
// twice and the other lanes 32..63 twice, so combining the two outputs
// lane-wise combines each lane with its partner (a VALU op, no LDS trip).
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Lane offset (elements) into a row-major V tile of pitch VP for the
// transposing reads: kv row 4 j + e and d column 16 (g % 2) + 4 a, where
// lane = 16 g + a + 4 e and j = lane / 32.
__device__ __forceinline__ int v_lane_offset(int lane, int vp) {
  const int s = lane & 15, g = lane >> 4;
  return (4 * (lane >> 5) + (s >> 2)) * vp + 16 * (g & 1) + 4 * (s & 3);
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                        (__attribute__((address_space(3))) s16x4*)(p)));
}

template <int D, int KP, int VP>
struct WaveAttn {
  static constexpr int DC = D / 16;   // 16-wide d chunks of QK^T
  static constexpr int DB = D / 32;   // 32-row d blocks of O^T

  f32x16 acc[DB];
  float l_run;                        // this lane's partial row sum (its kv half)
  float m_run;                        // reference max (log2 units, scaled)

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    l_run = 0.f;
    m_run = kNoMax;
  }

  // S^T for kv rows [0, 32 NK) of an LDS block: k_lane = &K[c][8 j] (pitch
  // KP), so every fragment read is the base plus a compile-time offset.
  template <int NK>
  __device__ __forceinline__ void qk(f32x16 (&sc)[NK], const uint16_t* __restrict__ k_lane,
                                     const bf16x8 (&qf)[DC]) const {
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
      sc[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(k_lane + 32 * kb * KP), qf[0], f32x16{});
#pragma unroll
    for (int dc = 1; dc < DC; ++dc)
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
        sc[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(k_lane + 32 * kb * KP + 16 * dc), qf[dc], sc[kb]);
  }

  // The softmax and PV of one block come in three parts, so that a caller can
  // interleave the S^T MFMAs of the next block with this block's exp work.
  //
  // (1) Mask, row max and the lazy rescale (the only branches), in two
  // parts so that a caller can compute a block's max ahead of its rescale.
  // Only rows in [valid_lo, valid_hi) whose bit in `absent` is clear count;
  // the rest are masked (a wave-uniform branch, taken only by a partial block
  // or one with absent rows).  valid_hi must be >= valid_lo.
  // (1a) Mask in place; returns the block's row max, scaled (log2 units).
  template <int NK>
  __device__ __forceinline__ float block_max(f32x16 (&sc)[NK], float sl2, int valid_hi, int j,
                                             int valid_lo = 0, uint64_t absent = 0) const {
    if (__builtin_expect(valid_hi < 32 * NK || valid_lo > 0 || absent != 0, 0)) {
      // rows r valid iff valid_lo <= r < valid_hi, as one unsigned compare
      const unsigned span = (unsigned)(valid_hi - valid_lo);
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
        const uint32_t half = (uint32_t)(absent >> (32 * kb)) >> (4 * j);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * kb + 8 * (i >> 2) + 4 * j + (i & 3);
          if ((unsigned)(r - valid_lo) >= span || ((half >> (8 * (i >> 2) + (i & 3))) & 1u)) sc[kb][i] = -INFINITY;
        }
      }
    }
    float mx = max_f(sc[0][0], sc[0][1]);
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int i = kb ? 0 : 2; i < 16; i += 2) mx = max_f(max_f(mx, sc[kb][i]), sc[kb][i + 1]);
    return max_halves(mx) * sl2;
  }

  // (1b) The lazy rescale for a block whose scaled row max is ms.
  __device__ __forceinline__ void rescale(float ms) {
    const bool need = ms > m_run + kRescaleLog2;
    if (__ballot(need)) {
      const float m_new = need ? ms : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      l_run *= alpha;
    }
  }

  template <int NK>
  __device__ __forceinline__ void prep(f32x16 (&sc)[NK], float sl2, int valid_hi, int j,
                                       int valid_lo = 0, uint64_t absent = 0) {
    rescale(block_max<NK>(sc, sl2, valid_hi, j, valid_lo, absent));
  }

  // (2) p = 2^(s * sl2 - m) in place, the row sums (float32, unrounded p)
  // and the bf16 P fragments (B operands of
  // PV: fragment 2 kb + h holds the lane's registers 8 h .. 8 h + 7 of block
  // kb).  With NXT, the S^T MFMAs of the next block (K at k_next) are issued
  // interleaved with that VALU work, about five VALU ops per MFMA.
  //
  // FENCE > 0 (with NXT): the same work in a fixed order, fenced from the
  // scheduler: the K fragment of MFMA m + 2 is read before MFMA m, and each
  // MFMA is followed by its share of the exp work (16 / DC elements) and the
  // P fragments that share completes.  For callers whose register pressure
  // makes the scheduler drop the grouped order above, which leaves every
  // MFMA waiting on its own K read and the exp work after the last MFMA.
  // FENCE == 2 also pins each exp result and P fragment to its slot with an
  // empty asm statement, for callers where instruction selection otherwise
  // moves that arithmetic past the fences (it can cost registers).
  template <int NK, bool NXT, int FENCE = 0>
  __device__ __forceinline__ void exp_qk(f32x16 (&sc)[NK], bf16x8 (&pf)[2 * NK], f32x16 (&sn)[NK],
                                         const uint16_t* __restrict__ k_next,
                                         const bf16x8 (&qf)[DC], float sl2) {
    if constexpr (NXT && FENCE > 0) {
      constexpr int M = NK * DC;             // S^T MFMAs, dc outer
      constexpr int EPM = 16 * NK / M;       // exp elements per MFMA
      static_assert(EPM * M == 16 * NK && M >= 2, "exp work must split evenly over the MFMAs");
      const float neg_m = -m_run;
      float ps = 0.f;
      auto kfrag = [&](int m) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(k_next + 32 * (m % NK) * KP + 16 * (m / NK));
      };
      bf16x8 k0 = kfrag(0), k1 = kfrag(1);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        bf16x8 k2;
        if (m + 2 < M) k2 = kfrag(m + 2);
        __builtin_amdgcn_sched_barrier(0);
        sn[m % NK] = mfma32x32x16(k0, qf[m / NK], m < NK ? f32x16{} : sn[m % NK]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = m * EPM; e < (m + 1) * EPM; ++e) {
          float p = __builtin_amdgcn_exp2f(fmaf(sc[e / 16][e % 16], sl2, neg_m));
          if constexpr (FENCE == 2) asm volatile("" : "+v"(p));
          sc[e / 16][e % 16] = p;
          ps += p;
        }
#pragma unroll
        for (int p = 0; p < 2 * NK; ++p)
          if (8 * p + 7 >= m * EPM && 8 * p + 7 < (m + 1) * EPM) {
            const f32x16& v = sc[p / 2];
            const int o = 8 * (p % 2);
            pf[p] = bf16x8{(__bf16)v[o + 0], (__bf16)v[o + 1], (__bf16)v[o + 2], (__bf16)v[o + 3],
                           (__bf16)v[o + 4], (__bf16)v[o + 5], (__bf16)v[o + 6], (__bf16)v[o + 7]};
            if constexpr (FENCE == 2) asm volatile("" : "+v"(pf[p]));
          }
        __builtin_amdgcn_sched_barrier(0);
        k0 = k1;
        k1 = k2;
      }
      l_run += ps;
      return;
    }
    const float neg_m = -m_run;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[kb][i] = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], sl2, neg_m));
        ps += sc[kb][i];
      }
    l_run += ps;
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pf[2 * kb + h] = bf16x8{(__bf16)sc[kb][8 * h + 0], (__bf16)sc[kb][8 * h + 1],
                                (__bf16)sc[kb][8 * h + 2], (__bf16)sc[kb][8 * h + 3],
                                (__bf16)sc[kb][8 * h + 4], (__bf16)sc[kb][8 * h + 5],
                                (__bf16)sc[kb][8 * h + 6], (__bf16)sc[kb][8 * h + 7]};
    if constexpr (NXT) {
      qk<NK>(sn, k_next, qf);
      // schedule: four K fragment reads ahead, then per MFMA about five VALU
      // ops and the next fragment read
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int m = 0; m < NK * DC; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
        if (m + 4 < NK * DC) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  }

  // (3) O^T += V^T P^T.  v_lane = V + v_lane_offset(lane, VP) (row-major V,
  // pitch VP).  Only the first n16 16-row pieces are accumulated: the caller
  // passes fewer when the rest hold only masked rows (p = 0 against zero V
  // rows, so skipping them changes nothing).
  //
  // AHEAD (every piece, no n16): the V reads of MFMA m + 1 are issued before
  // MFMA m, fenced from the scheduler, so their LDS latency overlaps the MFMA
  // before them (left alone, the compiler short of registers issues each
  // MFMA's reads just before it and waits for them).
  template <int NK, bool AHEAD = false>
  __device__ __forceinline__ void pv(const bf16x8 (&pf)[2 * NK], const uint16_t* __restrict__ v_lane,
                                     int n16 = 2 * NK) {
    if constexpr (AHEAD) {
      constexpr int M = 2 * NK * DB;
      auto read_v = [&](int m) __attribute__((always_inline)) {
        const int piece = m / DB, db = m % DB;
        const uint16_t* vp = v_lane + 16 * piece * VP + 32 * db;
        const bf16x4 lo = lds_read_tr16(vp);
        const bf16x4 hi = lds_read_tr16(vp + 8 * VP);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      bf16x8 va = read_v(0);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        bf16x8 vn;
        if (m + 1 < M) vn = read_v(m + 1);
        __builtin_amdgcn_sched_barrier(0);
        acc[m % DB] = mfma32x32x16(va, pf[m / DB], acc[m % DB]);
        __builtin_amdgcn_sched_barrier(0);
        if (m + 1 < M) va = vn;
      }
      return;
    }
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (2 * kb + h >= n16) break;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* vp = v_lane + (32 * kb + 16 * h) * VP + 32 * db;
          const bf16x4 lo = lds_read_tr16(vp);
          const bf16x4 hi = lds_read_tr16(vp + 8 * VP);
          const bf16x8 va = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[db] = mfma32x32x16(va, pf[2 * kb + h], acc[db]);
        }
      }
    }
  }

  // One whole block step, no interleaving.
  template <int NK>
  __device__ __forceinline__ void step(const uint16_t* __restrict__ k_lane,
                                       const uint16_t* __restrict__ v_lane, const bf16x8 (&qf)[DC],
                                       float sl2, int valid_hi, int j, int valid_lo = 0) {
    f32x16 sc[NK];
    bf16x8 pf[2 * NK];
    qk<NK>(sc, k_lane, qf);
    prep<NK>(sc, sl2, valid_hi, j, valid_lo);
    exp_qk<NK, false>(sc, pf, sc, nullptr, qf, sl2);
    pv<NK>(pf, v_lane, min(2 * NK, (valid_hi + 15) >> 4));
  }

  // One kv row j that is the only counted row of its block (the row past
  // the last full block of a chunk of C + 1 rows).  Its scores come from
  // VALU dot products instead of a 32-row S^T block whose other 31 rows would
  // be masked: k_row = &K[j][8 lh] holds the d values of the lane's query
  // fragments.  Then the lazy rescale, and the PV of one 16-row piece
  // (v_lane as in pv, at row j) whose P fragment holds only row j (element 0
  // of the lanes with lh = 0); the other 15 V rows get weight 0.  The row sum
  // takes p once, in the lh = 0 half.  Without PV only the softmax statistics
  // are updated (v_lane unused).
  template <bool PV = true>
  __device__ __forceinline__ void one_row(const uint16_t* __restrict__ k_row,
                                          const uint16_t* __restrict__ v_lane, const bf16x8 (&qf)[DC],
                                          float sl2, int lh) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float part[2] = {0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(k_row + 16 * dc);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part[e & 1] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{qf[dc][2 * e], qf[dc][2 * e + 1]},
                                                      bf16x2{kf[2 * e], kf[2 * e + 1]}, part[e & 1], false);
      if (dc & 1) __builtin_amdgcn_sched_barrier(0);   // at most two K fragments live
    }
    const float s = sum_halves(part[0] + part[1]);
    rescale(s * sl2);
    const float p = __builtin_amdgcn_exp2f(fmaf(s, sl2, -m_run));
    const float p0 = lh == 0 ? p : 0.f;
    l_run += p0;
    if constexpr (PV) {
      bf16x8 pf[2];
      pf[0] = bf16x8{(__bf16)p0, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f,
                     (__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
      pf[1] = pf[0];
      pv<1>(pf, v_lane, 1);
    }
  }

  // Full row sum (both kv halves) and natural-log normaliser.
  __device__ __forceinline__ float row_sum() const { return sum_halves(l_run); }
  __device__ __forceinline__ float lse(float l) const { return m_run * kLn2 + logf(l); }
};

// Query fragments (B operand of S^T): lane column c, d = 16 dc + 8 j ...
template <int DC, int STRIDE>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[DC], const uint16_t* row_plus_8j) {
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qf[dc] = *reinterpret_cast<const bf16x8*>(row_plus_8j + STRIDE * dc);
}

// Store a wavefront's O^T columns (times inv) as bf16 rows, 16 bytes per
// lane and store.  For accumulator block db and m-pair p, lane (c, j) holds
// d = 32 db + 16 p + 8 m' + 4 j + t (m' = 0, 1).  One v_permlane32_swap of the
// m' = 0 values (X) with the m' = 1 values (Y) leaves lane c with X of lanes
// c and c + 32 (d = 32 db + 16 p + 0..7) and lane c + 32 with Y of both
// (d = 32 db + 16 p + 8..15).  row_plus_8j = &O[row][8 j]; lanes c and c + 32
// (same row) must both take part.
template <int DB>
__device__ __forceinline__ void store_o_bf16(uint16_t* row_plus_8j, const f32x16 (&acc)[DB], float inv) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint32_t x[2], y[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        x[h] = pack_bf16x2(acc[db][8 * p + 2 * h] * inv, acc[db][8 * p + 2 * h + 1] * inv);
        y[h] = pack_bf16x2(acc[db][8 * p + 4 + 2 * h] * inv, acc[db][8 * p + 4 + 2 * h + 1] * inv);
      }
      const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false);
      *reinterpret_cast<u32x4*>(row_plus_8j + 32 * db + 16 * p) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
}

// Store a wavefront's O^T columns (times inv) as float32 rows: lane (c, j)
// holds d = 32 db + 8 m + 4 j + t (t = 0..3) of row c in registers 4 m + t
// of block db, 16 bytes per store.  row = &O[row][0].
template <int DB>
__device__ __forceinline__ void store_o_f32(float* row, const f32x16 (&acc)[DB], float inv, int j) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<f32x4*>(row + 32 * db + 8 * m + 4 * j) =
          f32x4{acc[db][4 * m] * inv, acc[db][4 * m + 1] * inv, acc[db][4 * m + 2] * inv, acc[db][4 * m + 3] * inv};
}

}  // namespace pdllm
