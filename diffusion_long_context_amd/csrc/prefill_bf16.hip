// Chunk-local bidirectional attention with fused per-key window scoring,
// bf16 inputs, gfx950 MFMA.
//
// What it computes (Prefilling-dLLM summary, Methodology 1: every chunk,
// BOS row first, is attended only within itself, bidirectionally;
// Methodology 2: a chunk's rows are ranked by the cumulative attention weight
// they receive from the query tokens):
//   o_chunk[c,r,h]   = sum_j softmax_j(scale <q_chunk[c,r,h], K[slot,j,g]>) V[slot,j,g]
//   part[c,g,j]      = sum_{h in group g} sum_w softmax_j(scale <q_win[w,h], K[slot,j,g]>)
// and the finalize kernel sums part over g in a fixed order into key_score.
//
// Design for CDNA4: one workgroup of 8 wavefronts per (chunk, kv head).  The
// chunk's whole K (row-major) and V (transposed) for that kv head are staged
// into LDS once -- up to 288 rows x 128 d x 2 tensors, about 150 KiB of the
// 160 KiB -- and every query row of the G grouped heads streams past it, so
// HBM traffic is one read of Q and the pool slot and one write of O.
// Wavefronts take 32-row blocks round-robin: chunk-row blocks run
// S^T = K Q^T, an online softmax over 64-row kv steps and O^T += V^T P^T;
// window-row blocks run S = Q K^T (which leaves each lane one key column),
// an exact row softmax over all keys, and accumulate each key's weight in
// registers.  Per-wave key sums meet in LDS and are added in wave order.
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 288;              // slot_rows <= 257, padded to 32
constexpr int kMaxKb = kMaxRows / 16;      // 16-row kv blocks

template <int D>
struct PSmem {
  static constexpr int KP = D + 8;          // K pitch (elements)
  static constexpr int VP = kMaxRows + 4;   // V^T pitch: 292 = 4 mod 8 -> conflict-free 16-row reads
  uint16_t k[kMaxRows * KP];
  uint16_t vt[D * VP];
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(const PrefillArgs a) {
  __shared__ PSmem<D> sm;
  constexpr int KP = PSmem<D>::KP, VP = PSmem<D>::VP;
  constexpr int DC = D / 32, DB = D / 16;
  constexpr int TPR = D / 8;
  static_assert(kThreads % TPR == 0, "loader mapping");

  const int c = blockIdx.x / a.h_kv;
  const int g = blockIdx.x - c * a.h_kv;
  const int R = a.slot_rows;
  const int rpad = (R + 31) & ~31;
  const int nkb = rpad / 16;
  const int slot = a.chunk_slot[c];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lj = lane >> 4;
  const int G = a.group;
  const float sl2 = a.scale_log2;

  // ---- stage the chunk's K and V^T (rows >= R are zero)
  {
    const uint16_t* pk = static_cast<const uint16_t*>(a.pool_k);
    const uint16_t* pv = static_cast<const uint16_t*>(a.pool_v);
    const int64_t base = (int64_t)slot * a.ps_slot + (int64_t)g * a.ps_head;
    const int d0 = 8 * (tid % TPR);
    constexpr int kQuadsPerPass = kThreads / TPR;
    for (int r0 = 4 * (tid / TPR); r0 < rpad; r0 += 4 * kQuadsPerPass) {
      u32x4 kr[4], vr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        if (r < R) {
          const int64_t off = base + (int64_t)r * a.ps_row + d0;
          kr[i] = *reinterpret_cast<const u32x4*>(pk + off);
          vr[i] = *reinterpret_cast<const u32x4*>(pv + off);
        } else {
          kr[i] = vr[i] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&sm.k[(r0 + i) * KP + d0]) = kr[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1, sh = (e & 1) * 16;
        const uint32_t lo = ((vr[0][w] >> sh) & 0xffffu) | (((vr[1][w] >> sh) & 0xffffu) << 16);
        const uint32_t hi = ((vr[2][w] >> sh) & 0xffffu) | (((vr[3][w] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(&sm.vt[(d0 + e) * VP + r0]) = u32x2{lo, hi};
      }
    }
  }
  __syncthreads();

  const int n_rows_c = R * G;
  const int n_cb = (n_rows_c + 31) / 32;
  const int n_rows_w = a.w * G;
  const int n_wb = (n_rows_w + 31) / 32;
  const uint16_t* qc = static_cast<const uint16_t*>(a.q_chunk);
  const uint16_t* qw = static_cast<const uint16_t*>(a.q_win) +
                       (int64_t)(c / a.chunks_per_win) * a.w * a.h_q * D;
  uint16_t* oc = static_cast<uint16_t*>(a.o_chunk);

  float colsum[kMaxKb];                     // lane: key 16 kb + lr, summed over its rows
#pragma unroll
  for (int kb = 0; kb < kMaxKb; ++kb) colsum[kb] = 0.f;

  auto load_q = [&](const uint16_t* base, int first, int n_rows, bf16x8 (&qf)[2][DC]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int x = first + 16 * b + lr;
      if (x < n_rows) {
        const int r = x / G, h = g * G + (x - r * G);
        const uint16_t* p = base + ((int64_t)r * a.h_q + h) * D + 8 * lj;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) qf[b][dc] = *reinterpret_cast<const bf16x8*>(p + 32 * dc);
      } else {
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) qf[b][dc] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      }
    }
  };

  for (int item = wave; item < n_cb + n_wb; item += kWaves) {
    bf16x8 qf[2][DC];
    if (item < n_cb) {
      // ================= chunk rows: attention output =================
      const int first = item * 32;
      load_q(qc + (int64_t)c * R * a.h_q * D, first, n_rows_c, qf);
      f32x4 acc[DB][2];
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][0] = acc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

      auto step = [&](int kv0, auto nk_tag) {
        constexpr int NK = decltype(nk_tag)::value;       // 16-row kv blocks in this step
        f32x4 sc[NK][2];
#pragma unroll
        for (int kb = 0; kb < NK; ++kb) sc[kb][0] = sc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
#pragma unroll
          for (int kb = 0; kb < NK; ++kb) {
            const bf16x8 ka =
                *reinterpret_cast<const bf16x8*>(&sm.k[(kv0 + 16 * kb + lr) * KP + 32 * dc + 8 * lj]);
            sc[kb][0] = mfma16x16x32(ka, qf[0][dc], sc[kb][0]);
            sc[kb][1] = mfma16x16x32(ka, qf[1][dc], sc[kb][1]);
          }
        const bool tail = kv0 + 16 * NK > R;
        bf16x8 pf[NK / 2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NK; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = sc[kb][b][e] * sl2;
              if (tail && kv0 + 16 * kb + 4 * lj + e >= R) x = -INFINITY;
              sc[kb][b][e] = x;
              mx = fmaxf(mx, x);
            }
          mx = wave_xor_max(mx, 16);
          mx = wave_xor_max(mx, 32);
          const float m_new = fmaxf(m_run[b], mx);
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          const float alpha = exp2f(m_run[b] - m_use);
          m_run[b] = m_new;
          float psum = 0.f;
#pragma unroll
          for (int kb = 0; kb < NK; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p = exp2f(sc[kb][b][e] - m_use);
              sc[kb][b][e] = p;
              psum += p;
            }
          l_run[b] = l_run[b] * alpha + psum;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db][b] *= alpha;
#pragma unroll
          for (int kc = 0; kc < NK / 2; ++kc)
            pf[kc][b] = bf16x8{(__bf16)sc[2 * kc][b][0], (__bf16)sc[2 * kc][b][1],
                               (__bf16)sc[2 * kc][b][2], (__bf16)sc[2 * kc][b][3],
                               (__bf16)sc[2 * kc + 1][b][0], (__bf16)sc[2 * kc + 1][b][1],
                               (__bf16)sc[2 * kc + 1][b][2], (__bf16)sc[2 * kc + 1][b][3]};
        }
#pragma unroll
        for (int kc = 0; kc < NK / 2; ++kc)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint16_t* vp = &sm.vt[(16 * db + lr) * VP + kv0 + 32 * kc + 4 * lj];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 16);
            const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            acc[db][0] = mfma16x16x32(va, pf[kc][0], acc[db][0]);
            acc[db][1] = mfma16x16x32(va, pf[kc][1], acc[db][1]);
          }
      };
      int kv0 = 0;
      for (; kv0 + 64 <= rpad; kv0 += 64) step(kv0, std::integral_constant<int, 4>{});
      if (kv0 < rpad) step(kv0, std::integral_constant<int, 2>{});

#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float l = l_run[b];
        l = wave_xor_sum(l, 16);
        l = wave_xor_sum(l, 32);
        const int x = first + 16 * b + lr;
        if (x >= n_rows_c) continue;
        const int r = x / G, h = g * G + (x - r * G);
        const float inv = 1.f / l;
        uint16_t* op = oc + (((int64_t)c * R + r) * a.h_q + h) * D + 4 * lj;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f32x4 v = acc[db][b] * inv;
          *reinterpret_cast<u32x2*>(op + 16 * db) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    } else {
      // ================= window rows: per-key weight =================
      const int first = (item - n_cb) * 32;
      load_q(qw, first, n_rows_w, qf);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x4 sw[kMaxKb];
#pragma unroll
        for (int kb = 0; kb < kMaxKb; ++kb) {
          sw[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (kb < nkb) {
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) {
              const bf16x8 kf =
                  *reinterpret_cast<const bf16x8*>(&sm.k[(16 * kb + lr) * KP + 32 * dc + 8 * lj]);
              sw[kb] = mfma16x16x32(qf[b][dc], kf, sw[kb]);     // S[q = 4 lj + e][key = 16 kb + lr]
            }
          }
        }
        float mx[4], sum[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) mx[e] = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < kMaxKb; ++kb) {
          const bool live = kb < nkb && 16 * kb + lr < R;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = live ? sw[kb][e] * sl2 : -INFINITY;
            sw[kb][e] = x;
            mx[e] = fmaxf(mx[e], x);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mx[e] = wave_xor_max(mx[e], 1);
          mx[e] = wave_xor_max(mx[e], 2);
          mx[e] = wave_xor_max(mx[e], 4);
          mx[e] = wave_xor_max(mx[e], 8);
          sum[e] = 0.f;
        }
#pragma unroll
        for (int kb = 0; kb < kMaxKb; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = exp2f(sw[kb][e] - mx[e]);
            sw[kb][e] = p;
            sum[e] += p;
          }
        float wgt[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[e] = wave_xor_sum(sum[e], 1);
          sum[e] = wave_xor_sum(sum[e], 2);
          sum[e] = wave_xor_sum(sum[e], 4);
          sum[e] = wave_xor_sum(sum[e], 8);
          const bool valid = first + 16 * b + 4 * lj + e < n_rows_w;
          wgt[e] = valid ? 1.f / sum[e] : 0.f;
        }
#pragma unroll
        for (int kb = 0; kb < kMaxKb; ++kb)
          colsum[kb] += sw[kb][0] * wgt[0] + sw[kb][1] * wgt[1] + sw[kb][2] * wgt[2] + sw[kb][3] * wgt[3];
      }
    }
  }

  // ---- per-key sums: across the 4 lane groups, then across waves in order
#pragma unroll
  for (int kb = 0; kb < kMaxKb; ++kb) {
    colsum[kb] = wave_xor_sum(colsum[kb], 16);
    colsum[kb] = wave_xor_sum(colsum[kb], 32);
  }
  __syncthreads();                          // K/V no longer needed: reuse LDS
  float* red = reinterpret_cast<float*>(sm.k);
  if (lj == 0) {
#pragma unroll
    for (int kb = 0; kb < kMaxKb; ++kb) red[wave * kMaxRows + 16 * kb + lr] = colsum[kb];
  }
  __syncthreads();
  float* part = a.part_score + ((int64_t)c * a.h_kv + g) * R;
  for (int j = tid; j < R; j += kThreads) {
    float s = 0.f;
    for (int w = 0; w < kWaves; ++w) s += red[w * kMaxRows + j];
    part[j] = s;
  }
}

// key_score[c][j] = sum over kv heads g = 0 .. h_kv-1 (in that order) of part[c][g][j].
__global__ __launch_bounds__(256) void score_finalize_kernel(const float* part, int n_chunks,
                                                             int h_kv, int slot_rows,
                                                             float* key_score) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n_chunks * slot_rows) return;
  const int64_t c = idx / slot_rows, j = idx - c * slot_rows;
  float s = 0.f;
  for (int g = 0; g < h_kv; ++g) s += part[(c * h_kv + g) * slot_rows + j];
  key_score[idx] = s;
}

}  // namespace

int launch_prefill_bf16(const PrefillArgs& a, int d, void* stream) {
  if (a.n_chunks == 0) return (int)hipSuccess;
  const dim3 grid(a.n_chunks * a.h_kv), block(kThreads);
  if (d == 128)
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, block, 0, (hipStream_t)stream, a);
  else if (d == 64)
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, block, 0, (hipStream_t)stream, a);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_score_finalize(const PrefillArgs& a, void* stream) {
  const int64_t n = (int64_t)a.n_chunks * a.slot_rows;
  if (n == 0) return (int)hipSuccess;
  hipLaunchKernelGGL(score_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, a.part_score, a.n_chunks, a.h_kv, a.slot_rows, a.key_score);
  return (int)hipGetLastError();
}

}  // namespace pdllm
