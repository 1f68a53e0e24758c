// Split-KV chunk-sparse decode attention for float32 inputs.
//
// Same operation, work decomposition, split plan and partial format as the
// bf16 MFMA kernel (Prefilling-dLLM summary, Methodology 2 and 3; "Attention
// kernel optimization"), computed with exact float32 FMAs: one wavefront per
// (sequence, kv head, 64 query rows, split), one lane per query row.  Each
// 64-row kv tile is gathered from the pool slots into LDS through the page
// table, scores of 16 rows at a time are formed first, then the running max, sum
// and output are rescaled once per 16 rows.
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

constexpr int kTile = kDecodeTile;
constexpr int64_t kMaskedRow = INT64_MIN;

// Element offset of attended row v (pool rows >= 0, response rows -1 - offset);
// an absent kept row (entry -1 of a partial chunk) is kMaskedRow.
template <int D>
__device__ __forceinline__ int64_t resolve_row_f32(const DecodeArgs& a, int s, int g, int k_s,
                                                   int v) {
  const int per = a.b + 1;
  if (v < k_s * per) {
    const int k = v / per;
    const int r = v - k * per;
    const int cg = s * a.n_chunks_per_seq + a.sel_chunk[(int64_t)s * a.k_max + k];
    const int slot = a.chunk_slot[cg];
    int row = 0;
    if (r) {
      const int kr = a.keep_rows != nullptr ? a.keep_rows[(int64_t)cg * a.b + r - 1] : r;
      if (kr < 0) return kMaskedRow;
      row = a.compact ? r : kr;
    }
    return (int64_t)slot * a.ps_slot + (int64_t)row * a.ps_row + (int64_t)g * a.ps_head;
  }
  const int j = v - k_s * per;
  return -1 - ((((int64_t)s * a.l_d + j) * a.h_kv + g) * D);
}

template <int D>
__global__ __launch_bounds__(64) void decode_f32_kernel(const DecodeArgs a) {
  __shared__ float ks[kTile][D + 1];
  __shared__ float vs[kTile][D + 1];
  __shared__ int64_t rowoff[kTile];

  const int wg = xcd_remap(blockIdx.x, a.total_wg);
  const int si = last_index_le(a.n_seq_launch, wg, [&](int i) { return a.seq[i].wg_begin; });
  const int k_s = a.seq[si].k_s, n_kv = a.seq[si].n_kv;
  const int n_splits = a.seq[si].n_splits, tps = a.seq[si].tiles_per_split;
  int local = wg - a.seq[si].wg_begin;
  const int split = local % n_splits;
  local /= n_splits;
  const int qt = local % a.q_tiles;
  const int g = local / a.q_tiles;
  const int s = a.seq0 + si;
  const int n_tiles = (n_kv + kTile - 1) / kTile;
  const int t_begin = split * tps, t_end = min(t_begin + tps, n_tiles);
  const int lane = threadIdx.x;
  const int G = a.group;
  const int r = qt * kDecodeRowsF32 + lane;
  const bool valid = r < a.l_d * G;
  const int i = valid ? r / G : 0;
  const int h = g * G + (valid ? r - i * G : 0);

  float q[D], acc[D];
  {
    const float* qp = static_cast<const float*>(a.q) + (((int64_t)s * a.l_d + i) * a.h_q + h) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      q[e] = valid ? qp[e] : 0.f;
      acc[e] = 0.f;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;
  const float* pk = static_cast<const float*>(a.pool_k);
  const float* pv = static_cast<const float*>(a.pool_v);
  const float* rk = static_cast<const float*>(a.k_resp);
  const float* rv = static_cast<const float*>(a.v_resp);

  for (int t = t_begin; t < t_end; ++t) {
    const int v = t * kTile + lane;
    rowoff[lane] = v < n_kv ? resolve_row_f32<D>(a, s, g, k_s, v) : kMaskedRow;
    __syncthreads();
    for (int rr = 0; rr < kTile; ++rr) {
      const int64_t off = rowoff[rr];
      for (int e = lane; e < D; e += 64) {
        float kx = 0.f, vx = 0.f;
        if (off != kMaskedRow) {
          const bool pool = off >= 0;
          const int64_t x = (pool ? off : -1 - off) + e;
          kx = (pool ? pk : rk)[x];
          vx = (pool ? pv : rv)[x];
        }
        ks[rr][e] = kx;
        vs[rr][e] = vx;
      }
    }
    __syncthreads();
    const int nvalid = min(kTile, n_kv - t * kTile);
    constexpr int kSub = 16;               // rows scored before one rescale
    for (int r0 = 0; r0 < nvalid; r0 += kSub) {
      float z[kSub];
      float mx = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < kSub; ++rr) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) dot = fmaf(q[e], ks[r0 + rr][e], dot);
        z[rr] = r0 + rr < nvalid && rowoff[r0 + rr] != kMaskedRow ? dot * sl2 : -INFINITY;
        mx = fmaxf(mx, z[rr]);
      }
      const float m_new = fmaxf(m_run, mx);
      if (m_new == -INFINITY) continue;    // only masked rows so far
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
      for (int rr = 0; rr < kSub; ++rr) {
        const float p = exp2f(z[rr] - m_new);
        l_run += p;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] = fmaf(p, vs[r0 + rr][e], acc[e]);
      }
    }
    __syncthreads();
  }

  if (!valid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;   // a split of absent rows only: o = 0, lse = -inf
  const float lse_v = m_run * kLn2 + logf(l_run);
  if (n_splits == 1) {
    float* op = static_cast<float*>(a.o) + (((int64_t)s * a.l_d + i) * a.h_q + h) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) op[e] = acc[e] * inv;
    if (a.lse != nullptr) a.lse[((int64_t)s * a.h_q + h) * a.l_d + i] = lse_v;
  } else {
    float* pp = static_cast<float*>(a.part_o) + a.seq[si].part_off + (((int64_t)split * a.l_d + i) * a.h_q + h) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) pp[e] = acc[e] * inv;
    a.part_lse[a.seq[si].lse_off + ((int64_t)split * a.l_d + i) * a.h_q + h] = lse_v;
  }
}

}  // namespace

int launch_decode_f32(const DecodeArgs& a, int d, void* stream) {
  const dim3 grid(a.total_wg), block(64);
  switch (d) {
    case 16: hipLaunchKernelGGL(decode_f32_kernel<16>, grid, block, 0, (hipStream_t)stream, a); break;
    case 32: hipLaunchKernelGGL(decode_f32_kernel<32>, grid, block, 0, (hipStream_t)stream, a); break;
    case 64: hipLaunchKernelGGL(decode_f32_kernel<64>, grid, block, 0, (hipStream_t)stream, a); break;
    case 128: hipLaunchKernelGGL(decode_f32_kernel<128>, grid, block, 0, (hipStream_t)stream, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace pdllm
