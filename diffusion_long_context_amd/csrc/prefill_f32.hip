// Chunk-local bidirectional attention with per-key window scoring for float32
// inputs (Prefilling-dLLM summary, Methodology 1 and 2), computed with exact
// float32 FMAs.  One workgroup per (chunk, kv head):
//  * chunk rows: one thread per (row, grouped head), an online softmax over
//    the chunk's rows read from the pool slot;
//  * window rows: threads first find each window row's softmax max and sum,
//    then one thread per key adds that key's weight over the window rows in
//    row order, so every sum has a fixed order.
// The workgroup writes its kv head's per-key partial sums; the finalize
// kernel (prefill_bf16.hip) adds the kv heads in order.
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

constexpr int kThreads = 256;

template <int D>
__device__ __forceinline__ float dot_row(const float* q, const float* k) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) s = fmaf(q[e], k[e], s);
  return s;
}

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(const PrefillArgs a) {
  __shared__ float wm[kThreads], wl[kThreads];
  __shared__ float colsum[4097];
  const int c = blockIdx.x / a.h_kv;
  const int g = blockIdx.x - c * a.h_kv;
  const int R = a.slot_rows, G = a.group;  // R: the layout's rows per chunk
  // rows this chunk holds (a partial last chunk holds fewer)
  const int Rc = a.chunk_rows != nullptr ? min(max(a.chunk_rows[c], 1), R) : R;
  const int slot = a.chunk_slot[c];
  const float* kb = static_cast<const float*>(a.pool_k) + (int64_t)slot * a.ps_slot + (int64_t)g * a.ps_head;
  const float* vb = static_cast<const float*>(a.pool_v) + (int64_t)slot * a.ps_slot + (int64_t)g * a.ps_head;
  const float sl2 = a.scale_log2;
  const int tid = threadIdx.x;

  // chunk rows
  const float* qc = static_cast<const float*>(a.q_chunk) + (int64_t)c * R * a.h_q * D;
  float* oc = static_cast<float*>(a.o_chunk) + (int64_t)c * R * a.h_q * D;
  for (int x = tid; x < Rc * G; x += kThreads) {
    const int r = x / G, h = g * G + (x - r * G);
    float q[D], acc[D];
#pragma unroll
    for (int e = 0; e < D; ++e) {
      q[e] = qc[((int64_t)r * a.h_q + h) * D + e];
      acc[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int j = 0; j < Rc; ++j) {
      const float z = dot_row<D>(q, kb + (int64_t)j * a.ps_row) * sl2;
      const float m_new = fmaxf(m, z);
      const float alpha = exp2f(m - m_new);
      const float p = exp2f(z - m_new);
      l = l * alpha + p;
      const float* v = vb + (int64_t)j * a.ps_row;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(p, v[e], acc[e] * alpha);
      m = m_new;
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) oc[((int64_t)r * a.h_q + h) * D + e] = acc[e] * inv;
  }

  // window rows -> per-key weight (only for a scored chunk; uniform)
  if (!chunk_scored(a, c)) return;
  const float* qw = static_cast<const float*>(a.q_win) + (int64_t)(c / a.chunks_per_win) * a.w * a.h_q * D;
  for (int j = tid; j < R; j += kThreads) colsum[j] = 0.f;
  const int n_win = a.w * G;
  for (int x0 = 0; x0 < n_win; x0 += kThreads) {
    const int x = x0 + tid;
    __syncthreads();
    if (x < n_win) {
      const int w = x / G, h = g * G + (x - w * G);
      const float* q = qw + ((int64_t)w * a.h_q + h) * D;
      float m = -INFINITY, l = 0.f;
      for (int j = 0; j < Rc; ++j) {
        const float z = dot_row<D>(q, kb + (int64_t)j * a.ps_row) * sl2;
        const float m_new = fmaxf(m, z);
        l = l * exp2f(m - m_new) + exp2f(z - m_new);
        m = m_new;
      }
      wm[tid] = m;
      wl[tid] = l;
    }
    __syncthreads();
    const int n_here = min(kThreads, n_win - x0);
    for (int j = tid; j < Rc; j += kThreads) {     // keys past Rc keep their 0
      const float* k = kb + (int64_t)j * a.ps_row;
      float s = colsum[j];
      for (int t = 0; t < n_here; ++t) {
        const int xx = x0 + t;
        const int w = xx / G, h = g * G + (xx - w * G);
        const float z = dot_row<D>(qw + ((int64_t)w * a.h_q + h) * D, k) * sl2;
        s += exp2f(z - wm[t]) / wl[t];
      }
      colsum[j] = s;
    }
  }
  __syncthreads();
  float* part = a.part_score + ((int64_t)c * a.h_kv + g) * a.parts * R;   // parts == 1
  for (int j = tid; j < R; j += kThreads) part[j] = colsum[j];
}

}  // namespace

int launch_prefill_f32(const PrefillArgs& a, int d, void* stream) {
  if (a.n_chunks == 0) return (int)hipSuccess;
  const dim3 grid(a.n_chunks * a.h_kv), block(kThreads);
  switch (d) {
    case 16: hipLaunchKernelGGL(prefill_f32_kernel<16>, grid, block, 0, (hipStream_t)stream, a); break;
    case 32: hipLaunchKernelGGL(prefill_f32_kernel<32>, grid, block, 0, (hipStream_t)stream, a); break;
    case 64: hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, (hipStream_t)stream, a); break;
    case 128: hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, (hipStream_t)stream, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace pdllm
