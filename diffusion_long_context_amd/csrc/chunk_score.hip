// Predictive chunk scores from the model's logits (Prefilling-dLLM summary,
// Methodology 1, predictive scoring: a chunk is scored by the negative
// log-likelihood of the query window given the chunk, s_I, and by the
// likelihood of the pseudo-labels given the chunk and the query, s_P, read
// as a log-likelihood; the top-K chunks by s = s_I + s_P are kept):
//   log p[r] = z[r][target[r]] - ln sum_v exp(z[r][v])   (row r of the logits)
//   s_I[c] = -sum_{t < n_query} log p[c][t],  s_P[c] = sum_{t >= n_query} log p[c][t]
//
// Design for CDNA4: the logits are read once, so the path is HBM-bound.
// One workgroup per row streams the row in 16-byte vectors (four in flight
// per thread) and keeps a running maximum and sum in base 2; one exp2 per
// logit, one rescale per vector.  The (max, sum) pairs combine lane by lane,
// then wave by wave, in a fixed order.  A second, tiny kernel adds each
// chunk's rows in a fixed order too, so the scores are bitwise reproducible.
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// (m, l) <- the pair for the union of the two value sets; m in log2 units,
// l = sum 2^(y - m).  An empty side has m = -inf, l = 0.
__device__ __forceinline__ void combine(float& m, float& l, float m2, float l2) {
  const float mn = max_f(m, m2);
  const float ref = mn == -INFINITY ? 0.f : mn;
  l = l * __builtin_amdgcn_exp2f(m - ref) + l2 * __builtin_amdgcn_exp2f(m2 - ref);
  m = mn;
}

template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4 w, float (&x)[BF16 ? 8 : 4]) {
  if constexpr (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = __uint_as_float(w[q] << 16);
      x[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = __uint_as_float(w[q]);
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void token_logp_kernel(const void* logits, int64_t row_stride,
                                                              int vocab, const int32_t* target, float* logp) {
  constexpr int EPV = BF16 ? 8 : 4;        // logits per 16-byte vector
  constexpr int ES = BF16 ? 2 : 4;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const char* base = static_cast<const char*>(logits) + row * row_stride * ES;
  typedef __attribute__((address_space(1))) const u32x4* gvec;
  const float kL2e = kLog2e;
  float m = -INFINITY, l = 0.f;
  auto add_vec = [&](const u32x4 w) {
    float x[EPV];
    unpack<BF16>(w, x);
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < EPV; ++e) mx = max_f(mx, x[e]);
    const float mn = max_f(m, mx * kL2e);
    const float ref = mn == -INFINITY ? 0.f : mn;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) s += __builtin_amdgcn_exp2f(fmaf(x[e], kL2e, -ref));
    l = fmaf(l, __builtin_amdgcn_exp2f(m - ref), s);
    m = mn;
  };
  const int n_vec = vocab / EPV;
  int v = tid;
  // kUnroll vectors per thread in flight: every load of a round is issued
  // before the first is used
  for (; v + (kUnroll - 1) * kThreads < n_vec; v += kUnroll * kThreads) {
    u32x4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = *(gvec)(base + (int64_t)(v + u * kThreads) * 16);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) add_vec(w[u]);
  }
  for (; v < n_vec; v += kThreads) add_vec(*(gvec)(base + (int64_t)v * 16));
  // the last vocab % EPV logits, one per thread
  for (int e = n_vec * EPV + tid; e < vocab; e += kThreads) {
    const float x = BF16 ? bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(base + (int64_t)e * 2))
                         : *reinterpret_cast<const float*>(base + (int64_t)e * 4);
    combine(m, l, x * kL2e, 1.f);
  }
  // lanes, then waves, in a fixed order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    combine(m, l, __shfl_xor(m, off, 64), __shfl_xor(l, off, 64));
  __shared__ float sm_m[kThreads / 64], sm_l[kThreads / 64];
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) {
    sm_m[wave] = m;
    sm_l[wave] = l;
  }
  __syncthreads();
  if (tid == 0) {
    float mm = sm_m[0], ll = sm_l[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) combine(mm, ll, sm_m[w], sm_l[w]);
    const int t = min(max(target[row], 0), vocab - 1);   // ids outside the vocabulary clamp into it
    const float zt = BF16 ? bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(base + (int64_t)t * 2))
                          : *reinterpret_cast<const float*>(base + (int64_t)t * 4);
    logp[row] = zt - (mm + __log2f(ll)) * kLn2;
  }
}

// One wavefront per chunk: lane j adds rows j, j + 64, ... (query rows into
// a, pseudo-label rows into b), then the lanes combine in a fixed xor tree.
__global__ __launch_bounds__(64) void chunk_sum_kernel(const float* logp, int n_query, int n_pseudo,
                                                       float* s_i, float* s_p, float* s) {
  const int c = blockIdx.x, lane = threadIdx.x;
  const int rows = n_query + n_pseudo;
  const float* r = logp + (int64_t)c * rows;
  float a = 0.f, b = 0.f;
  for (int t = lane; t < rows; t += 64) {
    const float v = r[t];
    if (t < n_query) a += v;
    else b += v;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a = wave_xor_sum(a, off);
    b = wave_xor_sum(b, off);
  }
  if (lane == 0) {
    if (s_i != nullptr) s_i[c] = -a;
    if (s_p != nullptr) s_p[c] = b;
    s[c] = b - a;
  }
}

}  // namespace

int launch_chunk_score(const ChunkScoreArgs& a, void* stream) {
  const int64_t rows = (int64_t)a.n_chunks * (a.n_query + a.n_pseudo);
  if (a.n_chunks == 0) return (int)hipSuccess;
  const hipStream_t st = (hipStream_t)stream;
  if (rows > 0 && a.bf16)
    hipLaunchKernelGGL(token_logp_kernel<true>, dim3((unsigned)rows), dim3(kThreads), 0, st, a.logits,
                       a.row_stride, a.vocab, a.target, a.logp);
  else if (rows > 0)
    hipLaunchKernelGGL(token_logp_kernel<false>, dim3((unsigned)rows), dim3(kThreads), 0, st, a.logits,
                       a.row_stride, a.vocab, a.target, a.logp);
  // with no scored rows every score is 0
  hipLaunchKernelGGL(chunk_sum_kernel, dim3(a.n_chunks), dim3(64), 0, st, a.logp, a.n_query, a.n_pseudo,
                     a.s_i, a.s_p, a.s);
  return (int)hipGetLastError();
}

}  // namespace pdllm
