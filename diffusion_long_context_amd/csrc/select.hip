// Top-B row selection per chunk and top-K chunk selection per sequence
// (Prefilling-dLLM summary, Methodology 2: intra-chunk sparsity keeps the B
// rows of a chunk with the largest cumulative attention weight, inter-chunk
// sparsity keeps the K chunks with the largest score; Methodology 1: the K
// most relevant chunks by s are selected).
//
// Both selections are exact and integer-only: a float score becomes an
// order-preserving 32-bit key (-0 and +0 share one key, NaN gets the lowest
// key), and candidate i gets the 64-bit key (key << 32) | ~i so that equal
// scores rank the lower index first and all keys differ.  A candidate is kept
// iff fewer than `count` candidates have a larger key (its rank).  Up to
// kRankMax candidates each count the larger keys directly; above that a
// radix select finds the count-th largest 32-bit score key in four 8-bit
// histogram passes, and ties at that key go to the lowest indices.  Either
// way the kept ones are written in ascending index order with a workgroup
// prefix count, and the two give the same set.
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

constexpr int kThreads = 256;
constexpr int kRankMax = 256;               // candidates up to which ranks are counted directly
static_assert(kThreads == 256, "one radix histogram bin per thread");

// Workgroup-wide prefix count of a per-thread flag over one round of
// kThreads candidates, in index order: returns the number of flagged threads
// before this one, and the round's total in `total` (all threads).
__device__ __forceinline__ int round_prefix(bool flag, int* wave_counts, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t mask = __ballot(flag);
  if (lane == 0) wave_counts[wave] = __popcll(mask);
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_counts[w];
  total = 0;
  for (int w = 0; w < kThreads / 64; ++w) total += wave_counts[w];
  __syncthreads();
  return before + __popcll(mask & ((1ull << lane) - 1ull));
}

// The count-th largest 32-bit score key among n keys (the high halves of
// keys[]) by radix select, 0 < count < n: returns it, and in *need how many
// of the candidates equal to it are kept (the others above it all are).
// hist: 256 words of LDS.
__device__ uint32_t radix_threshold(const uint64_t* keys, int n, int count, uint32_t* hist, int* need) {
  const int tid = threadIdx.x;
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  uint32_t prefix = 0, mask = 0;
  int want = count;                          // keys still to take among those matching the prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;                           // kThreads == 256 bins
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t k = (uint32_t)(keys[i] >> 32);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // the digit where the count from the top reaches want: lane l holds
      // digits 255 - 4 l - j (j = 0..3), a prefix sum over the lanes gives the
      // count above each lane's digits, and one lane's range holds want
      int h[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = (int)hist[255 - 4 * tid - j];
        sum += h[j];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off, 64);
        if (tid >= off) incl += t;
      }
      int above = incl - sum;
      if (above < want && want <= incl) {
        int j = 0;
        for (; j < 3 && above + h[j] < want; ++j) above += h[j];
        s_prefix = prefix | ((uint32_t)(255 - 4 * tid - j) << shift);
        s_need = want - above;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    want = s_need;
    mask |= 255u << shift;
    __syncthreads();
  }
  *need = want;
  return prefix;
}

// Select the `count` best of the n keys in `keys` (LDS) and write their
// indices + `index_base`, ascending, to out[0..count).
__device__ void select_sorted(const uint64_t* keys, int n, int count, int index_base,
                              int32_t* out, int* wave_counts) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (count >= n) {                         // every candidate is kept
    for (int i = tid; i < n; i += kThreads) out[i] = i + index_base;
    return;
  }
  if (count <= 0) return;
  if (n > kRankMax) {
    __shared__ uint32_t hist[kThreads];
    int need = 0;
    const uint32_t thr = radix_threshold(keys, n, count, hist, &need);
    int written = 0, equal_seen = 0;
    for (int base = 0; base < n; base += kThreads) {
      const int i = base + tid;
      const uint32_t k = i < n ? (uint32_t)(keys[i] >> 32) : 0u;
      const bool eq = i < n && k == thr;
      int eq_total;
      const int eq_rank = equal_seen + round_prefix(eq, wave_counts, eq_total);
      equal_seen += eq_total;
      const bool keep = i < n && (k > thr || (eq && eq_rank < need));
      int keep_total;
      const int at = written + round_prefix(keep, wave_counts, keep_total);
      if (keep) out[at] = i + index_base;
      written += keep_total;
    }
    return;
  }
  int written = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    bool keep = false;
    if (i < n) {
      const uint64_t mine = keys[i];
      // the rank: how many keys are larger (8 LDS reads in flight at a time)
      int rank = 0;
      int j = 0;
      for (; j + 8 <= n; j += 8) {
        uint64_t kj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kj[u] = keys[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += kj[u] > mine ? 1 : 0;
      }
      for (; j < n; ++j) rank += keys[j] > mine ? 1 : 0;
      keep = rank < count;
    }
    const uint64_t mask = __ballot(keep);
    if (lane == 0) wave_counts[wave] = __popcll(mask);
    __syncthreads();
    int before = written;
    for (int w = 0; w < wave; ++w) before += wave_counts[w];
    const int in_wave = __popcll(mask & ((1ull << lane) - 1ull));
    if (keep) out[before + in_wave] = i + index_base;
    int round_total = 0;
    for (int w = 0; w < kThreads / 64; ++w) round_total += wave_counts[w];
    written += round_total;
    __syncthreads();
  }
}

// One workgroup per chunk.  Candidates are the content rows 1..R_c-1, R_c =
// chunk_rows[c] (slot_rows when absent).  A chunk with fewer than b of them
// keeps them all and fills the rest of its row with -1.
__global__ __launch_bounds__(kThreads) void topb_kernel(const float* key_score, const int32_t* chunk_rows,
                                                        int slot_rows, int b, int32_t* keep_rows) {
  __shared__ uint64_t keys[4096];
  __shared__ int wave_counts[kThreads / 64];
  const int c = blockIdx.x;
  const int rc = chunk_rows != nullptr ? min(max(chunk_rows[c], 1), slot_rows) : slot_rows;
  const int n = rc - 1;
  const int count = min(b, n);
  const float* row = key_score + (int64_t)c * slot_rows + 1;
  int32_t* out = keep_rows + (int64_t)c * b;
  for (int i = count + threadIdx.x; i < b; i += kThreads) out[i] = -1;
  for (int i = threadIdx.x; i < n; i += kThreads) keys[i] = rank_key(row[i], (uint32_t)i);
  __syncthreads();
  select_sorted(keys, n, count, 1, out, wave_counts);
}

// One workgroup per sequence; the K_s of this launch's sequences travel in
// the arguments.  Entries K_s..k_max-1 are set to -1.
__global__ __launch_bounds__(kThreads) void topk_kernel(const TopkArgs a) {
  __shared__ uint64_t keys[8192];
  __shared__ int wave_counts[kThreads / 64];
  const int si = blockIdx.x;
  const int s = a.seq0 + si;
  const int ks = a.k[si];
  const float* row = a.chunk_score + (int64_t)s * a.n_chunks;
  int32_t* out = a.sel_chunk + (int64_t)s * a.k_max;
  for (int i = threadIdx.x; i < a.n_chunks; i += kThreads) keys[i] = rank_key(row[i], (uint32_t)i);
  for (int i = ks + threadIdx.x; i < a.k_max; i += kThreads) out[i] = -1;
  __syncthreads();
  select_sorted(keys, a.n_chunks, ks, 0, out, wave_counts);
}

// Score finalize, top-B and top-K in one launch (see FinalizeSelectArgs).
// key_score[c][j] is the float sum of the partial rows in index order, the
// same operations as score_finalize_kernel, so the scores, and the rows
// selected from them, match the separate calls bit for bit.
__global__ __launch_bounds__(kThreads) void finalize_select_kernel(const FinalizeSelectArgs a) {
  __shared__ uint64_t keys[8192];
  __shared__ int wave_counts[kThreads / 64];
  const int blk = blockIdx.x;
  if (blk >= a.n_chunks) {                // top-K of one sequence
    const int si = blk - a.n_chunks;
    const int s = a.topk.seq0 + si;
    const int ks = a.topk.k[si];
    const float* row = a.topk.chunk_score + (int64_t)s * a.topk.n_chunks;
    int32_t* out = a.topk.sel_chunk + (int64_t)s * a.topk.k_max;
    for (int i = threadIdx.x; i < a.topk.n_chunks; i += kThreads) keys[i] = rank_key(row[i], (uint32_t)i);
    for (int i = ks + threadIdx.x; i < a.topk.k_max; i += kThreads) out[i] = -1;
    __syncthreads();
    select_sorted(keys, a.topk.n_chunks, ks, 0, out, wave_counts);
    return;
  }
  const int c = blk;
  if (a.selected_only) {                    // only the chunks top-K selects (uniform)
    const int s = c / a.topk.n_chunks;
    if (!in_top_k(a.topk.chunk_score + (int64_t)s * a.topk.n_chunks, a.topk.n_chunks, c - s * a.topk.n_chunks,
                  a.topk.k[s]))
      return;
  }
  const int R = a.slot_rows;
  const int n_part = a.h_kv * a.parts;
  const float* pc = a.part + (int64_t)c * n_part * R;
  // keys j and j + kThreads together: the partial loads of both (32 each,
  // clamped to valid addresses) are all in flight at once; each sum is
  // added in index order
  for (int j = threadIdx.x; j < R; j += 2 * kThreads) {
    constexpr int kGroup = 32;
    const int j2 = min(j + kThreads, R - 1);
    float x = 0.f, x2 = 0.f;
    for (int q0 = 0; q0 < n_part; q0 += kGroup) {
      float v[kGroup], v2[kGroup];
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        const int64_t q = min(q0 + u, n_part - 1);
        v[u] = pc[q * R + j];
        v2[u] = pc[q * R + j2];
      }
#pragma unroll
      for (int u = 0; u < kGroup; ++u)
        if (q0 + u < n_part) {
          x += v[u];
          x2 += v2[u];
        }
    }
    a.key_score[(int64_t)c * R + j] = x;
    if (j > 0) keys[j - 1] = rank_key(x, (uint32_t)(j - 1));
    if (j + kThreads < R) {
      a.key_score[(int64_t)c * R + j2] = x2;
      keys[j2 - 1] = rank_key(x2, (uint32_t)(j2 - 1));
    }
  }
  if (a.b == 0) return;
  const int rc = a.chunk_rows != nullptr ? min(max(a.chunk_rows[c], 1), R) : R;
  const int n = rc - 1;
  const int count = min(a.b, n);
  int32_t* out = a.keep_rows + (int64_t)c * a.b;
  for (int i = count + threadIdx.x; i < a.b; i += kThreads) out[i] = -1;
  __syncthreads();
  select_sorted(keys, n, count, 1, out, wave_counts);
}

}  // namespace

int launch_finalize_select(const FinalizeSelectArgs& a, void* stream) {
  const int grid = a.n_chunks + a.topk.n_seq_launch;
  if (grid == 0) return (int)hipSuccess;
  hipLaunchKernelGGL(finalize_select_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_select_topb(const float* key_score, const int32_t* chunk_rows, int n_chunks, int slot_rows,
                       int b, int32_t* keep_rows, void* stream) {
  if (n_chunks == 0 || b == 0) return (int)hipSuccess;
  hipLaunchKernelGGL(topb_kernel, dim3(n_chunks), dim3(kThreads), 0, (hipStream_t)stream,
                     key_score, chunk_rows, slot_rows, b, keep_rows);
  return (int)hipGetLastError();
}

int launch_select_topk(const TopkArgs& a, void* stream) {
  if (a.n_seq_launch == 0 || a.k_max == 0) return (int)hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_seq_launch), dim3(kThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace pdllm
