// Compacted kept-row cache (Prefilling-dLLM summary, Methodology 2: after
// the intra-chunk selection only a chunk's top-B tokens stay in the KV
// cache).  For chunk c, held in slot s = chunk_slot[c]:
//   dst[s][0] = src[s][0]                       (the BOS anchor)
//   dst[s][1 + i] = src[s][keep_rows[c][i]]     (i < b, ascending rows)
// for every KV head, in K and in V.  An absent entry (-1: a partial chunk
// with fewer than b content rows) writes nothing.  The decode over the
// compacted pool then reads each selected chunk's b + 1 rows from
// consecutive slot rows.
//
// The same kernel gathers a decode's attended pool rows into one contiguous
// run per sequence (sel_chunk set): unit u = s k_max + k copies selected
// chunk c = sel_chunk[s][k] of sequence s (slot chunk_slot[s N + c]) to
// destination slot u, so with b + 1 rows per destination slot sequence s's
// rows sit contiguously, in the decode's order (the gather-to-contiguous
// copy that reading the pool in place avoids, kept as a comparator).
//
// Design for CDNA4: a pure copy, so the bound is HBM bandwidth.  The work of
// one (chunk, tensor) is a flat run of 16-byte vectors ordered (row, head,
// vector); each thread moves kCompactVec of them, kCompactThreads apart, with
// every load issued before the first store.  Indices past the end are
// clamped to the last vector for the loads (always a valid address) and
// skipped for the stores.  The kept-row index is the only dependent load.
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(const CompactArgs a) {
  // workgroup -> (chunk, tensor, block): blocks of one chunk's K and V are
  // adjacent, so one chunk's index row is read by neighbouring workgroups
  const int blk = blockIdx.x % a.blocks;
  const int ct = blockIdx.x / a.blocks;
  const int unit = ct >> 1;
  const bool is_v = ct & 1;
  const char* src = is_v ? a.src_v : a.src_k;
  char* dst = is_v ? a.dst_v : a.dst_k;
  const int per_row = a.h_kv * a.nvec;
  const int total = (a.b + 1) * per_row;
  const int f0 = blk * kCompactThreads * kCompactVec + (int)threadIdx.x;
  int c = unit;
  int64_t dslot;
  if (a.sel_chunk != nullptr) {            // gather: unit = (sequence, selected index)
    const int s = unit / a.k_max;
    const int sel = a.sel_chunk[unit];
    if (sel < 0 || unit - s * a.k_max >= a.k_s[s]) return;   // not selected (uniform)
    c = s * a.n_chunks_per_seq + sel;
    dslot = unit;
  } else {
    dslot = a.chunk_slot[c];
  }
  const int64_t slot = a.chunk_slot[c];
  typedef __attribute__((address_space(1))) const u32x4* gvec;
  typedef __attribute__((address_space(1))) const int32_t* gptr32;

  int r[kCompactVec], rem[kCompactVec], row[kCompactVec];
#pragma unroll
  for (int u = 0; u < kCompactVec; ++u) {
    const int f = min(f0 + u * kCompactThreads, total - 1);
    r[u] = f / per_row;
    rem[u] = f - r[u] * per_row;
  }
  // kept-row indices: clamped, always valid addresses (row 0 reads entry 0
  // and ignores it; with b = 0 there is no index row and chunk_slot is read)
#pragma unroll
  for (int u = 0; u < kCompactVec; ++u) {
    const int32_t* ip = a.b > 0 ? a.keep_rows + (int64_t)c * a.b + max(r[u] - 1, 0) : a.chunk_slot + c;
    row[u] = *(gptr32)ip;
  }
  u32x4 w[kCompactVec];
#pragma unroll
  for (int u = 0; u < kCompactVec; ++u) {
    const int h = rem[u] / a.nvec;
    const int vv = rem[u] - h * a.nvec;
    const int64_t sr = r[u] ? max(row[u], 0) : 0;    // an absent row reads the BOS row
    w[u] = *(gvec)(src + slot * a.ss + sr * a.sr + (int64_t)h * a.sh + 16 * (int64_t)vv);
  }
#pragma unroll
  for (int u = 0; u < kCompactVec; ++u) {
    if (f0 + u * kCompactThreads >= total || (r[u] > 0 && row[u] < 0)) continue;
    const int h = rem[u] / a.nvec;
    const int vv = rem[u] - h * a.nvec;
    *reinterpret_cast<u32x4*>(dst + dslot * a.ds + (int64_t)r[u] * a.dr + (int64_t)h * a.dh + 16 * (int64_t)vv) =
        w[u];
  }
}

}  // namespace

int launch_compact(const CompactArgs& a, void* stream) {
  if (a.n_chunks == 0) return (int)hipSuccess;
  const unsigned grid = (unsigned)((int64_t)a.n_chunks * 2 * a.blocks);
  hipLaunchKernelGGL(compact_kernel, dim3(grid), dim3(kCompactThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace pdllm
