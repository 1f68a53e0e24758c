// The attended pool rows of a decode page table, resolved once for the
// denoising steps that share it (Prefilling-dLLM summary, Methodology 2 and
// 3: the top-K chunks and their top-B rows are chosen once and the cached KV
// is reused at every step).  Entry (s, k, r) is the pool element offset / 8
// of row r (0 = the chunk's BOS row, then its kept rows) of the k-th selected
// chunk of sequence s, with bit 31 set for an absent kept row; the decode
// kernels add the kv head's offset.  One thread per entry; the two dependent
// index loads (sel_chunk, then chunk_slot and keep_rows) happen here once
// instead of in every decode call.
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

__global__ __launch_bounds__(256) void resolve_rows_kernel(const ResolveArgs a) {
  const int per = a.b + 1;
  const int64_t n = (int64_t)a.n_seq * a.k_max * per;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  const int64_t sk = idx / per;
  const int r = (int)(idx - sk * per);
  const int s = (int)(sk / a.k_max), k = (int)(sk - (int64_t)s * a.k_max);
  const int c = a.sel_chunk[(int64_t)s * a.k_max + k];
  const int cg = s * a.n_chunks_per_seq + min(max(c, 0), a.n_chunks_per_seq - 1);
  const int slot = a.chunk_slot[cg];
  int row = 0;
  bool absent = false;
  if (r > 0) {
    const int kr = a.keep_rows != nullptr ? a.keep_rows[(int64_t)cg * a.b + r - 1] : r;
    absent = kr < 0;
    row = absent ? 0 : a.compact ? r : kr;
  }
  const int64_t off = (int64_t)slot * a.ps_slot + (int64_t)row * a.ps_row;
  a.rows[idx] = (int32_t)((uint32_t)(off >> 3) | (absent ? 0x80000000u : 0u));
}

}  // namespace

int launch_resolve_rows(const ResolveArgs& a, void* stream) {
  const int64_t n = (int64_t)a.n_seq * a.k_max * (a.b + 1);
  if (n == 0) return (int)hipSuccess;
  hipLaunchKernelGGL(resolve_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace pdllm
