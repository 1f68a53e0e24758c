// C ABI of libpdllm (declared in include/pdllm.h): argument validation on the
// host, split planning, and kernel launches on the caller's stream.  Nothing
// here allocates device memory or synchronises with the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "pdllm.h"
#include "pdllm_internal.h"

static_assert(pdllm::kNoAllocScratchBytes == PDLLM_NOALLOC_SCRATCH_BYTES, "scratch size in the header");

namespace {

thread_local std::string g_last_error;

pdllm_status fail(pdllm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pdllm_status ok() {
  g_last_error.clear();
  return PDLLM_OK;
}

pdllm_status hip_status(int err, const char* what) {
  if (err == (int)hipSuccess) return PDLLM_OK;
  return fail(PDLLM_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == PDLLM_BF16 ? 2 : 4; }

bool d_supported(int dtype, int d) {
  if (dtype == PDLLM_BF16) return d == 64 || d == 128;
  return d == 16 || d == 32 || d == 64 || d == 128;
}

// Compute units of the current device, queried once per device.
int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cache[dev] = n;
  }
  return cache[dev];
}

pdllm_status check_pool(const pdllm_pool* pool) {
  if (pool == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "pool is NULL");
  if (pool->k == nullptr || pool->v == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "pool k/v is NULL");
  if (pool->dtype != PDLLM_F32 && pool->dtype != PDLLM_BF16)
    return fail(PDLLM_ERR_INVALID_ARG, "pool dtype %d is not PDLLM_F32 or PDLLM_BF16", pool->dtype);
  if (pool->n_slots < 1 || pool->slot_rows < 1 || pool->h_kv < 1 || pool->d < 1)
    return fail(PDLLM_ERR_INVALID_ARG, "pool sizes must be >= 1 (n_slots %d, slot_rows %d, h_kv %d, d %d)",
                pool->n_slots, pool->slot_rows, pool->h_kv, pool->d);
  if (!d_supported(pool->dtype, pool->d))
    return fail(PDLLM_ERR_UNSUPPORTED, "head dim %d is not supported for %s", pool->d,
                pool->dtype == PDLLM_BF16 ? "bf16 (64, 128)" : "f32 (16, 32, 64, 128)");
  const int64_t vec = pool->dtype == PDLLM_BF16 ? 8 : 4;
  if (pool->stride_head < pool->d || pool->stride_row < (int64_t)pool->h_kv * pool->d ||
      pool->stride_slot < (int64_t)pool->slot_rows * pool->stride_row)
    return fail(PDLLM_ERR_INVALID_ARG, "pool strides overlap (slot %lld, row %lld, head %lld)",
                (long long)pool->stride_slot, (long long)pool->stride_row, (long long)pool->stride_head);
  if (pool->stride_head % vec || pool->stride_row % vec || pool->stride_slot % vec)
    return fail(PDLLM_ERR_INVALID_ARG, "pool strides must be multiples of %lld elements", (long long)vec);
  if (!aligned16(pool->k) || !aligned16(pool->v))
    return fail(PDLLM_ERR_INVALID_ARG, "pool k/v must be 16-byte aligned");
  return PDLLM_OK;
}

pdllm_status check_tensor(const void* p, const char* name) {
  if (p == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(PDLLM_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return PDLLM_OK;
}

// Whether resolved rows (element offsets / 8 in 31 bits) can address the pool.
bool rows_addressable(const pdllm_pool* pool) {
  const int64_t pool_elems = (int64_t)(pool->n_slots - 1) * pool->stride_slot +
                             (int64_t)(pool->slot_rows - 1) * pool->stride_row;
  return (pool_elems >> 3) <= (int64_t)INT32_MAX;
}

pdllm::DecodeArgs base_decode_args(const pdllm_pool* pool, const pdllm_page_table* pt,
                                   const void* q, const void* k_resp, const void* v_resp,
                                   int l_d, int h_q, float scale, void* o, float* lse) {
  pdllm::DecodeArgs a{};
  a.pool_k = pool->k;
  a.pool_v = pool->v;
  a.ps_slot = pool->stride_slot;
  a.ps_row = pool->stride_row;
  a.ps_head = pool->stride_head;
  a.chunk_slot = pt->chunk_slot;
  a.sel_chunk = pt->sel_chunk;
  a.keep_rows = pt->keep_rows;
  a.idx_dummy = static_cast<const int32_t*>(q);   // any valid device memory of >= 16 bytes
  a.rows = pt->rows;
  a.rows_stride = (int64_t)pt->k_max * (pt->b + 1);
  a.q = q;
  a.k_resp = k_resp;
  a.v_resp = v_resp;
  a.o = o;
  a.lse = lse;
  a.n_chunks_per_seq = pt->n_chunks_per_seq;
  a.k_max = pt->k_max;
  a.b = pt->b;
  a.compact = pt->rows_compacted ? 1 : 0;
  a.l_d = l_d;
  a.h_q = h_q;
  a.h_kv = pool->h_kv;
  a.group = h_q / pool->h_kv;
  a.scale_log2 = scale * 1.4426950408889634f;
  return a;
}

pdllm_status check_decode(const pdllm_pool* pool, const pdllm_page_table* pt, int32_t n_seq,
                          int32_t l_d, int32_t h_q, int32_t num_splits) {
  pdllm_status st = check_pool(pool);
  if (st != PDLLM_OK) return st;
  if (pt == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "page table is NULL");
  if (n_seq < 1 || l_d < 1 || h_q < 1)
    return fail(PDLLM_ERR_INVALID_ARG, "n_seq, l_d and h_q must be >= 1 (got %d, %d, %d)", n_seq, l_d, h_q);
  if (h_q % pool->h_kv != 0)
    return fail(PDLLM_ERR_INVALID_ARG, "h_q %d is not a multiple of h_kv %d", h_q, pool->h_kv);
  if (num_splits < 0) return fail(PDLLM_ERR_INVALID_ARG, "num_splits must be >= 0");
  if (pt->n_chunks_per_seq < 1) return fail(PDLLM_ERR_INVALID_ARG, "n_chunks_per_seq must be >= 1");
  if (pt->k_max < 0 || pt->k_max > pt->n_chunks_per_seq)
    return fail(PDLLM_ERR_INVALID_ARG, "k_max %d outside [0, n_chunks_per_seq %d]", pt->k_max,
                pt->n_chunks_per_seq);
  if (pt->b < 0 || pt->b > pool->slot_rows - 1)
    return fail(PDLLM_ERR_INVALID_ARG, "b %d outside [0, slot_rows - 1 = %d]", pt->b, pool->slot_rows - 1);
  if (pt->k_per_seq == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "k_per_seq (host) is NULL");
  if (pt->rows_compacted != 0 && pt->rows_compacted != 1)
    return fail(PDLLM_ERR_INVALID_ARG, "rows_compacted must be 0 or 1 (got %d)", pt->rows_compacted);
  bool any_chunk = false;
  for (int s = 0; s < n_seq; ++s) {
    const int ks = pt->k_per_seq[s];
    if (ks < 0 || ks > pt->k_max)
      return fail(PDLLM_ERR_INVALID_ARG, "k_per_seq[%d] = %d outside [0, k_max %d]", s, ks, pt->k_max);
    any_chunk |= ks > 0;
  }
  // resolved rows (pdllm_resolve_rows) replace the index tables
  if (any_chunk && pt->rows == nullptr) {
    if (pt->chunk_slot == nullptr || pt->sel_chunk == nullptr)
      return fail(PDLLM_ERR_INVALID_ARG, "chunk_slot / sel_chunk is NULL");
    if (pt->b > 0 && !pt->rows_compacted && pt->keep_rows == nullptr)
      return fail(PDLLM_ERR_INVALID_ARG, "keep_rows is NULL");
  }
  if (pt->rows != nullptr) {
    if (pool->dtype != PDLLM_BF16) return fail(PDLLM_ERR_UNSUPPORTED, "resolved rows: bf16 pools only");
    if (reinterpret_cast<uintptr_t>(pt->rows) % 4 != 0)
      return fail(PDLLM_ERR_INVALID_ARG, "rows must be 4-byte aligned");
    if (!rows_addressable(pool))
      return fail(PDLLM_ERR_UNSUPPORTED, "resolved rows: the pool spans 2^34 elements or more");
  }
  return PDLLM_OK;
}

}  // namespace

pdllm_status pdllm_resolve_rows(const pdllm_pool* pool, const pdllm_page_table* pt, int32_t n_seq,
                                int32_t* rows, size_t rows_elems, void* stream) {
  pdllm_status st = check_pool(pool);
  if (st != PDLLM_OK) return st;
  if (pt == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "page table is NULL");
  if (n_seq < 1) return fail(PDLLM_ERR_INVALID_ARG, "n_seq must be >= 1 (got %d)", n_seq);
  if (pt->n_chunks_per_seq < 1) return fail(PDLLM_ERR_INVALID_ARG, "n_chunks_per_seq must be >= 1");
  if (pt->k_max < 0 || pt->k_max > pt->n_chunks_per_seq)
    return fail(PDLLM_ERR_INVALID_ARG, "k_max %d outside [0, n_chunks_per_seq %d]", pt->k_max,
                pt->n_chunks_per_seq);
  if (pt->b < 0 || pt->b > pool->slot_rows - 1)
    return fail(PDLLM_ERR_INVALID_ARG, "b %d outside [0, slot_rows - 1 = %d]", pt->b, pool->slot_rows - 1);
  if (pt->rows_compacted != 0 && pt->rows_compacted != 1)
    return fail(PDLLM_ERR_INVALID_ARG, "rows_compacted must be 0 or 1 (got %d)", pt->rows_compacted);
  const int64_t need = (int64_t)n_seq * pt->k_max * (pt->b + 1);
  if (need > 0) {
    if (pt->chunk_slot == nullptr || pt->sel_chunk == nullptr)
      return fail(PDLLM_ERR_INVALID_ARG, "chunk_slot / sel_chunk is NULL");
    if (pt->b > 0 && !pt->rows_compacted && pt->keep_rows == nullptr)
      return fail(PDLLM_ERR_INVALID_ARG, "keep_rows is NULL");
  }
  if (pool->dtype != PDLLM_BF16) return fail(PDLLM_ERR_UNSUPPORTED, "resolved rows: bf16 pools only");
  if (rows == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "rows is NULL");
  if (reinterpret_cast<uintptr_t>(rows) % 4 != 0) return fail(PDLLM_ERR_INVALID_ARG, "rows must be 4-byte aligned");
  if ((int64_t)rows_elems < need)
    return fail(PDLLM_ERR_INVALID_ARG, "rows holds %zu entries, %lld needed", rows_elems, (long long)need);
  if (!rows_addressable(pool))
    return fail(PDLLM_ERR_UNSUPPORTED, "resolved rows: the pool spans 2^34 elements or more");
  pdllm::ResolveArgs a{};
  a.chunk_slot = pt->chunk_slot;
  a.sel_chunk = pt->sel_chunk;
  a.keep_rows = pt->keep_rows;
  a.rows = rows;
  a.ps_slot = pool->stride_slot;
  a.ps_row = pool->stride_row;
  a.n_seq = n_seq;
  a.n_chunks_per_seq = pt->n_chunks_per_seq;
  a.k_max = pt->k_max;
  a.b = pt->b;
  a.compact = pt->rows_compacted ? 1 : 0;
  if ((st = hip_status(pdllm::launch_resolve_rows(a, stream), "resolve launch")) != PDLLM_OK) return st;
  return ok();
}

namespace {

// Validation of a decode call's scale and tensor pointers.
pdllm_status check_decode_io(float scale, const void* q, const void* k_resp, const void* v_resp, const void* o,
                             const float* lse) {
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PDLLM_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  pdllm_status st;
  if ((st = check_tensor(q, "q")) != PDLLM_OK) return st;
  if ((st = check_tensor(k_resp, "k_resp")) != PDLLM_OK) return st;
  if ((st = check_tensor(v_resp, "v_resp")) != PDLLM_OK) return st;
  if ((st = check_tensor(o, "o")) != PDLLM_OK) return st;
  if (lse != nullptr && !aligned16(lse)) return fail(PDLLM_ERR_INVALID_ARG, "lse must be 16-byte aligned");
  return PDLLM_OK;
}

// Whether the decode without splits can address the pool and the response
// rows with 32-bit byte offsets (bf16).
bool ws_addressable(const pdllm_pool* pool, int32_t n_seq, int32_t l_d) {
  const int64_t pool_elems = (int64_t)(pool->n_slots - 1) * pool->stride_slot +
                             (int64_t)(pool->slot_rows - 1) * pool->stride_row +
                             (int64_t)(pool->h_kv - 1) * pool->stride_head + pool->d;
  const int64_t resp_elems = (int64_t)n_seq * l_d * pool->h_kv * pool->d;
  return 2 * pool_elems <= (int64_t)UINT32_MAX && 2 * resp_elems <= (int64_t)UINT32_MAX;
}

// Validation of a decode call's shapes and options, then its split plan.
pdllm_status plan_call(const pdllm_pool* pool, const pdllm_page_table* pt, int32_t n_seq, int32_t l_d,
                       int32_t h_q, const pdllm_decode_opts* opts, pdllm::DecodePlan* plan) {
  if (opts == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "decode options are NULL");
  for (int r : opts->reserved)
    if (r != 0) return fail(PDLLM_ERR_INVALID_ARG, "reserved decode option fields must be 0");
  pdllm_status st = check_decode(pool, pt, n_seq, l_d, h_q, opts->num_splits);
  if (st != PDLLM_OK) return st;
  const int rows = opts->q_rows_per_wg;
  if (rows != 0) {
    const bool ok_rows = pool->dtype == PDLLM_BF16
                             ? rows == pdllm::kDecodeRowsBf16Small || rows == pdllm::kDecodeRowsBf16Large ||
                                   rows == pdllm::kDecodeRowsBf16Ws
                             : rows == pdllm::kDecodeRowsF32;
    if (!ok_rows)
      return fail(PDLLM_ERR_UNSUPPORTED, "q_rows_per_wg %d is not a workgroup shape of the %s kernel", rows,
                  pool->dtype == PDLLM_BF16 ? "bf16 (32, 128, 256)" : "f32 (64)");
  }
  if (opts->merge < 0 || opts->merge > 4)
    return fail(PDLLM_ERR_INVALID_ARG, "merge must be 0 .. 4 (got %d)", opts->merge);
  if ((opts->merge == 2 || opts->merge == 3) && pool->dtype != PDLLM_BF16)
    return fail(PDLLM_ERR_UNSUPPORTED, "the in-kernel merge is implemented for bf16 only");
  const char* err = "";
  if (!pdllm::plan_decode(pt->k_per_seq, n_seq, pt->b, l_d, h_q, pool->h_kv, pool->d, pool->dtype,
                          opts->num_splits, rows, opts->merge, device_cu_count(), plan, &err,
                          pool->dtype == PDLLM_BF16 && ws_addressable(pool, n_seq, l_d)))
    return fail(PDLLM_ERR_INVALID_ARG, "%s", err);
  // the 32-row decode addresses the pool and the response rows with 32-bit
  // byte offsets
  if (plan->ws && !ws_addressable(pool, n_seq, l_d))
    return fail(PDLLM_ERR_UNSUPPORTED, "32-row decode: the pool or the response rows span 4 GiB or more");
  // the in-kernel merge addresses its partials with 32-bit byte offsets
  if (plan->fused && plan->part_floats * plan->part_elem_bytes > (int64_t)INT32_MAX)
    return fail(PDLLM_ERR_UNSUPPORTED, "in-kernel merge: %lld bytes of partials exceed 2 GiB (use merge = 1)",
                (long long)(plan->part_floats * plan->part_elem_bytes));
  return PDLLM_OK;
}

// Validation and argument block of the chunk prefill (shared by the two
// entry points that run it).
pdllm_status prepare_prefill(const pdllm_pool* pool, const int32_t* chunk_slot, const int32_t* chunk_rows,
                             int32_t n_chunks, const void* q_chunk, int32_t h_q, const void* q_win, int32_t w,
                             int32_t chunks_per_win, float scale, void* o_chunk, float* key_score,
                             void* workspace, size_t workspace_bytes, pdllm::PrefillArgs* out);

pdllm_status launch_prefill_kernels(const pdllm::PrefillArgs& a, const pdllm_pool* pool, void* stream) {
  const bool streamed = pool->dtype == PDLLM_BF16 && pool->slot_rows > pdllm::kPrefillMaxRows;
  const int err = pool->dtype == PDLLM_F32 ? pdllm::launch_prefill_f32(a, pool->d, stream)
                  : streamed               ? pdllm::launch_prefill_stream(a, pool->d, stream)
                                           : pdllm::launch_prefill_bf16(a, pool->d, stream);
  return hip_status(err, "chunk prefill launch");
}

}  // namespace

extern "C" {

int pdllm_abi_version(void) { return PDLLM_ABI_VERSION; }

const char* pdllm_last_error(void) { return g_last_error.c_str(); }

size_t pdllm_prefill_score_workspace(int32_t n_chunks, int32_t h_q, int32_t h_kv, int32_t slot_rows,
                                     int32_t w) {
  if (n_chunks < 0 || h_kv < 1 || h_q < 1 || h_q % h_kv != 0 || slot_rows < 1 || w < 1) return 0;
  const auto align = [](int64_t b) { return (b + 255) / 256 * 256; };
  if (slot_rows <= pdllm::kPrefillMaxRows)   // resident kernel: per-wave partial key scores
    return (size_t)align((int64_t)n_chunks * h_kv * pdllm::kPrefillParts * slot_rows * 4);
  // streamed chunks: one partial row per (chunk, kv head), then the window
  // rows' normalisers (w * group rows, padded to 32)
  const int64_t rows_w = ((int64_t)w * (h_q / h_kv) + 31) / 32 * 32;
  return (size_t)(align((int64_t)n_chunks * h_kv * slot_rows * 4) + align((int64_t)n_chunks * h_kv * rows_w * 4));
}

pdllm_status pdllm_chunk_prefill_score(const pdllm_pool* pool, const int32_t* chunk_slot,
                                       const int32_t* chunk_rows, int32_t n_chunks,
                                       const void* q_chunk, int32_t h_q,
                                       const void* q_win, int32_t w, int32_t chunks_per_win,
                                       float scale, void* o_chunk, float* key_score,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  pdllm::PrefillArgs a{};
  pdllm_status st = prepare_prefill(pool, chunk_slot, chunk_rows, n_chunks, q_chunk, h_q, q_win, w, chunks_per_win,
                                    scale, o_chunk, key_score, workspace, workspace_bytes, &a);
  if (st != PDLLM_OK || n_chunks == 0) return st;
  if ((st = launch_prefill_kernels(a, pool, stream)) != PDLLM_OK) return st;
  if ((st = hip_status(pdllm::launch_score_finalize(a, stream), "score finalize launch")) != PDLLM_OK)
    return st;
  return ok();
}

pdllm_status pdllm_prefill_select(const pdllm_pool* pool, const int32_t* chunk_slot, const int32_t* chunk_rows,
                                  int32_t n_chunks, const void* q_chunk, int32_t h_q, const void* q_win, int32_t w,
                                  int32_t chunks_per_win, float scale, void* o_chunk, float* key_score, int32_t b,
                                  int32_t* keep_rows, const float* chunk_score, int32_t n_seq,
                                  const int32_t* k_per_seq, int32_t k_max, int32_t* sel_chunk,
                                  int32_t selected_only, void* workspace, size_t workspace_bytes, void* stream) {
  pdllm::PrefillArgs a{};
  pdllm_status st = prepare_prefill(pool, chunk_slot, chunk_rows, n_chunks, q_chunk, h_q, q_win, w, chunks_per_win,
                                    scale, o_chunk, key_score, workspace, workspace_bytes, &a);
  if (st != PDLLM_OK) return st;
  if (b < 0 || b > pool->slot_rows - 1)
    return fail(PDLLM_ERR_INVALID_ARG, "b %d outside [0, slot_rows - 1 = %d]", b, pool->slot_rows - 1);
  if (b > 0 && n_chunks > 0 && keep_rows == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "keep_rows is NULL");
  if (n_seq < 1 || n_chunks % n_seq != 0)
    return fail(PDLLM_ERR_INVALID_ARG, "n_seq %d must be >= 1 and divide n_chunks %d", n_seq, n_chunks);
  const int n_per_seq = n_chunks / n_seq;
  if (n_per_seq > 8192) return fail(PDLLM_ERR_UNSUPPORTED, "%d chunks per sequence > 8192", n_per_seq);
  if (k_max < 0 || k_max > n_per_seq)
    return fail(PDLLM_ERR_INVALID_ARG, "k_max %d outside [0, chunks per sequence %d]", k_max, n_per_seq);
  if (k_max > 0) {
    if (k_per_seq == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "k_per_seq (host) is NULL");
    for (int s = 0; s < n_seq; ++s)
      if (k_per_seq[s] < 0 || k_per_seq[s] > k_max)
        return fail(PDLLM_ERR_INVALID_ARG, "k_per_seq[%d] = %d outside [0, k_max %d]", s, k_per_seq[s], k_max);
    if (chunk_score == nullptr || sel_chunk == nullptr)
      return fail(PDLLM_ERR_INVALID_ARG, "chunk_score / sel_chunk is NULL");
  }
  if (selected_only != 0 && selected_only != 1)
    return fail(PDLLM_ERR_INVALID_ARG, "selected_only must be 0 or 1 (got %d)", selected_only);
  if (selected_only && chunk_score == nullptr)
    return fail(PDLLM_ERR_INVALID_ARG, "selected_only needs chunk_score");
  if (selected_only && k_max == 0 && k_per_seq == nullptr)
    return fail(PDLLM_ERR_INVALID_ARG, "k_per_seq (host) is NULL");
  if (n_chunks == 0) return ok();
  // only the selected chunks are scored: the sequences' K_s travel in the
  // launch arguments (up to kMaxSelSeq sequences; past that, every chunk is)
  const bool sel = selected_only && n_seq <= pdllm::kMaxSelSeq;
  if (sel) {
    a.sel_score = chunk_score;
    a.sel_per_seq = n_per_seq;
    int64_t scored = 0;
    for (int s = 0; s < n_seq; ++s) {
      a.sel_k[s] = k_max > 0 ? k_per_seq[s] : 0;
      scored += a.sel_k[s];
    }
    const int64_t n_cu = device_cu_count();
    a.rank_order = n_per_seq <= pdllm::kPrefillRankChunks && (int64_t)n_chunks * pool->h_kv > n_cu &&
                   scored * pool->h_kv <= n_cu;
  }
  if ((st = launch_prefill_kernels(a, pool, stream)) != PDLLM_OK) return st;
  pdllm::FinalizeSelectArgs f{};
  f.part = a.part_score;
  f.key_score = key_score;
  f.chunk_rows = chunk_rows;
  f.keep_rows = keep_rows;
  f.n_chunks = n_chunks;
  f.h_kv = a.h_kv;
  f.parts = a.parts;
  f.slot_rows = a.slot_rows;
  f.b = b;
  f.selected_only = sel ? 1 : 0;
  // top-K rides in the same launch for the first sequences, and in launches
  // of its own past kMaxTopkSeqPerLaunch of them
  for (int s0 = 0; s0 < std::max(n_seq, 1); s0 += pdllm::kMaxTopkSeqPerLaunch) {
    pdllm::TopkArgs& t = f.topk;
    t = pdllm::TopkArgs{};
    t.chunk_score = chunk_score;
    t.sel_chunk = sel_chunk;
    t.n_chunks = n_per_seq;
    t.k_max = k_max;
    t.seq0 = s0;
    t.n_seq_launch = k_max > 0 ? std::min(pdllm::kMaxTopkSeqPerLaunch, n_seq - s0) : 0;
    for (int i = 0; i < std::min(pdllm::kMaxTopkSeqPerLaunch, n_seq - s0); ++i)
      t.k[i] = k_max > 0 ? k_per_seq[s0 + i] : 0;
    if (s0 == 0) {
      st = hip_status(pdllm::launch_finalize_select(f, stream), "finalize / select launch");
    } else {
      st = hip_status(pdllm::launch_select_topk(t, stream), "top-K launch");
    }
    if (st != PDLLM_OK) return st;
  }
  return ok();
}

pdllm_status pdllm_select_topB(const float* key_score, const int32_t* chunk_rows, int32_t n_chunks,
                               int32_t slot_rows, int32_t b, int32_t* keep_rows, void* stream) {
  if (n_chunks < 0) return fail(PDLLM_ERR_INVALID_ARG, "n_chunks must be >= 0");
  if (slot_rows < 1) return fail(PDLLM_ERR_INVALID_ARG, "slot_rows must be >= 1");
  if (slot_rows > 4097) return fail(PDLLM_ERR_UNSUPPORTED, "slot_rows %d > 4097 is not supported", slot_rows);
  if (b < 0 || b > slot_rows - 1)
    return fail(PDLLM_ERR_INVALID_ARG, "b %d outside [0, slot_rows - 1 = %d]", b, slot_rows - 1);
  if (n_chunks == 0 || b == 0) return ok();
  if (key_score == nullptr || keep_rows == nullptr)
    return fail(PDLLM_ERR_INVALID_ARG, "key_score / keep_rows is NULL");
  pdllm_status st = hip_status(
      pdllm::launch_select_topb(key_score, chunk_rows, n_chunks, slot_rows, b, keep_rows, stream), "top-B launch");
  return st != PDLLM_OK ? st : ok();
}

pdllm_status pdllm_select_topK(const float* chunk_score, int32_t n_seq, int32_t n_chunks,
                               const int32_t* k_per_seq, int32_t k_max, int32_t* sel_chunk,
                               void* stream) {
  if (n_seq < 0) return fail(PDLLM_ERR_INVALID_ARG, "n_seq must be >= 0");
  if (n_chunks < 1) return fail(PDLLM_ERR_INVALID_ARG, "n_chunks must be >= 1");
  if (n_chunks > 8192) return fail(PDLLM_ERR_UNSUPPORTED, "n_chunks %d > 8192 is not supported", n_chunks);
  if (k_max < 0 || k_max > n_chunks)
    return fail(PDLLM_ERR_INVALID_ARG, "k_max %d outside [0, n_chunks %d]", k_max, n_chunks);
  if (n_seq == 0 || k_max == 0) return ok();
  if (k_per_seq == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "k_per_seq (host) is NULL");
  for (int s = 0; s < n_seq; ++s)
    if (k_per_seq[s] < 0 || k_per_seq[s] > k_max)
      return fail(PDLLM_ERR_INVALID_ARG, "k_per_seq[%d] = %d outside [0, k_max %d]", s, k_per_seq[s], k_max);
  if (chunk_score == nullptr || sel_chunk == nullptr)
    return fail(PDLLM_ERR_INVALID_ARG, "chunk_score / sel_chunk is NULL");
  for (int s0 = 0; s0 < n_seq; s0 += pdllm::kMaxTopkSeqPerLaunch) {
    pdllm::TopkArgs a{};
    a.chunk_score = chunk_score;
    a.sel_chunk = sel_chunk;
    a.n_chunks = n_chunks;
    a.k_max = k_max;
    a.seq0 = s0;
    a.n_seq_launch = std::min(pdllm::kMaxTopkSeqPerLaunch, n_seq - s0);
    for (int i = 0; i < a.n_seq_launch; ++i) a.k[i] = k_per_seq[s0 + i];
    pdllm_status st = hip_status(pdllm::launch_select_topk(a, stream), "top-K launch");
    if (st != PDLLM_OK) return st;
  }
  return ok();
}

pdllm_status pdllm_compact_kept_rows(const pdllm_pool* src, const int32_t* chunk_slot, int32_t n_chunks,
                                     const int32_t* keep_rows, int32_t b, void* dst_k, void* dst_v,
                                     int64_t dst_stride_slot, int64_t dst_stride_row,
                                     int64_t dst_stride_head, int32_t dst_slot_rows, void* stream) {
  pdllm_status st = check_pool(src);
  if (st != PDLLM_OK) return st;
  if (n_chunks < 0) return fail(PDLLM_ERR_INVALID_ARG, "n_chunks must be >= 0");
  if (b < 0 || b > src->slot_rows - 1)
    return fail(PDLLM_ERR_INVALID_ARG, "b %d outside [0, slot_rows - 1 = %d]", b, src->slot_rows - 1);
  if (dst_slot_rows < b + 1)
    return fail(PDLLM_ERR_INVALID_ARG, "dst_slot_rows %d < b + 1 = %d", dst_slot_rows, b + 1);
  // the destination must pass the same checks as a pool of the same shape
  pdllm_pool dst = *src;
  dst.k = dst_k;
  dst.v = dst_v;
  dst.stride_slot = dst_stride_slot;
  dst.stride_row = dst_stride_row;
  dst.stride_head = dst_stride_head;
  dst.slot_rows = dst_slot_rows;
  if ((st = check_pool(&dst)) != PDLLM_OK) return st;
  if (n_chunks == 0) return ok();
  if (chunk_slot == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "chunk_slot is NULL");
  if (b > 0 && keep_rows == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "keep_rows is NULL");
  const int64_t es = elem_bytes(src->dtype);
  pdllm::CompactArgs a{};
  a.src_k = static_cast<const char*>(src->k);
  a.src_v = static_cast<const char*>(src->v);
  a.dst_k = static_cast<char*>(dst_k);
  a.dst_v = static_cast<char*>(dst_v);
  a.ss = src->stride_slot * es;
  a.sr = src->stride_row * es;
  a.sh = src->stride_head * es;
  a.ds = dst_stride_slot * es;
  a.dr = dst_stride_row * es;
  a.dh = dst_stride_head * es;
  a.chunk_slot = chunk_slot;
  a.keep_rows = keep_rows;
  a.n_chunks = n_chunks;
  a.b = b;
  a.h_kv = src->h_kv;
  a.nvec = (int32_t)(src->d * es / 16);
  const int64_t total = (int64_t)(b + 1) * src->h_kv * a.nvec;
  const int64_t per_wg = (int64_t)pdllm::kCompactThreads * pdllm::kCompactVec;
  a.blocks = (int32_t)((total + per_wg - 1) / per_wg);
  if (total > INT32_MAX / 2 || (int64_t)n_chunks * 2 * a.blocks > INT32_MAX)
    return fail(PDLLM_ERR_UNSUPPORTED, "compaction grid too large");
  st = hip_status(pdllm::launch_compact(a, stream), "compaction launch");
  return st != PDLLM_OK ? st : ok();
}

pdllm_status pdllm_gather_kept_kv(const pdllm_pool* pool, const pdllm_page_table* pt, int32_t n_seq, void* dst_k,
                                  void* dst_v, int64_t dst_stride_slot, int64_t dst_stride_row,
                                  int64_t dst_stride_head, void* stream) {
  if (pt == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "page table is NULL");
  // the gather reads the index tables themselves (pt->rows is not used)
  pdllm_page_table tables = *pt;
  tables.rows = nullptr;
  pdllm_status st = check_decode(pool, &tables, n_seq, 1, pool != nullptr ? pool->h_kv : 1, 0);
  if (st != PDLLM_OK) return st;
  if (pt->rows_compacted) return fail(PDLLM_ERR_UNSUPPORTED, "gather: the pool must hold whole chunks");
  if (n_seq > pdllm::kMaxGatherSeq)
    return fail(PDLLM_ERR_UNSUPPORTED, "gather: %d sequences > %d", n_seq, pdllm::kMaxGatherSeq);
  // the destination passes the same checks as a pool of n_seq * k_max slots of b + 1 rows
  pdllm_pool dst = *pool;
  dst.k = dst_k;
  dst.v = dst_v;
  dst.stride_slot = dst_stride_slot;
  dst.stride_row = dst_stride_row;
  dst.stride_head = dst_stride_head;
  dst.slot_rows = pt->b + 1;
  dst.n_slots = std::max(1, n_seq * pt->k_max);
  if ((st = check_pool(&dst)) != PDLLM_OK) return st;
  if (pt->k_max == 0) return ok();
  const int64_t es = elem_bytes(pool->dtype);
  pdllm::CompactArgs a{};
  a.src_k = static_cast<const char*>(pool->k);
  a.src_v = static_cast<const char*>(pool->v);
  a.dst_k = static_cast<char*>(dst_k);
  a.dst_v = static_cast<char*>(dst_v);
  a.ss = pool->stride_slot * es;
  a.sr = pool->stride_row * es;
  a.sh = pool->stride_head * es;
  a.ds = dst_stride_slot * es;
  a.dr = dst_stride_row * es;
  a.dh = dst_stride_head * es;
  a.chunk_slot = pt->chunk_slot;
  a.keep_rows = pt->keep_rows;
  a.n_chunks = n_seq * pt->k_max;
  a.b = pt->b;
  a.h_kv = pool->h_kv;
  a.nvec = (int32_t)(pool->d * es / 16);
  a.sel_chunk = pt->sel_chunk;
  a.k_max = pt->k_max;
  a.n_chunks_per_seq = pt->n_chunks_per_seq;
  for (int s = 0; s < n_seq; ++s) a.k_s[s] = pt->k_per_seq[s];
  const int64_t total = (int64_t)(pt->b + 1) * pool->h_kv * a.nvec;
  const int64_t per_wg = (int64_t)pdllm::kCompactThreads * pdllm::kCompactVec;
  a.blocks = (int32_t)((total + per_wg - 1) / per_wg);
  if (total > INT32_MAX / 2 || (int64_t)a.n_chunks * 2 * a.blocks > INT32_MAX)
    return fail(PDLLM_ERR_UNSUPPORTED, "gather grid too large");
  st = hip_status(pdllm::launch_compact(a, stream), "gather launch");
  return st != PDLLM_OK ? st : ok();
}

size_t pdllm_chunk_score_workspace(int32_t n_chunks, int32_t n_query, int32_t n_pseudo) {
  if (n_chunks < 0 || n_query < 0 || n_pseudo < 0) return 0;
  return (size_t)(((int64_t)n_chunks * (n_query + n_pseudo) * 4 + 255) / 256 * 256);
}

pdllm_status pdllm_chunk_score(const void* logits, int32_t dtype, int64_t row_stride, int32_t vocab,
                               const int32_t* target, int32_t n_chunks, int32_t n_query, int32_t n_pseudo,
                               float* s_i, float* s_p, float* s, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (dtype != PDLLM_F32 && dtype != PDLLM_BF16) return fail(PDLLM_ERR_INVALID_ARG, "dtype %d is unknown", dtype);
  if (vocab < 1) return fail(PDLLM_ERR_INVALID_ARG, "vocab must be >= 1");
  if (row_stride < vocab) return fail(PDLLM_ERR_INVALID_ARG, "row_stride %lld < vocab %d", (long long)row_stride, vocab);
  if (n_chunks < 0 || n_query < 0 || n_pseudo < 0)
    return fail(PDLLM_ERR_INVALID_ARG, "n_chunks, n_query and n_pseudo must be >= 0");
  const int64_t rows = (int64_t)n_chunks * (n_query + n_pseudo);
  if (rows > INT32_MAX) return fail(PDLLM_ERR_UNSUPPORTED, "too many scored rows (%lld)", (long long)rows);
  if (n_chunks == 0) return ok();
  if (s == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "s is NULL");
  if (rows > 0) {
    pdllm_status st;
    if ((st = check_tensor(logits, "logits")) != PDLLM_OK) return st;
    if (target == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "target is NULL");
    const int64_t es = dtype == PDLLM_BF16 ? 2 : 4;
    if ((row_stride * es) % 16 != 0)
      return fail(PDLLM_ERR_INVALID_ARG, "row_stride * element size must be a multiple of 16 bytes");
  }
  const size_t need = pdllm_chunk_score_workspace(n_chunks, n_query, n_pseudo);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PDLLM_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  pdllm::ChunkScoreArgs a{};
  a.logits = logits;
  a.row_stride = row_stride;
  a.target = target;
  a.logp = static_cast<float*>(workspace);
  a.s_i = s_i;
  a.s_p = s_p;
  a.s = s;
  a.vocab = vocab;
  a.n_chunks = n_chunks;
  a.n_query = n_query;
  a.n_pseudo = n_pseudo;
  a.bf16 = dtype == PDLLM_BF16;
  return hip_status(pdllm::launch_chunk_score(a, stream), "chunk score launch");
}

pdllm_status pdllm_decode_plan(const int32_t* k_per_seq, int32_t n_seq, int32_t b, int32_t l_d,
                               int32_t h_q, int32_t h_kv, int32_t d, int32_t dtype,
                               int32_t num_splits, int32_t n_cu, int32_t* splits_per_seq,
                               int32_t* tiles_per_split, int32_t* q_rows_per_wg,
                               int64_t* workspace_bytes) {
  if (dtype != PDLLM_F32 && dtype != PDLLM_BF16) return fail(PDLLM_ERR_INVALID_ARG, "bad dtype %d", dtype);
  pdllm::DecodePlan plan;
  const char* err = "";
  if (!pdllm::plan_decode(k_per_seq, n_seq, b, l_d, h_q, h_kv, d, dtype, num_splits, 0, 0, n_cu, &plan, &err))
    return fail(PDLLM_ERR_INVALID_ARG, "%s", err);
  for (int s = 0; s < n_seq; ++s) {
    if (splits_per_seq) splits_per_seq[s] = plan.splits[s];
    if (tiles_per_split) tiles_per_split[s] = plan.tiles_per_split[s];
  }
  if (q_rows_per_wg) *q_rows_per_wg = plan.q_rows_per_wg;
  if (workspace_bytes) *workspace_bytes = plan.workspace_bytes;
  return ok();
}

size_t pdllm_split_attn_decode_ex_workspace(const pdllm_pool* pool, const pdllm_page_table* pt,
                                            int32_t n_seq, int32_t l_d, int32_t h_q,
                                            const pdllm_decode_opts* opts) {
  pdllm::DecodePlan plan;
  if (plan_call(pool, pt, n_seq, l_d, h_q, opts, &plan) != PDLLM_OK) return 0;
  return (size_t)plan.workspace_bytes;
}

size_t pdllm_split_attn_decode_workspace(const pdllm_pool* pool, const pdllm_page_table* pt,
                                         int32_t n_seq, int32_t l_d, int32_t h_q,
                                         int32_t num_splits) {
  pdllm_decode_opts o{};
  o.num_splits = num_splits;
  return pdllm_split_attn_decode_ex_workspace(pool, pt, n_seq, l_d, h_q, &o);
}

pdllm_status pdllm_split_attn_decode_ex(const pdllm_pool* pool, const pdllm_page_table* pt,
                                        const void* q, const void* k_resp, const void* v_resp,
                                        int32_t n_seq, int32_t l_d, int32_t h_q, float scale,
                                        const pdllm_decode_opts* opts, void* o, float* lse,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  pdllm::DecodePlan plan;
  pdllm_status st = plan_call(pool, pt, n_seq, l_d, h_q, opts, &plan);
  if (st != PDLLM_OK) return st;
  if ((st = check_decode_io(scale, q, k_resp, v_resp, o, lse)) != PDLLM_OK) return st;
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < (size_t)plan.workspace_bytes)
      return fail(PDLLM_ERR_WORKSPACE_TOO_SMALL, "workspace of %lld bytes needed, %zu given",
                  (long long)plan.workspace_bytes, workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned16(workspace)) return fail(PDLLM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }

  // Every launch's argument block is built and checked before the first one
  // is enqueued: a status other than PDLLM_OK from here on can only come
  // from the HIP runtime.
  pdllm::DecodeArgs a = base_decode_args(pool, pt, q, k_resp, v_resp, l_d, h_q, scale, o, lse);
  a.q_tiles = plan.q_tiles;
  if (plan.workspace_bytes > 0) {
    char* w = static_cast<char*>(workspace);
    if (plan.fused) a.sync = reinterpret_cast<int32_t*>(w);
    a.merge_kind = plan.fused ? (plan.fused_bf16 ? 2 : 1) : plan.sep_f32 ? 3 : 0;
    a.part_o = w + plan.sync_bytes;
    const int64_t part_bytes = (plan.part_floats * plan.part_elem_bytes + 255) / 256 * 256;
    a.part_lse = reinterpret_cast<float*>(w + plan.sync_bytes + part_bytes);
  }
  std::vector<pdllm::DecodeArgs> launches;
  std::vector<bool> merges;
  for (int s0 = 0; s0 < n_seq; s0 += pdllm::kMaxSeqPerLaunch) {
    const int n_here = std::min(pdllm::kMaxSeqPerLaunch, n_seq - s0);
    a.seq0 = s0;
    a.n_seq_launch = n_here;
    int64_t wg = 0;
    bool merge = false;
    for (int i = 0; i < pdllm::kMaxSeqPerLaunch; ++i) {
      pdllm::DecodeSeq& q_ = a.seq[i];
      q_ = pdllm::DecodeSeq{};
      if (i >= n_here) continue;
      const int s = s0 + i;
      q_.k_s = plan.k_s[s];
      q_.n_kv = plan.n_kv[s];
      q_.n_splits = plan.splits[s];
      q_.tiles_per_split = plan.tiles_per_split[s];
      q_.wg_begin = (int32_t)std::min<int64_t>(wg, INT32_MAX);
      q_.grp_begin = i * pool->h_kv * plan.q_tiles;
      q_.part_off = plan.part_off[s];
      q_.lse_off = plan.lse_off[s];
      wg += (int64_t)pool->h_kv * plan.q_tiles * plan.splits[s];
      merge |= plan.splits[s] > 1;
    }
    a.n_groups = n_here * pool->h_kv * plan.q_tiles;
    int64_t grid = wg;
    if (plan.ws) grid = (wg + pdllm::kXcdGroups - 1) / pdllm::kXcdGroups * pdllm::kXcdGroups;
    if (plan.fused) {             // every split of a merge group on one XCD
      std::vector<int> sizes;
      sizes.reserve(a.n_groups);
      for (int i = 0; i < n_here; ++i)
        for (int64_t k = 0; k < (int64_t)pool->h_kv * plan.q_tiles; ++k) sizes.push_back(a.seq[i].n_splits);
      grid = pdllm::kXcdGroups * pdllm::xcd_partition(sizes, a.xcd_grp);
    }
    if (grid > INT32_MAX) return fail(PDLLM_ERR_UNSUPPORTED, "decode grid too large (%lld workgroups)", (long long)grid);
    a.total_wg = (int32_t)wg;
    a.grid_wg = (int32_t)grid;
    launches.push_back(a);
    merges.push_back(merge);
  }
  for (size_t i = 0; i < launches.size(); ++i) {
    const pdllm::DecodeArgs& la = launches[i];
    const int e = plan.ws                     ? pdllm::launch_decode_ws(la, pool->d, stream)
                  : pool->dtype == PDLLM_BF16 ? pdllm::launch_decode_bf16(la, pool->d, plan.q_rows_per_wg, stream)
                                              : pdllm::launch_decode_f32(la, pool->d, stream);
    if ((st = hip_status(e, "decode launch")) != PDLLM_OK) return st;
    if (merges[i] && !plan.fused) {
      const bool bf16 = pool->dtype == PDLLM_BF16;
      st = hip_status(pdllm::launch_lse_merge(la, pool->d, bf16 && !plan.sep_f32, bf16, stream), "merge launch");
      if (st != PDLLM_OK) return st;
    }
  }
  return ok();
}

pdllm_status pdllm_split_attn_decode_noalloc(const pdllm_pool* pool, const pdllm_page_table* pt,
                                             const void* q, const void* k_resp, const void* v_resp,
                                             int32_t n_seq, int32_t l_d, int32_t h_q, float scale,
                                             int32_t num_splits, void* o, float* lse, void* stream) {
  pdllm_decode_opts opts{};
  opts.num_splits = num_splits;
  pdllm::DecodePlan plan;
  pdllm_status st = plan_call(pool, pt, n_seq, l_d, h_q, &opts, &plan);
  if (st != PDLLM_OK) return st;
  if ((st = check_decode_io(scale, q, k_resp, v_resp, o, lse)) != PDLLM_OK) return st;
  if ((size_t)plan.workspace_bytes > pdllm::kNoAllocScratchBytes)
    return fail(PDLLM_ERR_UNSUPPORTED,
                "this decode needs %lld bytes of scratch; the no-allocation entry point holds %zu bytes "
                "(use pdllm_split_attn_decode with a workspace)",
                (long long)plan.workspace_bytes, pdllm::kNoAllocScratchBytes);
  void* scratch = nullptr;
  if (plan.workspace_bytes > 0 &&
      (st = hip_status(pdllm::noalloc_scratch(&scratch), "scratch lookup")) != PDLLM_OK)
    return st;
  return pdllm_split_attn_decode_ex(pool, pt, q, k_resp, v_resp, n_seq, l_d, h_q, scale, &opts, o, lse, scratch,
                                    scratch != nullptr ? pdllm::kNoAllocScratchBytes : 0, stream);
}

pdllm_status pdllm_split_attn_decode(const pdllm_pool* pool, const pdllm_page_table* pt,
                                     const void* q, const void* k_resp, const void* v_resp,
                                     int32_t n_seq, int32_t l_d, int32_t h_q, float scale,
                                     int32_t num_splits, void* o, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  pdllm_decode_opts opts{};
  opts.num_splits = num_splits;
  return pdllm_split_attn_decode_ex(pool, pt, q, k_resp, v_resp, n_seq, l_d, h_q, scale, &opts, o, lse,
                                    workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

pdllm_status prepare_prefill(const pdllm_pool* pool, const int32_t* chunk_slot, const int32_t* chunk_rows,
                             int32_t n_chunks, const void* q_chunk, int32_t h_q, const void* q_win, int32_t w,
                             int32_t chunks_per_win, float scale, void* o_chunk, float* key_score,
                             void* workspace, size_t workspace_bytes, pdllm::PrefillArgs* out) {
  pdllm_status st = check_pool(pool);
  if (st != PDLLM_OK) return st;
  if (n_chunks < 0) return fail(PDLLM_ERR_INVALID_ARG, "n_chunks must be >= 0");
  if (h_q < 1 || h_q % pool->h_kv != 0)
    return fail(PDLLM_ERR_INVALID_ARG, "h_q %d must be a positive multiple of h_kv %d", h_q, pool->h_kv);
  if (w < 1 || chunks_per_win < 1)
    return fail(PDLLM_ERR_INVALID_ARG, "w and chunks_per_win must be >= 1 (got %d, %d)", w, chunks_per_win);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PDLLM_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  if (pool->slot_rows > 4097)
    return fail(PDLLM_ERR_UNSUPPORTED, "slot_rows %d > 4097 is not supported", pool->slot_rows);
  if (n_chunks == 0) return ok();
  if (chunk_slot == nullptr) return fail(PDLLM_ERR_INVALID_ARG, "chunk_slot is NULL");
  if ((st = check_tensor(q_chunk, "q_chunk")) != PDLLM_OK) return st;
  if ((st = check_tensor(q_win, "q_win")) != PDLLM_OK) return st;
  if ((st = check_tensor(o_chunk, "o_chunk")) != PDLLM_OK) return st;
  if ((st = check_tensor(key_score, "key_score")) != PDLLM_OK) return st;
  const size_t need = pdllm_prefill_score_workspace(n_chunks, h_q, pool->h_kv, pool->slot_rows, w);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(PDLLM_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed, %zu given", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(PDLLM_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  pdllm::PrefillArgs& a = *out;
  a = pdllm::PrefillArgs{};
  a.pool_k = pool->k;
  a.pool_v = pool->v;
  a.ps_slot = pool->stride_slot;
  a.ps_row = pool->stride_row;
  a.ps_head = pool->stride_head;
  a.chunk_slot = chunk_slot;
  a.chunk_rows = chunk_rows;
  a.q_chunk = q_chunk;
  a.q_win = q_win;
  a.o_chunk = o_chunk;
  a.key_score = key_score;
  a.part_score = static_cast<float*>(workspace);
  a.n_chunks = n_chunks;
  a.slot_rows = pool->slot_rows;
  a.h_q = h_q;
  a.h_kv = pool->h_kv;
  a.group = h_q / pool->h_kv;
  a.w = w;
  a.chunks_per_win = chunks_per_win;
  a.scale_log2 = scale * 1.4426950408889634f;
  const bool streamed = pool->dtype == PDLLM_BF16 && pool->slot_rows > pdllm::kPrefillMaxRows;
  a.parts = pool->dtype == PDLLM_BF16 && !streamed ? pdllm::kPrefillParts : 1;
  if (streamed) {
    const int64_t part_bytes = ((int64_t)n_chunks * pool->h_kv * pool->slot_rows * 4 + 255) / 256 * 256;
    a.win_norm = reinterpret_cast<float*>(static_cast<char*>(workspace) + part_bytes);
  }
  return PDLLM_OK;
}

}  // namespace
