// Host-only check of libpdllm's C-ABI layer and split planner, built with
// -fsanitize=address,undefined together with stub kernel launchers: every
// entry point is driven through its validation paths (invalid and valid
// arguments; fake device addresses that nothing dereferences) and the planner
// through a sweep of shapes, so that the sanitizers see every host-side code
// path.  Exits non-zero on an unexpected status.
#include <cstdio>
#include <cstdint>
#include <cmath>
#include <vector>

#include "pdllm.h"

namespace pdllm {
extern int g_launches;
}

static int g_fail = 0;
#define EXPECT(cond)                                                         \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, pdllm_last_error()); \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

static pdllm_pool pool_of(int dtype, int d, int rows = 257, int h_kv = 4, int n_slots = 128) {
  pdllm_pool p{};
  p.k = P(0x100000);
  p.v = P(0x200000);
  p.stride_head = d;
  p.stride_row = (int64_t)h_kv * d;
  p.stride_slot = (int64_t)rows * p.stride_row;
  p.n_slots = n_slots;
  p.slot_rows = rows;
  p.h_kv = h_kv;
  p.d = d;
  p.dtype = dtype;
  return p;
}

int main() {
  // ---- decode: invalid arguments, then valid calls that reach the launchers
  std::vector<int32_t> ks = {16};
  pdllm_pool pool = pool_of(PDLLM_BF16, 128);
  pdllm_page_table pt{};
  pt.chunk_slot = static_cast<const int32_t*>(P(0x300000));
  pt.sel_chunk = static_cast<const int32_t*>(P(0x310000));
  pt.keep_rows = static_cast<const int32_t*>(P(0x320000));
  pt.k_per_seq = ks.data();
  pt.n_chunks_per_seq = 128;
  pt.k_max = 16;
  pt.b = 256;
  void* q = P(0x400000);
  EXPECT(pdllm_split_attn_decode(nullptr, &pt, q, q, q, 1, 256, 28, 0.088f, 0, q, nullptr, nullptr, 0, nullptr) ==
         PDLLM_ERR_INVALID_ARG);
  EXPECT(pdllm_split_attn_decode(&pool, &pt, q, q, q, 1, 256, 27, 0.088f, 0, q, nullptr, nullptr, 0, nullptr) ==
         PDLLM_ERR_INVALID_ARG);
  EXPECT(pdllm_split_attn_decode(&pool, &pt, q, q, q, 1, 256, 28, -1.f, 0, q, nullptr, nullptr, 0, nullptr) ==
         PDLLM_ERR_INVALID_ARG);
  EXPECT(pdllm_split_attn_decode(&pool, &pt, q, q, q, 1, 256, 28, NAN, 0, q, nullptr, nullptr, 0, nullptr) ==
         PDLLM_ERR_INVALID_ARG);
  EXPECT(pdllm_split_attn_decode(&pool, &pt, q, q, q, 1, 256, 28, 0.088f, 0, q, nullptr, nullptr, 0, nullptr) ==
         PDLLM_ERR_WORKSPACE_TOO_SMALL);
  for (int merge = 0; merge <= 4; ++merge)
    for (int rows : {0, 128, 256})
      for (int ns : {0, 1, 3, 69}) {
        pdllm_decode_opts o{};
        o.num_splits = ns;
        o.q_rows_per_wg = rows;
        o.merge = merge;
        const size_t need = pdllm_split_attn_decode_ex_workspace(&pool, &pt, 1, 256, 28, &o);
        const int before = pdllm::g_launches;
        EXPECT(pdllm_split_attn_decode_ex(&pool, &pt, q, q, q, 1, 256, 28, 0.088f, &o, q, nullptr, P(0x1000000),
                                          need, nullptr) == PDLLM_OK);
        EXPECT(pdllm::g_launches > before);
      }
  // many sequences: several launches, mixed K_s, the in-kernel merge's XCD partition
  std::vector<int32_t> ks_many(70);
  for (int s = 0; s < 70; ++s) ks_many[s] = (7 * s) % 17;
  pdllm_page_table pt_many = pt;
  pt_many.k_per_seq = ks_many.data();
  for (int merge : {1, 3, 4}) {
    pdllm_decode_opts o{};
    o.merge = merge;
    const size_t need = pdllm_split_attn_decode_ex_workspace(&pool, &pt_many, 70, 64, 28, &o);
    EXPECT(pdllm_split_attn_decode_ex(&pool, &pt_many, q, q, q, 70, 64, 28, 0.088f, &o, q, nullptr, P(0x1000000), need,
                                      nullptr) == PDLLM_OK);
  }
  // no selected chunk: NULL index tables are accepted
  std::vector<int32_t> ks0 = {0, 0};
  pdllm_page_table pt0{};
  pt0.k_per_seq = ks0.data();
  pt0.n_chunks_per_seq = 4;
  pt0.b = 8;
  {
    const size_t need = pdllm_split_attn_decode_workspace(&pool, &pt0, 2, 300, 28, 0);
    EXPECT(pdllm_split_attn_decode(&pool, &pt0, q, q, q, 2, 300, 28, 0.088f, 0, q, nullptr, P(0x1000000), need,
                                   nullptr) == PDLLM_OK);
  }
  // f32 decode shapes
  for (int d : {16, 32, 64, 128}) {
    pdllm_pool pf = pool_of(PDLLM_F32, d, 65, 2, 16);
    std::vector<int32_t> k2 = {3};
    pdllm_page_table p2 = pt;
    p2.k_per_seq = k2.data();
    p2.n_chunks_per_seq = 16;
    p2.k_max = 4;
    p2.b = 20;
    const size_t need = pdllm_split_attn_decode_workspace(&pf, &p2, 1, 33, 6, 0);
    EXPECT(pdllm_split_attn_decode(&pf, &p2, q, q, q, 1, 33, 6, 0.125f, 0, q, nullptr, P(0x1000000), need,
                                   nullptr) == PDLLM_OK);
  }
  // the no-allocation entry point: plans beyond its scratch are rejected, others reach the scratch lookup
  EXPECT(pdllm_split_attn_decode_noalloc(&pool, &pt, q, q, q, 1, 256, 28, 0.088f, 69, q, nullptr, nullptr) ==
         PDLLM_ERR_UNSUPPORTED);
  EXPECT(pdllm_split_attn_decode_noalloc(&pool, &pt, q, q, q, 1, 256, 28, 0.088f, 0, q, nullptr, nullptr) ==
         PDLLM_ERR_HIP);
  // ---- planner sweep
  for (int n_seq : {1, 2, 5, 17})
    for (int kmax : {0, 1, 8, 33})
      for (int b : {0, 7, 128})
        for (int l_d : {1, 31, 256, 600})
          for (int ns : {0, 1, 4}) {
            std::vector<int32_t> k(n_seq);
            for (int s = 0; s < n_seq; ++s) k[s] = (s * 5 + kmax) % (kmax + 1);
            std::vector<int32_t> splits(n_seq), tps(n_seq);
            int32_t rows = 0;
            int64_t ws = 0;
            for (int dtype : {PDLLM_F32, PDLLM_BF16})
              EXPECT(pdllm_decode_plan(k.data(), n_seq, b, l_d, 28, 4, 128, dtype, ns, 256, splits.data(),
                                       tps.data(), &rows, &ws) == PDLLM_OK);
          }
  EXPECT(pdllm_decode_plan(ks.data(), 1, 8, 16, 6, 4, 128, PDLLM_BF16, 0, 256, nullptr, nullptr, nullptr, nullptr) ==
         PDLLM_ERR_INVALID_ARG);
  // ---- prefill, selection, compaction, gather, chunk scores
  const size_t pws = pdllm_prefill_score_workspace(128, 28, 4, 257, 64);
  EXPECT(pdllm_chunk_prefill_score(&pool, pt.chunk_slot, nullptr, 128, q, 28, q, 64, 128, 0.088f, q, (float*)q,
                                   P(0x1000000), pws, nullptr) == PDLLM_OK);
  EXPECT(pdllm_chunk_prefill_score(&pool, pt.chunk_slot, nullptr, 128, q, 28, q, 64, 128, 0.f, q, (float*)q,
                                   P(0x1000000), pws, nullptr) == PDLLM_ERR_INVALID_ARG);
  pdllm_pool big = pool_of(PDLLM_BF16, 128, 2049, 4, 16);
  const size_t sws = pdllm_prefill_score_workspace(16, 28, 4, 2049, 64);
  EXPECT(pdllm_chunk_prefill_score(&big, pt.chunk_slot, pt.chunk_slot, 16, q, 28, q, 64, 16, 0.088f, q, (float*)q,
                                   P(0x1000000), sws, nullptr) == PDLLM_OK);
  std::vector<int32_t> ks70(70, 1);
  EXPECT(pdllm_prefill_select(&pool, pt.chunk_slot, nullptr, 140, q, 28, q, 64, 2, 0.088f, q, (float*)q, 128,
                              (int32_t*)q, (const float*)q, 70, ks70.data(), 1, (int32_t*)q, 1, P(0x1000000),
                              pdllm_prefill_score_workspace(140, 28, 4, 257, 64), nullptr) == PDLLM_OK);
  EXPECT(pdllm_select_topB((const float*)q, nullptr, 128, 257, 128, (int32_t*)q, nullptr) == PDLLM_OK);
  EXPECT(pdllm_select_topB((const float*)q, nullptr, 128, 5000, 128, (int32_t*)q, nullptr) == PDLLM_ERR_UNSUPPORTED);
  EXPECT(pdllm_select_topK((const float*)q, 70, 128, ks70.data(), 16, (int32_t*)q, nullptr) == PDLLM_OK);
  EXPECT(pdllm_compact_kept_rows(&pool, pt.chunk_slot, 128, pt.keep_rows, 128, q, q, 129 * 512, 512, 128, 129,
                                 nullptr) == PDLLM_OK);
  EXPECT(pdllm_gather_kept_kv(&pool, &pt, 1, q, q, 257 * 512, 512, 128, nullptr) == PDLLM_OK);
  EXPECT(pdllm_gather_kept_kv(&pool, &pt_many, 40, q, q, 257 * 512, 512, 128, nullptr) == PDLLM_OK);
  EXPECT(pdllm_chunk_score(q, PDLLM_BF16, 152064, 152064, pt.chunk_slot, 128, 64, 64, nullptr, nullptr, (float*)q,
                           P(0x1000000), pdllm_chunk_score_workspace(128, 64, 64), nullptr) == PDLLM_OK);
  EXPECT(pdllm_abi_version() == PDLLM_ABI_VERSION);
  std::printf("host check: %d failure(s), %d launches reached\n", g_fail, pdllm::g_launches);
  return g_fail != 0;
}
