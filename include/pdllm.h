/*
 * pdllm.h -- C ABI of the chunk-sparse attention path of Prefilling-dLLM on
 * AMD Instinct MI355X (gfx950).
 *
 * Source of the operations: the technical summary of "Prefilling-dLLM:
 * Predictive Prefilling for Long-Context Inference in Diffusion Language
 * Models" (gist.science, paper 2606.10537), sections Methodology 1 ("Chunked
 * prefill and KV cache"), Methodology 2 ("Two-level sparsity"),
 * Methodology 3 ("Decoding with static KV reuse") and "Attention kernel
 * optimization".
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named "device" are device memory owned by the caller; the
 *   library never allocates, frees or retains them.  Pointers named "host"
 *   are read synchronously during the call and may be reused on return.
 * - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *   enqueued on it, nothing synchronises with the host, and no device memory
 *   is allocated, so the calls can be captured in a HIP graph.
 * - Arguments are validated on the host before anything is enqueued.  On
 *   PDLLM_ERR_INVALID_ARG, PDLLM_ERR_UNSUPPORTED and
 *   PDLLM_ERR_WORKSPACE_TOO_SMALL nothing was enqueued and the outputs are
 *   untouched.  PDLLM_ERR_HIP (the runtime refused a launch) can follow
 *   earlier launches of the same call, so the outputs are then undefined.
 *   pdllm_last_error() describes the problem.  The library never aborts and
 *   never throws across this boundary.
 * - The contents of device index tables are trusted (chunk ids, slots and
 *   rows must be in range); their shapes are checked.
 * - Floating data is PDLLM_F32 (float) or PDLLM_BF16 (bfloat16 bits, round
 *   to nearest even on output).  Softmax, accumulation and merges run in
 *   float32.  The softmax scale is an explicit argument (usually 1/sqrt(d)):
 *   it must be finite and > 0 (PDLLM_ERR_INVALID_ARG otherwise).
 * - Grouped-query attention: query head h reads KV head h / G with
 *   G = h_q / h_kv, i.e. G consecutive query heads share one KV head.
 * - Tensors are row-major with the last index contiguous.  Pool tensors
 *   carry explicit element strides; every other tensor is dense.
 * - bf16 tensors must be 16-byte aligned and their strides multiples of 8
 *   elements; f32 tensors 16-byte aligned with strides multiples of 4.
 */
#ifndef PDLLM_H
#define PDLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 11: pdllm_decode_opts.q_rows_per_wg = 32 (the decode without kv splits);
 *     pdllm_page_table.rows and pdllm_resolve_rows */
#define PDLLM_ABI_VERSION 11

typedef enum {
  PDLLM_OK = 0,
  PDLLM_ERR_INVALID_ARG = 1,        /* a null pointer, bad size or inconsistent shape */
  PDLLM_ERR_UNSUPPORTED = 2,        /* valid, but outside what the kernels implement  */
  PDLLM_ERR_WORKSPACE_TOO_SMALL = 3,/* workspace_bytes below the size query's answer  */
  PDLLM_ERR_HIP = 4                 /* a HIP runtime error while enqueueing            */
} pdllm_status;

typedef enum { PDLLM_F32 = 0, PDLLM_BF16 = 1 } pdllm_dtype;

/*
 * One layer's static chunk KV pool (Methodology 1 and 3: every chunk's KV is
 * computed once and cached; "Attention kernel optimization": the cached
 * chunks sit non-contiguously).  A slot holds one chunk: slot_rows = C + 1
 * rows, row 0 the chunk's BOS token, rows 1..C its tokens.
 *   k, v   device  [n_slots][slot_rows][h_kv][d] with element strides
 *                  stride_slot, stride_row, stride_head (d is contiguous)
 */
typedef struct {
  const void* k;
  const void* v;
  int64_t stride_slot;
  int64_t stride_row;
  int64_t stride_head;
  int32_t n_slots;
  int32_t slot_rows;
  int32_t h_kv;
  int32_t d;
  int32_t dtype;                    /* pdllm_dtype */
} pdllm_pool;

/*
 * The chunk page table of a decode call (Methodology 2: only the top-K
 * chunks of a sequence, and only the top-B rows of each, are attended).
 *   chunk_slot  device [n_seq * n_chunks_per_seq]   slot of chunk c of sequence
 *                      s at index s * n_chunks_per_seq + c
 *   sel_chunk   device [n_seq][k_max]   the selected chunk ids of a sequence
 *                      (its first k_per_seq[s] entries are used), as written
 *                      by pdllm_select_topK
 *   keep_rows   device [n_seq * n_chunks_per_seq][b]   kept content rows
 *                      (1..C) of every chunk, as written by pdllm_select_topB;
 *                      an entry of -1 is an absent row (a partial last chunk
 *                      with fewer than b content rows) and is not attended.
 *                      Absent entries must come after every kept row of
 *                      their chunk's row (pdllm_select_topB writes them so):
 *                      the decode finds a chunk's absent rows by its last
 *                      entry
 *   k_per_seq   host   [n_seq]   K_s, 0 <= K_s <= k_max
 *   (chunk_slot, sel_chunk and keep_rows may be NULL when every K_s is 0:
 *   they are then not read)
 *   rows_compacted  0: the pool holds whole chunks and keep_rows names the
 *                      kept rows;  1: the pool holds compacted slots (the
 *                      layout pdllm_compact_kept_rows writes), whose kept
 *                      rows are rows 1..b in order -- keep_rows is then read
 *                      only for its absent (-1) entries, and may be NULL when
 *                      there are none
 *   rows        device [n_seq][k_max (b + 1)] or NULL: the same attended pool
 *                      rows resolved once by pdllm_resolve_rows for this pool
 *                      and page table (bf16 pools only).  The selection is static over the
 *                      denoising steps of a prompt (Methodology 3), so a
 *                      caller resolves it once and every decode call reads one
 *                      entry per row instead of the chunk_slot / sel_chunk /
 *                      keep_rows chain (which may then be NULL)
 * A selected chunk contributes its BOS row and its b kept rows (less the
 * absent ones), in that order; chunks are visited in sel_chunk order.
 */
typedef struct {
  const int32_t* chunk_slot;
  const int32_t* sel_chunk;
  const int32_t* keep_rows;
  const int32_t* k_per_seq;
  int32_t n_chunks_per_seq;
  int32_t k_max;
  int32_t b;
  int32_t rows_compacted;
  const int32_t* rows;
} pdllm_page_table;

/* ------------------------------------------------------------------------ *
 * Prefill side                                                              *
 * ------------------------------------------------------------------------ */

/* Bytes of workspace pdllm_chunk_prefill_score needs for the same n_chunks,
 * h_q, h_kv (the pool's), slot_rows (the pool's) and w (0 when the arguments
 * are invalid).  Pure host function. */
size_t pdllm_prefill_score_workspace(int32_t n_chunks, int32_t h_q, int32_t h_kv, int32_t slot_rows,
                                     int32_t w);

/*
 * Chunk-local bidirectional attention with fused per-key scoring
 * (Methodology 1: each chunk, BOS first, is processed on its own with
 * bidirectional attention inside the chunk; Methodology 2: a chunk's tokens
 * are ranked by the cumulative bidirectional attention weight they receive
 * from the query tokens).
 *
 *   q_chunk    device [n_chunks][slot_rows][h_q][d]  the chunk rows' queries
 *   q_win      device [n_chunks / chunks_per_win][w][h_q][d]  query windows;
 *              chunk c is scored by window c / chunks_per_win
 *   o_chunk    device [n_chunks][slot_rows][h_q][d]  (pool dtype) out:
 *              o[c,r,h] = sum_j softmax_j(scale <q_chunk[c,r,h], K[s,j,g]>) V[s,j,g]
 *              with s = chunk_slot[c], g = h / G, j over the slot's rows
 *   key_score  device [n_chunks][slot_rows] float out:
 *              key_score[c,j] = sum_h sum_w softmax_j(scale <q_win[.,w,h], K[s,j,g]>)
 *              (the window rows' softmax runs over the chunk's own rows only)
 *   chunk_slot device [n_chunks]
 *   chunk_rows device [n_chunks], nullable: rows R_c (1..slot_rows, BOS
 *              included) that chunk c holds at the start of its slot; NULL =
 *              slot_rows for every chunk.  A prefix whose length is not a
 *              multiple of C ends in a partial chunk of fewer rows: its keys
 *              j >= R_c take no part (key_score[c,j] = 0) and its output rows
 *              r >= R_c are not written.
 *   workspace  device, >= pdllm_prefill_score_workspace(n_chunks, h_q, h_kv, slot_rows, w),
 *              16-byte aligned
 * Supported: slot_rows <= 4097 (chunk sizes up to 4096 plus BOS); f32 with d
 * in {16, 32, 64, 128}; bf16 with d in {64, 128}.  For bf16, a chunk of up
 * to 288 rows is held on chip in one pass; longer chunks stream their K and
 * V through on-chip tiles, and their window rows make a second pass (their
 * softmax normalisers first, then the per-key weights) -- the same results.
 * The per-key sums are reduced in a fixed order: results are bitwise
 * reproducible run to run.
 */
pdllm_status pdllm_chunk_prefill_score(const pdllm_pool* pool, const int32_t* chunk_slot,
                                       const int32_t* chunk_rows, int32_t n_chunks,
                                       const void* q_chunk, int32_t h_q,
                                       const void* q_win, int32_t w, int32_t chunks_per_win,
                                       float scale, void* o_chunk, float* key_score,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-B rows per chunk (Methodology 2, intra-chunk sparsity).
 *   key_score  device [n_chunks][slot_rows] float
 *   chunk_rows device [n_chunks], nullable: rows R_c each chunk holds (see
 *              pdllm_chunk_prefill_score); NULL = slot_rows
 *   keep_rows  device [n_chunks][b] int32 out: the b best rows among the
 *              content rows 1..R_c-1 (row 0, the BOS anchor, is always kept
 *              and is not a candidate), in ascending order.  A chunk with
 *              fewer than b content rows keeps them all and fills the rest of
 *              its row with -1 (absent).
 * Order: larger score first; equal scores (-0 == +0) go to the lower row;
 * NaN ranks after every number.  0 <= b <= slot_rows - 1, slot_rows <= 4097.
 * Bit-exact: integer comparisons only.
 */
pdllm_status pdllm_select_topB(const float* key_score, const int32_t* chunk_rows, int32_t n_chunks,
                               int32_t slot_rows, int32_t b, int32_t* keep_rows, void* stream);

/*
 * Top-K chunks per sequence over given chunk scores (Methodology 1,
 * selection of the K most relevant chunks by s; Methodology 2, inter-chunk
 * sparsity).  Producing s itself needs the language model and is not part of
 * this library.
 *   chunk_score device [n_seq][n_chunks] float
 *   k_per_seq   host   [n_seq]  0 <= K_s <= k_max <= n_chunks
 *   sel_chunk   device [n_seq][k_max] int32 out: the K_s best chunk ids in
 *               ascending order, then -1 up to k_max.
 * Same order and ties as pdllm_select_topB.  1 <= n_chunks <= 8192
 * (PDLLM_ERR_UNSUPPORTED above).
 */
pdllm_status pdllm_select_topK(const float* chunk_score, int32_t n_seq, int32_t n_chunks,
                               const int32_t* k_per_seq, int32_t k_max, int32_t* sel_chunk,
                               void* stream);

/*
 * Compacted kept-row cache (Methodology 2: after the intra-chunk selection
 * only the top-B tokens of a chunk stay in the KV cache).  Chunk c, held in
 * slot s = chunk_slot[c] of the source pool, is written to slot s of the
 * destination: its BOS row first, then its b kept rows in keep_rows order,
 *   dst[s][0] = src[s][0],   dst[s][1 + i] = src[s][keep_rows[c][i]],
 * for every KV head, in K and in V.  The copy is bit-exact; destination rows
 * past b, rows of absent (-1) entries and slots of no listed chunk are not
 * written.  A decode over the destination with rows_compacted = 1 and the
 * same b (and keep_rows, when it has absent entries) attends exactly the
 * rows a decode over the source with keep_rows attends, in the same order.
 *   src        the whole-chunk pool
 *   chunk_slot device [n_chunks]
 *   keep_rows  device [n_chunks][b] rows in 1..src->slot_rows-1 or -1 (as
 *              written by pdllm_select_topB); may be NULL when b = 0
 *   dst_k, dst_v  device, the source's dtype, h_kv, d and n_slots, with
 *              dst_slot_rows >= b + 1 rows per slot and element strides
 *              dst_stride_slot, dst_stride_row, dst_stride_head (d contiguous;
 *              the same rules as a pdllm_pool's); must not overlap the source
 * Supported: every dtype and d a pdllm_pool supports; 0 <= b <= slot_rows - 1.
 */
pdllm_status pdllm_compact_kept_rows(const pdllm_pool* src, const int32_t* chunk_slot, int32_t n_chunks,
                                     const int32_t* keep_rows, int32_t b, void* dst_k, void* dst_v,
                                     int64_t dst_stride_slot, int64_t dst_stride_row,
                                     int64_t dst_stride_head, int32_t dst_slot_rows, void* stream);

/*
 * Gather-to-contiguous of a decode's attended pool rows: the copy that the
 * split decode avoids by reading the non-contiguous pool in place
 * ("Attention kernel optimization"), provided as the comparator that times
 * it.  For sequence s and its k-th selected chunk c = sel_chunk[s][k]
 * (k < K_s), in slot chunk_slot[s N + c], destination slot u = s k_max + k
 * gets the chunk's BOS row, then its b kept rows in keep_rows order --
 * exactly the rows, and the order, in which the decode attends them:
 *   dst[u][0] = src[slot][0],   dst[u][1 + i] = src[slot][keep_rows[s N + c][i]].
 * With dst_stride_slot = (b + 1) dst_stride_row, sequence s's K_s (b + 1) rows
 * are one contiguous run starting at slot s k_max.  A decode over that run
 * (one compacted chunk of K_s (b + 1) rows per sequence) attends the same
 * rows in the same order.  Slots past K_s and rows of absent (-1) entries are
 * not written.
 *   pool, pt   as pdllm_split_attn_decode (pt->rows_compacted must be 0)
 *   dst_k, dst_v  device, [n_seq k_max][b + 1][h_kv][d] with the given
 *              element strides (the rules of a pdllm_pool's), the pool's dtype
 * Supported: n_seq <= 64.
 */
pdllm_status pdllm_gather_kept_kv(const pdllm_pool* pool, const pdllm_page_table* pt, int32_t n_seq, void* dst_k,
                                  void* dst_v, int64_t dst_stride_slot, int64_t dst_stride_row,
                                  int64_t dst_stride_head, void* stream);

/*
 * The prefill side in one call: pdllm_chunk_prefill_score, then
 * pdllm_select_topB over its key scores, and pdllm_select_topK over the given
 * chunk scores, with the same outputs bit for bit.  The key-score finalize and
 * both selections share one launch after the attention kernels, so the call
 * pays one kernel boundary where the three calls pay three.
 *   pool .. workspace   as pdllm_chunk_prefill_score (the same workspace size)
 *   b, keep_rows        as pdllm_select_topB (slot_rows = pool->slot_rows,
 *                       chunk_rows as given); keep_rows may be NULL when b = 0
 *   chunk_score, n_seq, k_per_seq, k_max, sel_chunk
 *                       as pdllm_select_topK, with n_chunks / n_seq chunks
 *                       per sequence (n_seq must divide n_chunks); chunk_score,
 *                       k_per_seq and sel_chunk may be NULL when k_max = 0
 *   selected_only       0: every chunk is scored and gets its top-B rows.
 *                       1: only the chunks top-K selects (Methodology 2 keeps
 *                       top-B rows inside the K kept chunks): the scoring
 *                       window runs on those chunks only, and key_score and
 *                       keep_rows are written for them only, with the same
 *                       values as with 0; o_chunk is written for every chunk
 *                       either way.  Needs chunk_score.  With more than 64
 *                       sequences every chunk is scored.
 */
pdllm_status pdllm_prefill_select(const pdllm_pool* pool, const int32_t* chunk_slot, const int32_t* chunk_rows,
                                  int32_t n_chunks, const void* q_chunk, int32_t h_q, const void* q_win, int32_t w,
                                  int32_t chunks_per_win, float scale, void* o_chunk, float* key_score, int32_t b,
                                  int32_t* keep_rows, const float* chunk_score, int32_t n_seq,
                                  const int32_t* k_per_seq, int32_t k_max, int32_t* sel_chunk,
                                  int32_t selected_only, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace pdllm_chunk_score needs (0 when the arguments are
 * invalid).  Pure host function. */
size_t pdllm_chunk_score_workspace(int32_t n_chunks, int32_t n_query, int32_t n_pseudo);

/*
 * Predictive chunk scores from the model's logits (Methodology 1, predictive
 * scoring: each chunk is scored by the negative log-likelihood of the query
 * window given the chunk, s_I, and by the likelihood of the pseudo-labels
 * given the chunk and the query, s_P -- read as a log-likelihood -- and the
 * top-K chunks by s = s_I + s_P are selected; its output feeds
 * pdllm_select_topK).  For each scored row r, with z the row's logits:
 *   log p[r] = z[target[r]] - ln sum_v exp(z[v])
 *
 *   logits     device, row r = c (n_query + n_pseudo) + t at logits + r row_stride
 *              (elements of dtype PDLLM_F32 or PDLLM_BF16), vocab logits per row;
 *              16-byte aligned, row_stride * element size a multiple of 16 bytes.
 *              Rows t < n_query predict the chunk's query-window tokens, the
 *              next n_pseudo rows its pseudo-label tokens.  Logits are finite
 *              or -inf; a row of all -inf has no defined result.
 *   target     device [n_chunks][n_query + n_pseudo] int32 token ids; ids
 *              outside [0, vocab) are clamped into it
 *   s_i        device [n_chunks] float out, nullable: -sum_{t < n_query} log p
 *   s_p        device [n_chunks] float out, nullable: sum_{t >= n_query} log p
 *   s          device [n_chunks] float out: s_i + s_p
 *   workspace  device, >= pdllm_chunk_score_workspace(n_chunks, n_query, n_pseudo)
 *              (the per-row log-probabilities)
 * Each row's sum over the vocabulary and each chunk's sum over its rows are
 * taken in a fixed order: results are bitwise reproducible run to run.
 */
pdllm_status pdllm_chunk_score(const void* logits, int32_t dtype, int64_t row_stride, int32_t vocab,
                               const int32_t* target, int32_t n_chunks, int32_t n_query, int32_t n_pseudo,
                               float* s_i, float* s_p, float* s, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------ *
 * Decode side                                                               *
 * ------------------------------------------------------------------------ */

/*
 * The attended pool rows of a page table, resolved once (Methodology 2 and
 * 3: the top-K chunks and their top-B rows stay fixed over the denoising
 * steps of a prompt).  Entry rows[s * k_max (b + 1) + k (b + 1) + r] is the
 * element offset / 8 of row r (0 = BOS, then the kept rows) of the k-th
 * selected chunk of sequence s in the pool -- slot * stride_slot +
 * row * stride_row, without the kv head's offset -- with bit 31 set for an
 * absent kept row (which points at the BOS row); entries of chunks k >= K_s
 * are written from the clamped sel_chunk entries and never read.  Pass the
 * array as pdllm_page_table.rows to the decode calls over the same pool and
 * page table.
 *   pool, pt       as for pdllm_split_attn_decode (pt->rows is ignored)
 *   rows           device [n_seq][k_max (b + 1)] int32 out, 4-byte aligned;
 *                  rows_elems its length in elements
 * Errors: PDLLM_ERR_INVALID_ARG for what pdllm_split_attn_decode rejects in
 * the pool and page table, a NULL or short rows; PDLLM_ERR_UNSUPPORTED for a
 * float32 pool or a pool of 2^34 elements or more (bf16 strides are
 * multiples of 8 elements, so offset / 8 is exact).  Nothing is enqueued on
 * error.
 */
pdllm_status pdllm_resolve_rows(const pdllm_pool* pool, const pdllm_page_table* pt, int32_t n_seq,
                                int32_t* rows, size_t rows_elems, void* stream);

/*
 * The split plan of a decode call (host only, deterministic).  The attended
 * rows of sequence s, N_s = K_s (b + 1) + l_d, are cut into kv tiles; a
 * split is a run of consecutive tiles.  num_splits = 0 lets the planner pick
 * the split count from the work and n_cu (the device's compute units);
 * num_splits > 0 forces that many splits per sequence (capped at the
 * sequence's tile count).  For bf16 with num_splits = 0 the planner may
 * choose the decode without kv splits (q_rows_per_wg = 32: one workgroup per
 * 32 query rows over every kv row of the sequence, no partials, no
 * workspace) when a cost model measured on MI355X rates it faster, which
 * happens when each sequence attends few kv rows.
 *   splits_per_seq  host [n_seq] out   tiles_per_split host [n_seq] out
 *   q_rows_per_wg   host out: query rows (token x grouped head) per workgroup
 *   workspace_bytes host out: the workspace the call needs
 * Any output pointer may be NULL.
 */
pdllm_status pdllm_decode_plan(const int32_t* k_per_seq, int32_t n_seq, int32_t b, int32_t l_d,
                               int32_t h_q, int32_t h_kv, int32_t d, int32_t dtype,
                               int32_t num_splits, int32_t n_cu, int32_t* splits_per_seq,
                               int32_t* tiles_per_split, int32_t* q_rows_per_wg,
                               int64_t* workspace_bytes);

/* Bytes of workspace pdllm_split_attn_decode needs on the current device
 * (0 when the arguments are invalid).  Host function; queries the device's
 * compute-unit count once (256 is assumed when no device is visible). */
size_t pdllm_split_attn_decode_workspace(const pdllm_pool* pool, const pdllm_page_table* pt,
                                         int32_t n_seq, int32_t l_d, int32_t h_q,
                                         int32_t num_splits);

/*
 * Split-KV chunk-sparse decode attention with log-sum-exp merge
 * (Methodology 3: the static cached rows of the selected chunks plus the
 * freshly recomputed query/response rows are attended by every decode row,
 * with no mask; "Attention kernel optimization": the KV dimension is split,
 * each split is processed independently straight from the non-contiguous
 * pool, and the splits are merged by a log-sum-exp reduction).
 *
 *   q        device [n_seq][l_d][h_q][d]
 *   k_resp   device [n_seq][l_d][h_kv][d]   (pool dtype)
 *   v_resp   device [n_seq][l_d][h_kv][d]
 *   o        device [n_seq][l_d][h_q][d] out (pool dtype):
 *            o[s,i,h] = sum_a softmax_a(scale <q[s,i,h], k_a[g]>) v_a[g] over
 *            the attended rows a of sequence s (see pdllm_page_table) followed
 *            by its l_d response rows
 *   lse      device [n_seq][h_q][l_d] float out, nullable: natural-log
 *            normaliser ln sum_a exp(scale <q, k_a>)
 *   workspace device, >= pdllm_split_attn_decode_workspace(...) for the same
 *            arguments, 16-byte aligned: the per-split partial outputs (each
 *            normalised by its own softmax sum) and their float32
 *            log-sum-exps.  When the splits are merged inside the decode
 *            launch (pdllm_decode_opts.merge 2 or 3), the workspace begins
 *            with synchronisation words that must be zero when a workspace is
 *            first used -- zero-fill a new workspace once -- and that every
 *            call returns to zero; keep such a workspace for decode calls, and
 *            give calls that may overlap (other streams) workspaces of their
 *            own.
 * The result does not depend on num_splits beyond rounding: with bf16 inputs
 * the partials are rounded once to bf16 before the merge (float32 with merge
 * 2 or 4), with f32 inputs they are float32.
 * Supported: f32 with d in {16, 32, 64, 128}; bf16 with d in {64, 128}.
 */
pdllm_status pdllm_split_attn_decode(const pdllm_pool* pool, const pdllm_page_table* pt,
                                     const void* q, const void* k_resp, const void* v_resp,
                                     int32_t n_seq, int32_t l_d, int32_t h_q, float scale,
                                     int32_t num_splits, void* o, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Options of a decode call.  Zero-initialise the struct: every field's 0 is
 * the library's choice.
 *   num_splits     as pdllm_split_attn_decode's (0 = planner)
 *   q_rows_per_wg  0 = planner; otherwise the query rows (token x grouped
 *                  head) of one workgroup, a shape of the dtype's kernel:
 *                  128 or 256 for bf16, 64 for f32 (PDLLM_ERR_UNSUPPORTED
 *                  for any other).  32 (bf16) selects the decode without kv
 *                  splits: num_splits must be 0 or 1 and merge 0 or 1, each
 *                  sequence may attend at most 4864 pool rows (K_s (b + 1)),
 *                  and the pool and the response rows must each span under
 *                  4 GiB; otherwise PDLLM_ERR_INVALID_ARG.  It needs
 *                  no workspace.  The result does not depend on the shape
 *                  beyond rounding; tests use it to run every kernel
 *                  instance.
 *   merge          how the splits are merged: 0 = the library's choice
 *                  (1); 1 = a second kernel launch over partials stored in
 *                  the pool dtype; 2 / 3 = inside the decode launch, over
 *                  float32 / bf16 partials exchanged through the L2 of one
 *                  XCD (bf16 inputs only, PDLLM_ERR_UNSUPPORTED for f32);
 *                  4 = a second kernel launch over float32 partials (for
 *                  bf16 inputs the output is then rounded once, at the
 *                  merge; twice the workspace of 1; for f32 inputs the same
 *                  as 1).  With 2 and 3 the workspace holds synchronisation
 *                  words, see pdllm_split_attn_decode.  Other values:
 *                  PDLLM_ERR_INVALID_ARG.
 */
typedef struct {
  int32_t num_splits;
  int32_t q_rows_per_wg;
  int32_t merge;
  int32_t reserved[5];              /* must be 0 */
} pdllm_decode_opts;

/* pdllm_split_attn_decode_workspace with options (0 when invalid). */
size_t pdllm_split_attn_decode_ex_workspace(const pdllm_pool* pool, const pdllm_page_table* pt,
                                            int32_t n_seq, int32_t l_d, int32_t h_q,
                                            const pdllm_decode_opts* opts);

/* pdllm_split_attn_decode with options (same operation, arguments and
 * errors; opts must not be NULL).  pdllm_split_attn_decode(..., num_splits,
 * ...) is this call with opts = {num_splits, 0}. */
pdllm_status pdllm_split_attn_decode_ex(const pdllm_pool* pool, const pdllm_page_table* pt,
                                        const void* q, const void* k_resp, const void* v_resp,
                                        int32_t n_seq, int32_t l_d, int32_t h_q, float scale,
                                        const pdllm_decode_opts* opts, void* o, float* lse,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * pdllm_split_attn_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments and errors, with num_splits as
 * there, but no workspace argument.  The split partials live in a scratch
 * array the library holds on each GPU (64 MiB, PDLLM_NOALLOC_SCRATCH_BYTES,
 * held until the process ends); the call itself allocates nothing, and the
 * caller still provides q, k_resp, v_resp, o and lse.  A call whose plan needs
 * more scratch than that returns PDLLM_ERR_UNSUPPORTED before enqueueing
 * anything (pdllm_split_attn_decode_workspace gives the need).  Every call on
 * one GPU shares its scratch: calls that overlap on one GPU (different
 * streams, or host threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe.
 */
#define PDLLM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pdllm_status pdllm_split_attn_decode_noalloc(const pdllm_pool* pool, const pdllm_page_table* pt,
                                             const void* q, const void* k_resp, const void* v_resp,
                                             int32_t n_seq, int32_t l_d, int32_t h_q, float scale,
                                             int32_t num_splits, void* o, float* lse, void* stream);

/* ------------------------------------------------------------------------ */

/* Message of the calling thread's last non-OK status ("" if none). */
const char* pdllm_last_error(void);

/* PDLLM_ABI_VERSION of the loaded library. */
int pdllm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PDLLM_H */
