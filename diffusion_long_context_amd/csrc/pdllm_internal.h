// Internal declarations shared by the C-ABI layer and the HIP kernels of
// libpdllm.  Not part of the public interface (include/pdllm.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace pdllm {

// ---------------------------------------------------------------- planning
// kv rows per tile of the split-KV decode; a split is a run of whole tiles
constexpr int kDecodeTile = 64;
// query rows (token x grouped head) handled by one decode workgroup: the bf16
// kernel runs 4 or 8 wavefronts of 32 rows, the planner picks per call
constexpr int kDecodeRowsBf16Small = 128;
constexpr int kDecodeRowsBf16Large = 256;
// bf16 decode without kv splits (decode_ws.hip): 32 query rows per
// workgroup, every kv row of the sequence, pool rows through an LDS row table
// of at most kWsMaxPoolRows entries.
constexpr int kDecodeRowsBf16Ws = 32;
constexpr int kWsMaxPoolRows = 4864;
constexpr int kDecodeRowsF32 = 64;
// sequences whose per-sequence plan travels in one launch's arguments (the
// argument block is then about 2.7 KB); a batch of small-window decodes
// gathers its K/V in one launch, with no split merge, up to this many
constexpr int kMaxSeqPerLaunch = 64;

struct DecodePlan {
  int n_seq = 0;
  int q_rows_per_wg = 0;   // query rows per workgroup
  int q_tiles = 0;         // workgroups along the query rows of one (seq, kv head)
  std::vector<int> k_s, n_kv, n_tiles, splits, tiles_per_split;
  std::vector<int64_t> part_off, lse_off;   // element offsets into the partial regions
  int64_t part_floats = 0, lse_floats = 0;  // element counts (partial O, partial lse)
  int part_elem_bytes = 4;                  // partial O element: bf16 (2) or float32 (4)
  // In-kernel merge (bf16): the splits of a group merge their float32
  // partials in the decode launch itself, synchronised through int32 words at
  // the start of the workspace (started, exited, then per group one arrival
  // count and one claim count per 32-row slice).
  bool fused = false;
  bool fused_bf16 = false;                  // in-kernel merge over bf16 (else float32) partials
  bool sep_f32 = false;                     // bf16 inputs, separate merge kernel over float32 partials
  bool ws = false;                          // bf16 decode without splits (decode_ws.hip)
  int64_t sync_words = 0;
  int64_t sync_bytes = 0;                   // 256-aligned; the partials follow
  int64_t workspace_bytes = 0;
  int64_t total_workgroups = 0;
};

// Fills `plan`; returns false (with a message in *err) on invalid input.
// force_rows > 0 fixes the query rows per workgroup (a shape of the dtype's
// kernel, checked by the caller); 0 lets the planner choose.
// merge: 0 = the library's choice (1), 1 = a separate merge kernel over
// partials in the input dtype, 2 / 3 = in-kernel over float32 / bf16
// partials (bf16 only; the caller checked), 4 = a separate merge kernel over
// float32 partials (the same as 1 for float32 inputs).
bool plan_decode(const int32_t* k_per_seq, int n_seq, int b, int l_d, int h_q, int h_kv,
                 int d, int dtype, int num_splits, int force_rows, int merge, int n_cu, DecodePlan* plan,
                 const char** err, bool ws_allowed = true);

// ---------------------------------------------------------------- scratch
// Bytes of the library-held device scratch of the no-allocation decode entry
// point (one copy per GPU, held until the process ends).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of the current device's scratch (looked up once per
// device); returns a hipError_t value as int.
int noalloc_scratch(void** ptr);

// ---------------------------------------------------------------- decode
// Workgroup b runs on XCD b % kXcdGroups (dispatch is round-robin over the
// XCDs; with fewer XCDs per device, b % 8 still implies the same XCD).
constexpr int kXcdGroups = 8;
// Contiguous partition of `sizes` (workgroups per merge group, in order) into
// kXcdGroups ranges with the smallest largest sum; bounds[x] .. bounds[x + 1]
// is range x.  Returns that largest sum.
int64_t xcd_partition(const std::vector<int>& sizes, int32_t* bounds);

struct DecodeSeq {
  int32_t k_s;              // selected chunks of this sequence
  int32_t n_kv;             // attended rows: k_s * (b + 1) + l_d
  int32_t n_splits;
  int32_t tiles_per_split;
  int32_t wg_begin;         // first workgroup of this sequence in the launch
  int32_t grp_begin;        // first merge group (kv head, query tile) of this sequence in the launch
  int64_t part_off;         // element offset of its partial outputs
  int64_t lse_off;          // float offset of its partial lse values
};

struct DecodeArgs {
  const void* pool_k;
  const void* pool_v;
  int64_t ps_slot, ps_row, ps_head;   // pool strides (elements)
  const int32_t* chunk_slot;
  const int32_t* sel_chunk;
  const int32_t* keep_rows;
  const int32_t* idx_dummy;  // valid device memory read in place of absent index tables
  const int32_t* rows;       // nullable: the resolved pool rows (pdllm_resolve_rows), [n_seq][rows_stride]
  int64_t rows_stride;       // k_max (b + 1)
  const void* q;
  const void* k_resp;
  const void* v_resp;
  void* o;
  float* lse;
  void* part_o;             // partial outputs: bf16 (separate merge) or float32
  float* part_lse;
  int32_t* sync;            // in-kernel merge: sync words (nullptr: separate merge kernel)
  int32_t n_groups;         // merge groups of this launch
  int32_t merge_kind;       // bf16 kernel: 0 / 3 separate merge over bf16 / float32 partials,
                            // 1 / 2 in-kernel over float32 / bf16 partials
  int32_t grid_wg;          // workgroups launched (in-kernel merge: 8 x the largest XCD share)
  int32_t xcd_grp[kXcdGroups + 1];   // in-kernel merge: XCD x runs groups [xcd_grp[x], xcd_grp[x + 1])
  int32_t n_chunks_per_seq, k_max, b;
  int32_t compact;          // 1: a chunk's kept rows are rows 1..b of its slot (keep_rows unused)
  int32_t l_d, h_q, h_kv, group;
  int32_t q_tiles;
  int32_t seq0;             // first sequence of this launch
  int32_t n_seq_launch;
  int32_t total_wg;
  float scale_log2;         // softmax scale * log2(e)
  DecodeSeq seq[kMaxSeqPerLaunch];
};

// Launchers (return a hipError_t value as int).
int launch_decode_bf16(const DecodeArgs& a, int d, int q_rows_per_wg, void* stream);
int launch_decode_f32(const DecodeArgs& a, int d, void* stream);
int launch_decode_ws(const DecodeArgs& a, int d, void* stream);
// pdllm_resolve_rows (resolve_rows.hip)
struct ResolveArgs {
  const int32_t* chunk_slot;
  const int32_t* sel_chunk;
  const int32_t* keep_rows;  // nullable (b = 0, or compacted slots without absent rows)
  int32_t* rows;
  int64_t ps_slot, ps_row;
  int32_t n_seq, n_chunks_per_seq, k_max, b, compact;
};
int launch_resolve_rows(const ResolveArgs& a, void* stream);
// bf16_part: the partials are bf16 (else float32); bf16_out: so is o.
int launch_lse_merge(const DecodeArgs& a, int d, bool bf16_part, bool bf16_out, void* stream);

// ---------------------------------------------------------------- prefill
constexpr int kMaxSelSeq = 64;           // sequences whose K_s a prefill launch carries
// Chunks per sequence up to which the resident prefill kernel can take
// chunks in score order (ranks counted directly in LDS).
constexpr int kPrefillRankChunks = 256;
struct PrefillArgs {
  const void* pool_k;
  const void* pool_v;
  int64_t ps_slot, ps_row, ps_head;
  const int32_t* chunk_slot;
  const int32_t* chunk_rows; // nullable [n_chunks]: rows held by each chunk (default slot_rows)
  const void* q_chunk;
  const void* q_win;
  void* o_chunk;
  float* key_score;
  float* part_score;        // workspace [n_chunks][h_kv][parts][slot_rows]
  float* win_norm;          // streaming path: workspace [n_chunks][h_kv][w * group padded to 32]
  int32_t n_chunks, slot_rows, h_q, h_kv, group, w, chunks_per_win;
  int32_t parts;            // partial key-score rows per (chunk, kv head)
  float scale_log2;
  // Scoring only the chunks top-K selects (sel_score != nullptr): chunk c,
  // chunk c % sel_per_seq of sequence c / sel_per_seq, is scored iff it is
  // among the sel_k[sequence] best of its sequence's row of sel_score.
  const float* sel_score;   // [n_seq][sel_per_seq] or nullptr (score every chunk)
  int32_t sel_per_seq;
  int32_t sel_k[kMaxSelSeq];
  // With sel_score: workgroups take chunks in descending score order (the
  // resident bf16 kernel), so that the scored chunks run first.  Set when
  // the scored workgroups fit in one round on the device and the launch has
  // more than one round (then no CU draws two scored chunks), and the
  // sequences have at most kPrefillRankChunks chunks.
  int32_t rank_order;
};


// partial key-score rows per (chunk, kv head): one per wavefront of the bf16
// kernel, one for the f32 kernel; the workspace is sized for the larger
constexpr int kPrefillParts = 8;
int launch_prefill_bf16(const PrefillArgs& a, int d, void* stream);
int launch_prefill_f32(const PrefillArgs& a, int d, void* stream);
// bf16 chunks longer than the on-chip limit (kPrefillMaxRows), streamed
int launch_prefill_stream(const PrefillArgs& a, int d, void* stream);
constexpr int kPrefillMaxRows = 288;     // bf16 rows the resident kernel holds in LDS
int launch_score_finalize(const PrefillArgs& a, void* stream);

// ---------------------------------------------------------------- select
int launch_select_topb(const float* key_score, const int32_t* chunk_rows, int n_chunks, int slot_rows,
                       int b, int32_t* keep_rows, void* stream);
constexpr int kMaxTopkSeqPerLaunch = 64;
struct TopkArgs {
  const float* chunk_score;
  int32_t* sel_chunk;
  int32_t n_chunks, k_max, seq0, n_seq_launch;
  int32_t k[kMaxTopkSeqPerLaunch];
};
int launch_select_topk(const TopkArgs& a, void* stream);

// Score finalize fused with both selections (one launch): workgroup c <
// n_chunks adds chunk c's key-score partials (the order of the finalize
// kernel) and selects its top-B rows; the next topk.n_seq_launch workgroups
// select the top-K chunks of one sequence each.
struct FinalizeSelectArgs {
  const float* part;        // [n_chunks][h_kv][parts][slot_rows]
  float* key_score;         // [n_chunks][slot_rows] out
  const int32_t* chunk_rows;   // nullable
  int32_t* keep_rows;       // [n_chunks][b] out
  int32_t n_chunks, h_kv, parts, slot_rows, b;
  int32_t selected_only;    // 1: only chunks top-K selects (topk holds every sequence) are finalized
  TopkArgs topk;            // n_seq_launch = 0: no top-K work
};
int launch_finalize_select(const FinalizeSelectArgs& a, void* stream);

// ---------------------------------------------------------------- chunk scores
struct ChunkScoreArgs {
  const void* logits;       // [n_chunks][n_query + n_pseudo] rows of `vocab` logits
  int64_t row_stride;       // elements between rows
  const int32_t* target;    // [n_chunks][n_query + n_pseudo]
  float* logp;              // workspace [n_chunks][n_query + n_pseudo]
  float* s_i;               // nullable
  float* s_p;               // nullable
  float* s;
  int32_t vocab, n_chunks, n_query, n_pseudo;
  bool bf16;
};
int launch_chunk_score(const ChunkScoreArgs& a, void* stream);

// ---------------------------------------------------------------- kept-row compaction
constexpr int kMaxGatherSeq = 64;        // sequences one gather launch carries
struct CompactArgs {
  const char* src_k;
  const char* src_v;
  char* dst_k;
  char* dst_v;
  int64_t ss, sr, sh;       // source slot / row / head strides (bytes)
  int64_t ds, dr, dh;       // destination strides (bytes)
  const int32_t* chunk_slot;
  const int32_t* keep_rows; // [n_chunks][b]
  int32_t n_chunks, b, h_kv;
  int32_t nvec;             // 16-byte vectors per (row, head)
  int32_t blocks;           // workgroups per (chunk, tensor)
  // gather (sel_chunk set): n_chunks = n_seq * k_max units, unit s k_max + k
  // copies selected chunk sel_chunk[unit] of sequence s (if k < k_s[s]) to slot unit
  const int32_t* sel_chunk;
  int32_t k_max, n_chunks_per_seq;
  int32_t k_s[kMaxGatherSeq];
};

constexpr int kCompactThreads = 256;
constexpr int kCompactVec = 4;           // 16-byte vectors per thread
int launch_compact(const CompactArgs& a, void* stream);

}  // namespace pdllm
