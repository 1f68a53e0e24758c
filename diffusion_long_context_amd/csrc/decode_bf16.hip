// Split-KV chunk-sparse decode attention for bf16 inputs on gfx950 (MFMA).
//
// What it computes (Prefilling-dLLM summary, Methodology 2 and 3, and
// "Attention kernel optimization"): every decode row (token i, query head h)
// of a sequence attends, without a mask, to the BOS row and the kept rows of
// each selected chunk -- read in place from the non-contiguous chunk pool --
// followed by the sequence's recomputed response rows.  The kv rows are split
// into runs of 64-row tiles; each workgroup handles one (sequence, kv head,
// 128 or 256 query rows, split) and emits either the final output (single
// split) or a partial output (normalised) and its float32 log-sum-exp.  The
// splits are merged either inside this launch, by the splits themselves
// (merge_group), or by a second kernel (lse_merge_kernel).
//
// Design for CDNA4:
// * Query rows of one kv head are packed as (token, grouped head) pairs, so
//   the G = h_q / h_kv heads sharing a kv head make the contraction dense.
// * Each wavefront owns 32 query rows; S^T = K Q^T and O^T += V^T P^T run on
//   v_mfma_f32_32x32x16_bf16 (attn_tile.h).  Computing S transposed leaves
//   each lane with the probabilities of one query column, which feed the PV
//   product as its B operand directly (no shuffle through LDS).
// * K/V tiles are gathered straight from pool slots into LDS through a
//   per-workgroup row-pointer table (no gather-to-contiguous copy); K and V
//   are stored row-major and the PV A operand is read with gfx950's
//   transposing LDS load (ds_read_b64_tr_b16).  Tiles are
//   double-buffered in LDS (one barrier per tile); the global loads of tiles
//   t+2 and t+3 are in flight (in staging registers) while tile t computes.
// * Online softmax in base 2: the scale and log2(e) fold into one FMA before
//   v_exp_f32 and the running max moves lazily (see kRescaleLog2).
#include "attn_tile.h"
#include "device_common.h"
#include "pdllm_internal.h"
#include "xwg_sync.h"

namespace pdllm {
namespace {

constexpr int kTile = kDecodeTile;         // kv rows per tile
// Polls of a group's arrival count before a waiting split gives up its merge
// slices to the group's last arrival (about 20 ms).
constexpr int kSpinLimit = 1 << 14;

// Roles of a wavefront in the tile loop (see the kernel).
constexpr int kRunAll = 0, kRunIdle = 1, kRunCons = 2, kRunProd = 3;
constexpr int kProdStages = 3;             // staging sets of the loader wavefronts


// LDS of one workgroup.  The 8-wave variant (one workgroup per CU) uses the
// V pitch that keeps the transposing reads conflict-free on the 64-bank LDS
// (4 rows x 64 B per 32 lanes) and an 8-tile row table; the 4-wave variant
// stays under half of the 160 KiB so two workgroups share a CU.
template <int D, int WAVES>
struct Smem {
  static constexpr int KP = D + 8;         // K pitch (elements): 8-row 16-byte reads conflict-free
  static constexpr int VP = WAVES == 8 ? D + 32 : D + 16;   // V pitch (elements)
  static constexpr int kTableTiles = WAVES == 8 ? 8 : 4;    // row-table capacity (tiles)
  uint16_t k[2][kTile * KP];               // double-buffered tiles, both row-major
  uint16_t v[2][kTile * VP];
  gptr16 kptr[kTableTiles * kTile];        // K / V address of each attended row
  gptr16 vptr[kTableTiles * kTile];
  uint64_t absent[kTableTiles];            // per table tile: bit r = row r is an absent kept row
  uint64_t kmask[2];                       // the absent mask of the tile in each K buffer
  int flag[WAVES];                         // per wavefront: the split holds an absent row
  int xw[4];                               // words broadcast by thread 0 (in-kernel merge)
  // The separate-merge epilogue's scalars, written by thread 0 before the
  // loop: reading them back here after the loop costs an LDS read, where
  // the argument segment would cost dependent scalar-cache misses.
  struct Epi {
    void* o;
    float* lse;
    void* part_o;
    float* part_lse;
    int64_t part_off, lse_off;
    int s, g, qt, split, n_splits, l_d, h_q, group;
  } epi;
};

// Element offset of attended row v of sequence s for kv head g.  Pool rows
// are >= 0 (relative to pool k/v); response rows are encoded as -1 - offset
// (relative to k_resp/v_resp).  Chunk k of the sequence contributes rows
// [k (b+1), (k+1)(b+1)): its BOS row 0, then its kept rows -- looked up in
// keep_rows, or rows 1..b of the slot when the pool holds compacted slots.
// A kept-row entry of -1 (a partial chunk with fewer than b content rows)
// is an absent row: `absent` is set and the offset is the chunk's BOS row
// (finite data; its score is masked).
template <int D>
__device__ __forceinline__ int64_t resolve_row(const DecodeArgs& a, int s, int g, int k_s,
                                               int v, bool& absent) {
  const int per = a.b + 1;
  absent = false;
  if (v < k_s * per && a.rows != nullptr) {   // resolved once (pdllm_resolve_rows)
    const int e = a.rows[(int64_t)s * a.rows_stride + v];
    absent = e < 0;
    return ((int64_t)(uint32_t)(e & 0x7fffffff) << 3) + (int64_t)g * a.ps_head;
  }
  if (v < k_s * per) {
    const int k = v / per;
    const int r = v - k * per;
    const int cg = s * a.n_chunks_per_seq + a.sel_chunk[(int64_t)s * a.k_max + k];
    const int slot = a.chunk_slot[cg];
    int row = 0;
    if (r) {
      const int kr = a.keep_rows != nullptr ? a.keep_rows[(int64_t)cg * a.b + r - 1] : r;
      absent = kr < 0;
      row = absent ? 0 : a.compact ? r : kr;
    }
    return (int64_t)slot * a.ps_slot + (int64_t)row * a.ps_row + (int64_t)g * a.ps_head;
  }
  const int j = v - k_s * per;
  return -1 - ((((int64_t)s * a.l_d + j) * a.h_kv + g) * D);
}

// The work item of a workgroup: (sequence, kv head, query tile, split).
// Separate merge: query tiles vary fastest, so the workgroups that share one
// (kv head, split) -- and therefore its K/V rows -- sit on one XCD and hit its
// L2.  In-kernel merge: every split of a merge group (sequence, kv head,
// query tile) runs on one XCD, so that the partials never leave its L2.
// Workgroups are dispatched round-robin over the XCDs, so workgroup b runs on
// XCD b % 8 (b % 4, b % 2 with fewer XCDs per device: the same grouping);
// XCD x takes the groups [xcd_grp[x], xcd_grp[x + 1]), its k-th workgroup the
// k-th split in that range, and workgroups past the range have no item.
struct WorkItem {
  int si, s, g, qt, split, n_splits, gi;
  bool valid;
};
template <bool FUSED, class A>
__device__ __forceinline__ WorkItem work_item(const A& a, int bid) {
  WorkItem w;
  int si = 0, local;
  w.valid = true;
  if constexpr (FUSED) {
    const int x = bid & 7, ge = a.xcd_grp[x + 1];
    int k = bid >> 3, gi = a.xcd_grp[x];
    w.valid = false;
    for (; gi < ge; ++gi) {
      while (si + 1 < a.n_seq_launch && gi >= a.seq[si + 1].grp_begin) ++si;
      if (k < a.seq[si].n_splits) {
        w.valid = true;
        break;
      }
      k -= a.seq[si].n_splits;
    }
    gi = min(gi, ge - 1);
    while (si + 1 < a.n_seq_launch && gi >= a.seq[si + 1].grp_begin) ++si;
    local = gi - a.seq[si].grp_begin;
    w.split = k;
    w.gi = gi;
    w.qt = local % a.q_tiles;
    w.g = local / a.q_tiles;
  } else {
    const int wg = xcd_remap(bid, a.total_wg);
    si = last_index_le(a.n_seq_launch, wg, [&](int i) { return a.seq[i].wg_begin; });
    local = wg - a.seq[si].wg_begin;
    w.qt = local % a.q_tiles;
    local /= a.q_tiles;
    w.split = local % a.seq[si].n_splits;
    w.g = local / a.seq[si].n_splits;
    w.gi = a.seq[si].grp_begin + w.g * a.q_tiles + w.qt;
  }
  w.si = si;
  w.s = a.seq0 + si;
  w.n_splits = a.seq[si].n_splits;
  return w;
}

// Layout of the in-kernel merge's partials, private to this file: the
// outputs of one (split, group) are WAVES blocks of 32 rows, one per
// wavefront, each stored as its lanes hold it -- chunk c = 4 db + m of lane l
// (d = 32 db + 8 m + 4 (l / 32) + t, t < 4, row l % 32) at (64 c + l) * 4
// elements -- so that every store instruction writes one contiguous run.
// Their lse values are [split][group][32 WAVES rows].
template <int D, int WAVES>
__device__ __forceinline__ int64_t fused_block(int64_t part_off, int h_kv, int q_tiles, int split, int gl, int wave) {
  return part_off + ((int64_t)(split * h_kv * q_tiles + gl) * WAVES + wave) * (32 * D);
}

// Merge slice x (the 32 rows of wavefront x) of a group over its splits.
// Work item k: row r = k % 32 and d-pair p = k / 32 (d = 8 p .. 8 p + 7: the
// four values of chunk p in lane r, then the four in lane 32 + r).
template <int D, int WAVES, bool PBF16, class A>
__device__ __forceinline__ void merge_slice(const A& a, int tid, int si, int s, int g, int qt, int x,
                                            int n_splits) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int P = D / 8;                 // d-pairs per row
  constexpr int KB = PBF16 ? 16 : 8;       // splits whose loads are in flight together
  constexpr uint32_t EB = PBF16 ? 2 : 4;   // bytes per partial element
  const int G = a.group;
  const int64_t part_off = a.seq[si].part_off, lse_off = a.seq[si].lse_off;
  const int gl = g * a.q_tiles + qt;
  const int64_t split_stride = (int64_t)a.h_kv * a.q_tiles * WAVES * (32 * D);   // elements
  const int64_t lse_stride = (int64_t)a.h_kv * a.q_tiles * 32 * WAVES;
  const auto rp = buffer_rsrc(a.part_o);
  const auto rl = buffer_rsrc(a.part_lse);
  for (int k = tid; k < 32 * P; k += kThreads) {
    const int r = k & 31, pr = k >> 5;
    const int qrow = qt * (32 * WAVES) + 32 * x + r;
    if (qrow >= a.l_d * G) continue;
    const int i = qrow / G, h = g * G + (qrow - i * G);
    const int64_t b0 = fused_block<D, WAVES>(part_off, a.h_kv, a.q_tiles, 0, gl, x) + (int64_t)(64 * pr + r) * 4;
    const int64_t l0 = lse_off + (int64_t)gl * 32 * WAVES + 32 * x + r;
    float mx = -INFINITY, tot = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int j0 = 0; j0 < n_splits; j0 += KB) {
      float t[KB], xv[KB][8];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int j = min(j0 + u, n_splits - 1);           // past the end: a valid split, weight 0
        const float lj = load_l2_f32(rl, 4u * (uint32_t)(l0 + j * lse_stride));
        t[u] = j0 + u < n_splits ? lj * kLog2e : -INFINITY;
        const uint32_t ob = EB * (uint32_t)(b0 + j * split_stride);
        if constexpr (PBF16) {
          const u32x2 w0 = load_l2_b64(rp, ob), w1 = load_l2_b64(rp, ob + 128u * EB);
          xv[u][0] = bf16_bits_to_f32(w0[0] & 0xffffu);
          xv[u][1] = bf16_bits_to_f32(w0[0] >> 16);
          xv[u][2] = bf16_bits_to_f32(w0[1] & 0xffffu);
          xv[u][3] = bf16_bits_to_f32(w0[1] >> 16);
          xv[u][4] = bf16_bits_to_f32(w1[0] & 0xffffu);
          xv[u][5] = bf16_bits_to_f32(w1[0] >> 16);
          xv[u][6] = bf16_bits_to_f32(w1[1] & 0xffffu);
          xv[u][7] = bf16_bits_to_f32(w1[1] >> 16);
        } else {
          const u32x4 w0 = load_l2_b128(rp, ob), w1 = load_l2_b128(rp, ob + 128u * EB);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[u][e] = __uint_as_float(w0[e]);
            xv[u][4 + e] = __uint_as_float(w1[e]);
          }
        }
      }
      float m_new = mx;
#pragma unroll
      for (int u = 0; u < KB; ++u) m_new = fmaxf(m_new, t[u]);
      const float ref = m_new == -INFINITY ? 0.f : m_new;  // every split so far empty: all weights 0
      const float c = __builtin_amdgcn_exp2f(mx - ref);
      tot *= c;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= c;
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const float w = __builtin_amdgcn_exp2f(t[u] - ref);
        tot += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += w * xv[u][e];
      }
      mx = m_new;
    }
    const float inv = 1.f / tot;
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + (((int64_t)s * a.l_d + i) * a.h_q + h) * D + 8 * pr) =
        u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
              pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
    if (a.lse != nullptr && pr == 0) a.lse[((int64_t)s * a.h_q + h) * a.l_d + i] = (mx + __log2f(tot)) * kLn2;
  }
}

// In-kernel LSE merge ("Attention kernel optimization": the splits of a
// (sequence, kv head, query tile) group are merged by a log-sum-exp
// reduction).  The rows of a group are cut into WAVES slices of 32 rows;
// split j owns the slices x with x % n_splits == j.  All splits of a group run
// on one XCD (work_item) and exchange their partials through its L2
// (xwg_sync.h).  After publishing its partial, a split adds its arrival to the
// group's count:
//  * the last arrival merges its own slices, then every slice that no other
//    split has claimed;
//  * an earlier arrival, once every workgroup of the launch has started (so
//    the group's other splits are running or done), waits (bounded) for the
//    count to reach n_splits and merges its own slices; on time-out it leaves
//    them to the last arrival.
// A slice is merged by whoever claims it first (one counter per slice), so
// each is merged once, and no wait depends on a workgroup that has not
// started.
template <int D, int WAVES, bool PBF16, class A, class Sm>
__device__ __forceinline__ void merge_group(const A& a, Sm& sm, int tid, int si, int s, int g, int qt,
                                            int split, int n_splits) {
  const int gi = a.seq[si].grp_begin + g * a.q_tiles + qt;   // the launch's group index
  int* done = a.sync + 2 + gi;
  int* claimed = a.sync + 2 + a.n_groups + (int64_t)gi * WAVES;
  if (tid == 0) {
    sm.xw[0] = counter_add(done, 1);
    sm.xw[1] = counter_load(a.sync);       // workgroups of the launch that have started
  }
  __syncthreads();
  const bool last = sm.xw[0] == n_splits - 1;
  bool go = last;
  if (!last && sm.xw[1] >= a.total_wg) {
    if (tid == 0) {
      int it = 0;
      while (counter_load(done) < n_splits && ++it < kSpinLimit) __builtin_amdgcn_s_sleep(8);
      sm.xw[2] = it < kSpinLimit;
    }
    __syncthreads();
    go = sm.xw[2] != 0;
  }
  if (!go) return;
  // claim (own slices, then -- the last arrival only -- the others), one
  // atomic per slice from the first WAVES threads, then merge those won
  for (int pass = 0; pass < (last ? 2 : 1); ++pass) {
    bool won = false;
    if (tid < WAVES && ((tid % n_splits == split) == (pass == 0))) won = counter_add(claimed + tid, 1) == 0;
    const uint64_t mask = __ballot(won);
    __syncthreads();                       // xw[3] is free
    if (tid == 0) sm.xw[3] = (int)mask;
    __syncthreads();
    const int m = sm.xw[3];
    for (int x = 0; x < WAVES; ++x)
      if (m & (1 << x)) merge_slice<D, WAVES, PBF16>(a, tid, si, s, g, qt, x, n_splits);
  }
}

// MERGE: 0 / 3 = partials for the separate merge kernel (bf16 / float32,
// row-major); 1 / 2 = merged in this launch over float32 / bf16 partials.
//
// The 4-wave instance is compiled for two workgroups per CU (at most 256
// registers per lane; the few values spilled are reloaded outside the tile
// loop or in its row-table refill): left at one, it
// took 384 and ran 7-11% slower per call even with one workgroup per CU.
template <int D, int WAVES, int MERGE>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void decode_bf16_kernel(const DecodeArgs a) {
  constexpr bool FUSED = MERGE == 1 || MERGE == 2;   // the merge runs in this launch
  constexpr bool PBF16 = MERGE == 2;
  constexpr int kThreads = 64 * WAVES;
  constexpr int kRows = 32 * WAVES;        // query rows of the workgroup
  __shared__ Smem<D, WAVES> sm;
  constexpr int KP = Smem<D, WAVES>::KP, VP = Smem<D, WAVES>::VP;
  constexpr int kTableTiles = Smem<D, WAVES>::kTableTiles;
  using Attn = WaveAttn<D, KP, VP>;
  constexpr int DC = Attn::DC, DB = Attn::DB;
  constexpr int TPR = D / 8;               // loader threads per kv row (16 B each)
  constexpr int RPT = kTile * TPR / kThreads;   // kv rows per loader thread
  static_assert(RPT == 1 || RPT == 2 || RPT == 4, "loader mapping");

  // ---- work item: (sequence, kv head, query tile, split).  The launch
  // header and the first two sequence plans are read in one batch first.
  warm_args<0, __builtin_offsetof(DecodeArgs, seq) + 2 * sizeof(DecodeSeq)>(a);
  const WorkItem w0 = work_item<FUSED>(a, blockIdx.x);
  if (!w0.valid) return;                   // padding of a short XCD range
  const int si = w0.si, qt = w0.qt, split = w0.split, g = w0.g, s = w0.s;
  const int k_s = a.seq[si].k_s;
  const int n_kv = a.seq[si].n_kv;
  const int tps = a.seq[si].tiles_per_split;
  const int n_tiles = (n_kv + kTile - 1) / kTile;
  const int t_begin = split * tps;
  const int t_end = min(t_begin + tps, n_tiles);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lc = lane & 31, lj = lane >> 5;     // query column, kv / d half
  const int G = a.group;
  if (!FUSED && tid == 0)
    sm.epi = typename Smem<D, WAVES>::Epi{a.o, a.lse, a.part_o, a.part_lse, a.seq[si].part_off, a.seq[si].lse_off,
                                          s, g, qt, split, w0.n_splits, a.l_d, a.h_q, G};
  if constexpr (FUSED)
    if (tid == 0) counter_add(a.sync, 1);       // this workgroup has started
  const int rows_total = a.l_d * G;
  const uint16_t* pk = static_cast<const uint16_t*>(a.pool_k);
  const uint16_t* pv = static_cast<const uint16_t*>(a.pool_v);
  const uint16_t* rk = static_cast<const uint16_t*>(a.k_resp);
  const uint16_t* rv = static_cast<const uint16_t*>(a.v_resp);

  // ---- row-pointer table for tiles [tw, tw + kTableTiles); rows past n_kv
  // point at the sequence's last row (finite data, masked scores).  Thread
  // tid fills row tid, so wavefront w fills table tile w and its ballot is
  // that tile's absent mask.
  auto build_table = [&](int tw) __attribute__((always_inline)) {
    const int nrow = (min(tw + kTableTiles, t_end) - tw) * kTile;
    bool absent = false;
    if (tid < nrow) {
      const int v = tw * kTile + tid;
      const int64_t off = resolve_row<D>(a, s, g, k_s, min(v, n_kv - 1), absent);
      absent = absent && v < n_kv;
      const bool pool = off >= 0;
      const int64_t e = pool ? off : -1 - off;
      sm.kptr[tid] = (gptr16)((pool ? pk : rk) + e);
      sm.vptr[tid] = (gptr16)((pool ? pv : rv) + e);
    }
    const uint64_t m = __ballot(absent);
    if (lane == 0) sm.absent[wave] = m;
  };
  int tw = t_begin;

  // ---- first fill of the row table, and the queries.  Each thread resolves
  // at most one row.  Its two dependent index loads (sel_chunk, then
  // chunk_slot and keep_rows) read clamped, always valid addresses, so they
  // are unconditional; the query loads are issued after the second pair.
  // Loads retire in issue order, so the wait for the indices does not
  // include the queries, which arrive while the table is written and the
  // first tiles are fetched.
  bf16x8 qf[DC];
  const int qrow = qt * kRows + wave * 32 + lc;
  {
    static_assert(kTableTiles * kTile == kThreads, "one table row per thread");
    typedef __attribute__((address_space(1))) const int32_t* gptr32;
    const int nrow = (min(tw + kTableTiles, t_end) - tw) * kTile;
    const int per = a.b + 1;
    const int v = max(0, min(tw * kTile + min(tid, nrow - 1), n_kv - 1));
    const int kk = min(v / per, max(k_s - 1, 0));
    const int r = min(v - kk * per, per - 1);   // BOS row 0, then kept rows 1..b
    // the chunks this split's rows fall in (one per thread, clamped): any
    // with an absent row has -1 as its last kept-row entry
    const bool tbl = k_s > 0 && a.b > 0 && a.keep_rows != nullptr;
    const int k_lo = min(t_begin * kTile / per, max(k_s - 1, 0));
    const int k_hi = min((t_end * kTile - 1) / per, max(k_s - 1, 0));
    const int kx = min(k_lo + tid, k_hi);
    // a sequence with no selected chunk reads only idx_dummy (valid device
    // memory): its chunk_slot / sel_chunk may be NULL
    const int32_t* dummy = a.idx_dummy;
    const bool rmode = a.rows != nullptr;      // resolved rows: one load, no index chain
    const int32_t* rt = rmode ? a.rows + (int64_t)s * a.rows_stride : dummy;
    if (rmode) {
      const bool pool = v < k_s * per;
      const int e_ld = *(gptr32)(pool ? rt + v : dummy);
      // any absent row among the split's pool rows (one row a thread per
      // 512 rows of the split)
      bool any = false;
      for (int vv = t_begin * kTile + tid; vv < min(t_end * kTile, k_s * per); vv += kThreads)
        any = any || *(gptr32)(rt + vv) < 0;
      __builtin_amdgcn_sched_barrier(0);   // the row loads go out before the queries
      {
        const int qr = min(qrow, rows_total - 1);
        const int i = qr / G, h = g * G + (qr - i * G);
        load_q<DC, 16>(qf, static_cast<const uint16_t*>(a.q) + (((int64_t)s * a.l_d + i) * a.h_q + h) * D + 8 * lj);
      }
      const bool absent = pool && e_ld < 0;
      const int64_t e = pool ? ((int64_t)(uint32_t)(e_ld & 0x7fffffff) << 3) + (int64_t)g * a.ps_head
                             : (((int64_t)s * a.l_d + (v - k_s * per)) * a.h_kv + g) * D;
      sm.kptr[tid] = (gptr16)((pool ? pk : rk) + e);
      sm.vptr[tid] = (gptr16)((pool ? pv : rv) + e);
      const uint64_t m = __ballot(absent && tid < nrow);
      if (lane == 0) sm.absent[wave] = m;
      const uint64_t fw = __ballot(any);
      if (lane == 0) sm.flag[wave] = fw != 0;
    } else {
    const int c0 = *(gptr32)(k_s > 0 ? a.sel_chunk + (int64_t)s * a.k_max + kk : dummy);
    const int cx = *(gptr32)(k_s > 0 ? a.sel_chunk + (int64_t)s * a.k_max + kx : dummy);
    const int cg = s * a.n_chunks_per_seq + min(max(c0, 0), a.n_chunks_per_seq - 1);
    const int cgx = s * a.n_chunks_per_seq + min(max(cx, 0), a.n_chunks_per_seq - 1);
    const int slot = *(gptr32)(k_s > 0 ? a.chunk_slot + cg : dummy);
    const int krow_ld = *(gptr32)(tbl ? a.keep_rows + (int64_t)cg * a.b + max(r - 1, 0) : dummy);
    const int klast = *(gptr32)(tbl ? a.keep_rows + (int64_t)cgx * a.b + (a.b - 1) : dummy);
    // compacted slots: kept row i sits at row 1 + i; keep_rows, when given,
    // only marks absent rows (-1), which point at the BOS row
    const bool absent = r > 0 && a.keep_rows != nullptr && krow_ld < 0;
    const int krow = absent ? 0 : a.compact ? r : krow_ld;
    __builtin_amdgcn_sched_barrier(0);     // the index loads go out before the queries
    // queries: B-operand fragments of S^T (lane: query column lc, d = 16 dc
    // + 8 lj ..); rows past the end read the last row (never stored)
    {
      const int qr = min(qrow, rows_total - 1);
      const int i = qr / G, h = g * G + (qr - i * G);
      load_q<DC, 16>(qf, static_cast<const uint16_t*>(a.q) + (((int64_t)s * a.l_d + i) * a.h_q + h) * D + 8 * lj);
    }
    // every entry is written (those past nrow hold a valid clamped row and are
    // never read), so the index values have one unconditional use
    const bool pool = v < k_s * per;
    const int64_t e = pool ? (int64_t)slot * a.ps_slot + (int64_t)(r ? krow : 0) * a.ps_row + (int64_t)g * a.ps_head
                           : (((int64_t)s * a.l_d + (v - k_s * per)) * a.h_kv + g) * D;
    sm.kptr[tid] = (gptr16)((pool ? pk : rk) + e);
    sm.vptr[tid] = (gptr16)((pool ? pv : rv) + e);
    const uint64_t m = __ballot(pool && absent && tid < nrow);
    if (lane == 0) sm.absent[wave] = m;
    // a split spanning more chunks than threads (a long split of short
    // chunks) takes the masked path unchecked: its masks are exact either way
    const bool flag = tbl && k_s > 0 && t_begin * kTile < k_s * per && (klast < 0 || k_hi - k_lo >= kThreads);
    const uint64_t fw = __ballot(flag);
    if (lane == 0) sm.flag[wave] = fw != 0;
    }
  }

  Attn at;
  at.init();
  const float sl2 = a.scale_log2;
  const int k_lane = lc * KP + 8 * lj;      // lane offsets inside one LDS buffer
  const int v_lane = v_lane_offset(lane, VP);
  constexpr int NK = kTile / 32;
  const uint16_t* k_base = &sm.k[0][0] + k_lane;
  const uint16_t* v_base = &sm.v[0][0] + v_lane;

  __syncthreads();                         // row table ready
  bool has_absent = false;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) has_absent = has_absent || sm.flag[w];
  has_absent = __builtin_amdgcn_readfirstlane((int)has_absent) != 0;

  // The tile loader, prologue and main loop, in instances (compile-time):
  // ABS for a split that holds an absent kept row, and the plain one; and a
  // MODE:
  //   kRunAll   every wavefront loads its share of each tile and computes;
  //   kRunIdle  a wavefront whose 32 query rows all lie past the last one
  //             (L_d * G not a multiple of the workgroup's rows): it loads
  //             its share and meets the barriers, with no attention
  //             arithmetic;
  //   kRunCons / kRunProd  when the last four wavefronts of an 8-wave
  //             workgroup hold no query rows (L_d * G <= 128 past the tile's
  //             first row): waves 0-3 only compute, and waves 4-7 load every
  //             row of every tile, with kProdStages staging sets, so that three
  //             load units (96 KB of K/V for d = 128) are in flight per CU
  //             instead of two -- the small-L_d decode is bound by the bytes
  //             it keeps in flight.  Both run the same loop control and
  //             barriers.  (Four sets measured no different in registers but
  //             made the compiler copy the argument block to scratch.)
  auto run = [&](auto abs_flag, auto mode_c) __attribute__((always_inline)) {
    constexpr bool ABS = decltype(abs_flag)::value;
    constexpr int MODE = decltype(mode_c)::value;
    constexpr bool SPLIT = MODE == kRunCons || MODE == kRunProd;
    constexpr bool LOADS = MODE != kRunCons;            // this wavefront loads tiles
    constexpr bool COMPUTES = MODE == kRunAll || MODE == kRunCons;
    // ---- tile loader.  A loader thread owns LRPT consecutive kv rows x 8 d
    // values of a tile.  K runs one tile ahead of V: load unit a carries K
    // of tile a and V of tile a-1 (local tile numbers u = t - t_begin,
    // clamped to the split, so a unit past its end re-reads valid rows that
    // are never stored).  ST staging register sets let a unit's loads be
    // issued ST iterations before its LDS store.
    // The prologue fetches the row pointers of units up to 2 + ST without a
    // refill check, so they must lie in the first table fill: the 4-wave
    // table (4 tiles) allows one staging set only.
    constexpr int LTHREADS = SPLIT ? kThreads / 2 : kThreads;   // loader threads
    constexpr int LRPT = kTile * TPR / LTHREADS;
    constexpr int ST = SPLIT ? kProdStages : (RPT <= 2 && 2 + 2 < kTableTiles) ? 2 : 1;
    // loop unroll: a multiple of ST (staging sets are compile-time indices)
    // and of 2 (the score buffers alternate with the parity of u)
    constexpr int UNR = ST % 2 == 0 ? ST : 2 * ST;
    static_assert(LRPT == 1 || LRPT == 2 || LRPT == 4, "loader mapping");
    static_assert(2 + ST < kTableTiles, "prologue units must lie in the first row table");
    static_assert(UNR % ST == 0 && UNR % 2 == 0, "unroll");
    const int ltid = SPLIT ? tid - kThreads / 2 : tid;   // loader thread index (loaders only)
    const bool lead = ltid == 0;               // the loader thread that writes tile masks
    const int ld_d0 = 8 * (ltid % TPR);
    const int ld_r0 = LRPT * (ltid / TPR);
    const int n_loc = t_end - t_begin;
    constexpr int NSET = LOADS ? ST : 1;
    u32x4 kreg[NSET][LRPT], vreg[NSET][LRPT];
    gptr16 kp_next[LRPT], vp_next[LRPT];     // row pointers of the next unit to load
    // A K tile's absent mask (bit r: row r is an absent kept row) travels with
    // its rows: read from the table with the pointers, held with the staged
    // registers, written beside the tile into LDS, read back with the tile's
    // S^T (wave-uniform values; ABS instance only).
    uint64_t km_next = 0, km_set[NSET];
    auto fetch_ptrs = [&](int uk, int uv) __attribute__((always_inline)) {   // local tiles of K and V rows
      if constexpr (LOADS) {
        const int tk = t_begin + min(uk, n_loc - 1) - tw;
        const int ik = tk * kTile + ld_r0;
        const int iv = (t_begin + min(max(uv, 0), n_loc - 1) - tw) * kTile + ld_r0;
#pragma unroll
        for (int i = 0; i < LRPT; ++i) {
          kp_next[i] = sm.kptr[ik + i];
          vp_next[i] = sm.vptr[iv + i];
        }
        if constexpr (ABS) km_next = uniform_u64(sm.absent[tk]);
      }
    };
    auto load_unit = [&](int set) __attribute__((always_inline)) {
      if constexpr (LOADS) {
#pragma unroll
        for (int i = 0; i < LRPT; ++i) {
          kreg[set][i] = *reinterpret_cast<__attribute__((address_space(1))) const u32x4*>(kp_next[i] + ld_d0);
          vreg[set][i] = *reinterpret_cast<__attribute__((address_space(1))) const u32x4*>(vp_next[i] + ld_d0);
        }
        if constexpr (ABS) km_set[set] = km_next;
      }
    };
    auto store_k = [&](int buf, int set) __attribute__((always_inline)) {
      if constexpr (LOADS) {
#pragma unroll
        for (int i = 0; i < LRPT; ++i)
          *reinterpret_cast<u32x4*>(&sm.k[buf][(ld_r0 + i) * KP + ld_d0]) = kreg[set][i];
        if constexpr (ABS)
          if (lead) sm.kmask[buf] = km_set[set];
      }
    };
    auto store_v = [&](int buf, int set) __attribute__((always_inline)) {
      if constexpr (LOADS) {
#pragma unroll
        for (int i = 0; i < LRPT; ++i)
          *reinterpret_cast<u32x4*>(&sm.v[buf][(ld_r0 + i) * VP + ld_d0]) = vreg[set][i];
      }
    };

    // ---- prologue: K and V of tile 0 and K of tile 1 into LDS, units 2 ..
    // 1 + ST in flight, S^T of tile 0 computed
    fetch_ptrs(0, 0);
    load_unit(0);
    if constexpr (ST >= 2) {                 // tiles 0 and 1 in one memory round trip
      fetch_ptrs(1, 1);
      load_unit(1);
      store_k(0, 0);
      store_v(0, 0);
      store_k(1, 1);
    } else {
      store_k(0, 0);
      store_v(0, 0);
      fetch_ptrs(1, 1);
      load_unit(0);
      store_k(1, 0);
    }
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      fetch_ptrs(2 + i, 1 + i);
      load_unit((2 + i) % ST);
    }
    fetch_ptrs(2 + ST, 1 + ST);
    __syncthreads();
    f32x16 sc_a[NK], sc_b[NK];
    float ms_a = 0.f, ms_b = 0.f;
    if constexpr (COMPUTES) {
      at.template qk<NK>(sc_a, k_base, qf);
      uint64_t am0 = 0;                      // the absent mask of tile 0
      if constexpr (ABS) am0 = uniform_u64(sm.kmask[0]);
      // each tile's mask and scaled row max are taken one iteration ahead,
      // after the previous tile's PV MFMAs (ms_a / ms_b go with sc_a / sc_b)
      ms_a = at.template block_max<NK>(sc_a, sl2, n_kv - t_begin * kTile, lj, 0, am0);
    }
    __syncthreads();                         // K buffer 0 is rewritten in iteration 0

    // ---- main loop.  Iteration u stores unit u+2 (K of tile u+2 into K buffer
    // u & 1, whose tile u was last read in iteration u-1; V of tile u+1 into V
    // buffer (u+1) & 1, last read by tile u-1), issues the loads of unit
    // u+2+ST into the staging set just freed, then runs the softmax of tile u
    // with the S^T MFMAs of tile u+1 interleaved, and the PV of tile u.
    // Every iteration issues exactly one unit's loads, so the wait before a
    // store covers only loads issued ST iterations earlier.  One barrier per
    // tile.  R = u % UNR (compile-time): unit u+2 sits in set (R + 2) % ST.
    auto iter = [&](auto r_c, int u, f32x16 (&cur)[NK], f32x16 (&nxt)[NK], float ms_cur,
                    float& ms_nxt) __attribute__((always_inline)) {
      constexpr int set = (decltype(r_c)::value + 2) % ST;
      if (u + 2 < n_loc) store_k(u & 1, set);
      if (u + 1 < n_loc) store_v((u + 1) & 1, set);
      load_unit(set);
      const int un = u + 3 + ST;             // the unit the next iteration loads
      if (un <= n_loc) {                     // beyond, the clamped pointers stay valid
        if (t_begin + min(un, n_loc - 1) - tw >= kTableTiles) {   // refill the row table (rare)
          __syncthreads();                   // every wave has read the old table
          tw = t_begin + min(un, n_loc - 1) - 1;
          build_table(tw);
          __syncthreads();
        }
        fetch_ptrs(un, un - 1);
      }
      const int t = t_begin + u;
      if constexpr (COMPUTES) {
        bf16x8 pf[2 * NK];
        // softmax at raised wave priority, PV at the default (as in the
        // prefill's chunk items)
        __builtin_amdgcn_s_setprio(3);
        at.rescale(ms_cur);
        uint64_t am_nxt = 0;
        if (u + 1 < n_loc) {
          if constexpr (ABS) am_nxt = uniform_u64(sm.kmask[(u + 1) & 1]);
          at.template exp_qk<NK, true, LOADS ? 1 : 0>(cur, pf, nxt, k_base + ((u + 1) & 1) * (kTile * KP), qf, sl2);
        } else {
          at.template exp_qk<NK, false>(cur, pf, nxt, nullptr, qf, sl2);
        }
        // every 16-row piece, the last tile's too: its rows past n_kv hold
        // finite data (the last row) and p = 0, so they add exactly zero, and
        // with no branch between the pieces the V reads can run ahead of the
        // MFMAs
        __builtin_amdgcn_s_setprio(0);
        at.template pv<NK, true>(pf, v_base + (u & 1) * (kTile * VP));
        if (u + 1 < n_loc) ms_nxt = at.template block_max<NK>(nxt, sl2, n_kv - (t + 1) * kTile, lj, 0, am_nxt);
      }
      __syncthreads();
    };
    {
      // the UNR copies are unconditional inside the loop, so the loop head is
      // reached only after the last copy's loads (exact wait counts before
      // stores); the remaining iterations follow, each under its bound
      int u = 0;
      for (; u + UNR - 1 < n_loc; u += UNR)
        static_for<0, UNR>([&](auto r_c) __attribute__((always_inline)) {
          constexpr int R = decltype(r_c)::value;
          if constexpr (R % 2 == 0)
            iter(r_c, u + R, sc_a, sc_b, ms_a, ms_b);
          else
            iter(r_c, u + R, sc_b, sc_a, ms_b, ms_a);
        });
      static_for<0, UNR - 1>([&](auto r_c) __attribute__((always_inline)) {
        constexpr int R = decltype(r_c)::value;
        if (u + R < n_loc) {
          if constexpr (R % 2 == 0)
            iter(r_c, u + R, sc_a, sc_b, ms_a, ms_b);
          else
            iter(r_c, u + R, sc_b, sc_a, ms_b, ms_a);
        }
      });
    }
  };
  // whole workgroup: the last four wavefronts hold no query rows
  const bool split_roles =
      WAVES == 8 && __builtin_amdgcn_readfirstlane(qt * kRows + (WAVES / 2) * 32 >= rows_total ? 1 : 0) != 0;
  const bool idle = __builtin_amdgcn_readfirstlane(qt * kRows + wave * 32 >= rows_total ? 1 : 0) != 0;
  if constexpr (WAVES == 8) {
    if (split_roles) {
      if (wave >= WAVES / 2) {
        if (has_absent)
          run(BoolConst<true>{}, IntConst<kRunProd>{});
        else
          run(BoolConst<false>{}, IntConst<kRunProd>{});
      } else if (has_absent) {
        run(BoolConst<true>{}, IntConst<kRunCons>{});
      } else {
        run(BoolConst<false>{}, IntConst<kRunCons>{});
      }
    }
  }
  if (!split_roles) {
    if (idle)
      run(BoolConst<false>{}, IntConst<kRunIdle>{});
    else if (has_absent)
      run(BoolConst<true>{}, IntConst<kRunAll>{});
    else
      run(BoolConst<false>{}, IntConst<kRunAll>{});
  }

  // ---- epilogue (lanes lc and lc + 32 hold halves of the same query row).
  // None of the work item's scalars stays live in registers across the main
  // loop: the separate-merge path reads them back from LDS (sm.epi); the
  // in-kernel merge derives the work item again from the block id (the empty
  // asm hides that it was computed before) and reads the kernel arguments
  // again from the argument segment, through a pointer the compiler cannot
  // see through.  The lane's row is derived again from the thread id.
  int bid = blockIdx.x;
  asm volatile("" : "+s"(bid));
  KernArgs<DecodeArgs> ap = kernarg<DecodeArgs>();
  {
  const auto& a = *ap;
  typename Smem<D, WAVES>::Epi e;
  int si = 0;
  if constexpr (!FUSED) {
    auto rf = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    auto rp = [](auto* p) { return reinterpret_cast<decltype(p)>(uniform_u64(reinterpret_cast<uint64_t>(p))); };
    e.o = rp(sm.epi.o);
    e.lse = rp(sm.epi.lse);
    e.part_o = rp(sm.epi.part_o);
    e.part_lse = rp(sm.epi.part_lse);
    e.part_off = (int64_t)uniform_u64((uint64_t)sm.epi.part_off);
    e.lse_off = (int64_t)uniform_u64((uint64_t)sm.epi.lse_off);
    e.s = rf(sm.epi.s);
    e.g = rf(sm.epi.g);
    e.qt = rf(sm.epi.qt);
    e.split = rf(sm.epi.split);
    e.n_splits = rf(sm.epi.n_splits);
    e.l_d = rf(sm.epi.l_d);
    e.h_q = rf(sm.epi.h_q);
    e.group = rf(sm.epi.group);
  } else {
    const WorkItem w = work_item<FUSED>(a, bid);
    si = w.si;
    e = typename Smem<D, WAVES>::Epi{a.o, a.lse, a.part_o, a.part_lse, 0, 0, w.s, w.g, w.qt, w.split,
                                     w.n_splits, a.l_d, a.h_q, a.group};
  }
  const int s = e.s, g = e.g, qt = e.qt, split = e.split, n_splits = e.n_splits, G = e.group;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lj = (tid & 63) >> 5;
  const int qrow = qt * kRows + (tid >> 6) * 32 + (tid & 31);
  const int rows_total = e.l_d * G;
  const float l = at.row_sum();
  const float inv = l > 0.f ? 1.f / l : 0.f;     // a split of absent rows only: o = 0, lse = -inf
  const float lse_v = at.lse(l);
  const bool row_ok = qrow < rows_total;
  const int qr = min(qrow, rows_total - 1);
  const int i = qr / G, h = g * G + (qr - i * G);
  if (n_splits == 1) {
    if (row_ok) {
      store_o_bf16<DB>(static_cast<uint16_t*>(e.o) + (((int64_t)s * e.l_d + i) * e.h_q + h) * D + 8 * lj,
                       at.acc, inv);
      if (e.lse != nullptr && lj == 0) e.lse[((int64_t)s * e.h_q + h) * e.l_d + i] = lse_v;
    }
  } else if constexpr (!FUSED) {
    if (row_ok) {
      const int64_t prow = e.part_off + (((int64_t)split * e.l_d + i) * e.h_q + h) * D;
      if constexpr (MERGE == 3)
        store_o_f32<DB>(static_cast<float*>(e.part_o) + prow, at.acc, inv, lj);
      else
        store_o_bf16<DB>(static_cast<uint16_t*>(e.part_o) + prow + 8 * lj, at.acc, inv);
      if (lj == 0) e.part_lse[e.lse_off + ((int64_t)split * e.l_d + i) * e.h_q + h] = lse_v;
    }
  } else {
    // the partial, into this XCD's L2 in the merge's lane-major layout: one
    // contiguous run per store instruction (rows past the end hold finite
    // values the merge never reads)
    {
      const int gl = g * a.q_tiles + qt, wv = (tid >> 6) & (WAVES - 1), ln = tid & 63;
      const auto rp = buffer_rsrc(a.part_o);
      const int64_t blk = fused_block<D, WAVES>(a.seq[si].part_off, a.h_kv, a.q_tiles, split, gl, wv);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float v0 = at.acc[db][4 * m] * inv, v1 = at.acc[db][4 * m + 1] * inv;
          const float v2 = at.acc[db][4 * m + 2] * inv, v3 = at.acc[db][4 * m + 3] * inv;
          const uint32_t off = (uint32_t)(blk + (int64_t)(64 * (4 * db + m) + ln) * 4);
          if constexpr (PBF16)
            store_l2(rp, 2u * off, u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)});
          else
            store_l2(rp, 4u * off, u32x4{__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2),
                                               __float_as_uint(v3)});
        }
      if (lj == 0)
        store_l2(buffer_rsrc(a.part_lse),
                       4u * (uint32_t)(a.seq[si].lse_off + (int64_t)(split * a.h_kv * a.q_tiles + gl) * 32 * WAVES +
                                       32 * wv + (ln & 31)),
                       lse_v);
    }
    wait_vm_all();                         // this thread's partial is stored
    __syncthreads();                       // ... and every thread's
    merge_group<D, WAVES, PBF16>(a, sm, tid, si, s, g, qt, split, n_splits);
  }
  }
  if constexpr (FUSED) {
    const auto& a = *ap;
    // The workgroup that leaves last returns the sync words to zero for the
    // next launch; every other workgroup has made its last access to them
    // (each waits for its own atomics before counting itself out).
    __syncthreads();
    if (tid == 0) sm.xw[0] = counter_add(a.sync + 1, 1);
    __syncthreads();
    if (sm.xw[0] == a.total_wg - 1) {
      const int n = 2 + a.n_groups * (1 + WAVES);
      for (int k = tid; k < n; k += kThreads) counter_store(a.sync + k, 0);
    }
  }
}

// LSE merge of the per-split partials ("Attention kernel optimization"):
// lse = M + ln sum_j exp(lse_j - M), o = sum_j exp(lse_j - lse) o_j, summed
// in float32 and rounded once to the output type.  With PBF16 the partial
// outputs are bf16 and each thread takes 8 values of a row, otherwise
// float32 and 4 values; OBF16: o is bf16 (else float32).
template <int D, bool PBF16, bool OBF16, int kBatch>
__global__ __launch_bounds__(256) void lse_merge_kernel(const DecodeArgs a) {
  constexpr bool BF16 = PBF16;
  constexpr int EPT = BF16 ? 8 : 4;        // values per thread (16 bytes of partial)
  constexpr int TPR = D / EPT;
  constexpr int RPB = 256 / TPR;
  const int si = blockIdx.y;                // the grid has one row per sequence of the launch
  // this sequence's plan and the launch header, read in one batch
  const int n_splits = a.seq[si].n_splits;
  const int64_t part_off = a.seq[si].part_off, lse_off = a.seq[si].lse_off;
  warm_args<0, __builtin_offsetof(DecodeArgs, seq)>(a);
  asm volatile("" ::"s"(n_splits), "s"(part_off), "s"(lse_off));
  if (n_splits <= 1) return;
  const int rows = a.l_d * a.h_q;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  const int e0 = EPT * (threadIdx.x % TPR);
  const float* pl = a.part_lse + lse_off + row;
  const int64_t po = part_off + (int64_t)row * D + e0;   // element offset
  const int64_t sl = rows, so = (int64_t)rows * D;
  // A split's 16 bytes of partial output are held as loaded and widened to
  // float32 only where they are summed: widening at the load made the
  // compiler wait for each load in turn (to keep the wider values' registers
  // few), one memory round trip per split.
  auto load = [&](int j) {
    return *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.part_o) + (po + j * so) * (BF16 ? 2 : 4));
  };
  auto value = [&](const u32x4& w, int e) {
    if constexpr (BF16)
      return bf16_bits_to_f32(e % 2 ? w[e / 2] >> 16 : w[e / 2] & 0xffffu);
    else
      return __uint_as_float(w[e]);
  };
  // Splits are visited in groups of kBatch (4 to 16, fitted at launch to
  // the largest split count) whose lse and partial loads are all in flight
  // together: one memory round trip per group.  The weights of a group are
  // taken against the running maximum (in log2 units), and the sums of
  // earlier groups are rescaled when it grows.
  float mx = -INFINITY, tot = 0.f;
  float o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
  for (int j0 = 0; j0 < n_splits; j0 += kBatch) {
    float t[kBatch];
    u32x4 x[kBatch];
    // every load is unconditional (past the end: a valid split, weight 0 by
    // the select below), so no branch splits them and the compiler waits
    // once for the whole group rather than after each lse load
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = min(j0 + u, n_splits - 1);
      t[u] = pl[j * sl];
      x[u] = load(j);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) t[u] = j0 + u < n_splits ? t[u] * kLog2e : -INFINITY;
    float m_new = mx;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) m_new = fmaxf(m_new, t[u]);
    // every split so far empty (lse = -inf): weigh against 0, all weights are 0
    const float ref = m_new == -INFINITY ? 0.f : m_new;
    const float c = __builtin_amdgcn_exp2f(mx - ref);   // 0 on the first group
    tot *= c;
#pragma unroll
    for (int e = 0; e < EPT; ++e) o[e] *= c;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = __builtin_amdgcn_exp2f(t[u] - ref);   // 0 for an empty split and past the end
      tot += w;
#pragma unroll
      for (int e = 0; e < EPT; ++e) o[e] += w * value(x[u], e);
    }
    mx = m_new;
  }
  const float inv = 1.f / tot;
  const int s = a.seq0 + si;
  const int i = row / a.h_q, h = row - i * a.h_q;
  const int64_t out = ((int64_t)s * rows + row) * D + e0;
  if constexpr (BF16) {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + out) =
        u32x4{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
              pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
  } else if constexpr (OBF16) {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + out) =
        u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + out) =
        f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  }
  if (a.lse != nullptr && e0 == 0) a.lse[((int64_t)s * a.h_q + h) * a.l_d + i] = (mx + __log2f(tot)) * kLn2;
}

template <int D, bool PBF16, bool OBF16>
int merge_launch(const DecodeArgs& a, void* stream) {
  constexpr int RPB = 256 / (D / (PBF16 ? 8 : 4));
  const int rows = a.l_d * a.h_q;
  dim3 grid((rows + RPB - 1) / RPB, a.n_seq_launch);
  int ns = 1;
  for (int i = 0; i < a.n_seq_launch; ++i) ns = max(ns, a.seq[i].n_splits);
  const hipStream_t st = (hipStream_t)stream;
  if (ns <= 4)
    hipLaunchKernelGGL((lse_merge_kernel<D, PBF16, OBF16, 4>), grid, dim3(256), 0, st, a);
  else if (ns <= 8)
    hipLaunchKernelGGL((lse_merge_kernel<D, PBF16, OBF16, 8>), grid, dim3(256), 0, st, a);
  else if (ns <= 12)
    hipLaunchKernelGGL((lse_merge_kernel<D, PBF16, OBF16, 12>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((lse_merge_kernel<D, PBF16, OBF16, 16>), grid, dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

template <int MERGE>
int launch_decode_bf16_t(const DecodeArgs& a, int d, int q_rows_per_wg, hipStream_t st) {
  const dim3 grid(a.grid_wg);
  if (d == 128 && q_rows_per_wg == 256)
    hipLaunchKernelGGL((decode_bf16_kernel<128, 8, MERGE>), grid, dim3(512), 0, st, a);
  else if (d == 128 && q_rows_per_wg == 128)
    hipLaunchKernelGGL((decode_bf16_kernel<128, 4, MERGE>), grid, dim3(256), 0, st, a);
  else if (d == 64 && q_rows_per_wg == 256)
    hipLaunchKernelGGL((decode_bf16_kernel<64, 8, MERGE>), grid, dim3(512), 0, st, a);
  else if (d == 64 && q_rows_per_wg == 128)
    hipLaunchKernelGGL((decode_bf16_kernel<64, 4, MERGE>), grid, dim3(256), 0, st, a);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace

int launch_decode_bf16(const DecodeArgs& a, int d, int q_rows_per_wg, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  switch (a.merge_kind) {
    case 0: return launch_decode_bf16_t<0>(a, d, q_rows_per_wg, st);
    case 1: return launch_decode_bf16_t<1>(a, d, q_rows_per_wg, st);
    case 2: return launch_decode_bf16_t<2>(a, d, q_rows_per_wg, st);
    case 3: return launch_decode_bf16_t<3>(a, d, q_rows_per_wg, st);
    default: return (int)hipErrorInvalidValue;
  }
}

int launch_lse_merge(const DecodeArgs& a, int d, bool bf16_part, bool bf16_out, void* stream) {
  if (bf16_part && !bf16_out) return (int)hipErrorInvalidValue;
  // (bf16 partials, bf16 o) for bf16 inputs, (float32, bf16) for bf16 inputs
  // with float32 partials, (float32, float32) for float32 inputs
  switch (d) {
    case 16: return bf16_out ? merge_launch<16, false, true>(a, stream) : merge_launch<16, false, false>(a, stream);
    case 32: return bf16_out ? merge_launch<32, false, true>(a, stream) : merge_launch<32, false, false>(a, stream);
    case 64:
      return bf16_part  ? merge_launch<64, true, true>(a, stream)
             : bf16_out ? merge_launch<64, false, true>(a, stream)
                        : merge_launch<64, false, false>(a, stream);
    case 128:
      return bf16_part  ? merge_launch<128, true, true>(a, stream)
             : bf16_out ? merge_launch<128, false, true>(a, stream)
                        : merge_launch<128, false, false>(a, stream);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace pdllm
