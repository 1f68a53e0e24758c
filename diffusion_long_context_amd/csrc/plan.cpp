// Split planner of the split-KV decode (host only, deterministic).
//
// The decode attention of one sequence covers N_s = K_s (B + 1) + L_d kv
// rows (every selected chunk's BOS row and B kept rows, then the response
// rows; Prefilling-dLLM summary, Methodology 2 and 3).  "Attention kernel
// optimization" splits that KV dimension into independently processed parts
// merged by log-sum-exp.  Here a split is a run of whole 64-row kv tiles and
// a workgroup computes one (sequence, kv head, query tile, split).
//
// With num_splits = 0 the planner picks one tiles-per-split value for the
// call by a small cost model measured in tile-times.  Workgroups of one
// launch have nearly equal length, so they run in rounds of `slots` (compute
// units times the workgroups resident per CU):
//   time(tps) = sum over launches of ceil(n_wg / slots) * (tps + c0) + merge(max_splits)
// where c0 is a workgroup's fixed cost (index table, query load, epilogue)
// and merge() charges the extra merge pass and its partial-output traffic;
// a call of more than kMaxSeqPerLaunch sequences runs as several launches,
// one after the other, each of which must fill the GPU on its own.  Ties go
// to fewer splits.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "pdllm_internal.h"

namespace pdllm {

namespace {
constexpr double kFixedTiles = 2.0;        // c0: per-workgroup overhead in tile-times
constexpr double kMergeBase = 1.0;         // merge launch + pass, in tile-times
constexpr double kMergePerSplit = 0.25;    // partial write + read per split
constexpr int kFusedBf16Merge = 3;         // merge option: in-kernel over bf16 partials
constexpr int kSeparateF32Merge = 4;       // merge option: separate kernel over float32 partials
// The library's choice for bf16 inputs: the separate merge kernel.  Merging
// in the decode launch measured slower on every workload here (32K prefix:
// 57-59 against 44 us a call), because its tail -- partials through the L2,
// arrival atomics, a slice merge -- is longer than a kernel boundary plus the
// merge kernel.
constexpr int kDefaultBf16Merge = 1;
constexpr double kFusedMergeBase = 0.75;   // in-kernel merge: arrival, wait and one slice
constexpr double kFusedMergePerSplit = 0.05;
constexpr int kResidentBf16Large = 1;      // 8-wave bf16 workgroups per CU
constexpr int kResidentBf16Small = 1;      // 4-wave bf16 workgroups per CU (over 256 registers per lane)
constexpr int kResidentF32 = 4;
// Measured on MI355X (fits over graph-replayed decode calls at the 8K, 32K
// and full-step shapes), in microseconds: the split decode costs a
// workgroup's fixed part plus its tiles, then the merge kernel and the
// partials' round trip; the decode without splits costs its fixed part (row
// table, first tile, the wavefronts' merge in LDS) plus one step per round of
// eight 32-row tiles.  They decide between the two designs only.
constexpr double kSplitWgUs = 3.7, kSplitTileUs = 1.71, kSplitTileSmallUs = 1.43;
constexpr double kSplitMergeUs = 6.6, kSplitMergePerSplitUs = 1.0;
constexpr double kWsFixedUs = 10.5, kWsRoundUs = 1.8;

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Ranges needed when no range may sum above `cap` (greedy from the front).
int ranges_needed(const std::vector<int>& sizes, int64_t cap) {
  int n = 1;
  int64_t cur = 0;
  for (int v : sizes) {
    if (cur + v > cap) {
      ++n;
      cur = 0;
    }
    cur += v;
  }
  return n;
}
}  // namespace

int64_t xcd_partition(const std::vector<int>& sizes, int32_t* bounds) {
  int64_t lo = 0, hi = 0;
  for (int v : sizes) {
    lo = std::max<int64_t>(lo, v);
    hi += v;
  }
  while (lo < hi) {               // smallest cap that kXcdGroups ranges can meet
    const int64_t mid = (lo + hi) / 2;
    if (ranges_needed(sizes, mid) <= kXcdGroups)
      hi = mid;
    else
      lo = mid + 1;
  }
  int x = 0;
  int64_t cur = 0;
  bounds[0] = 0;
  for (int i = 0; i < (int)sizes.size(); ++i) {
    if (cur + sizes[i] > lo) {
      bounds[++x] = i;
      cur = 0;
    }
    cur += sizes[i];
  }
  while (x < kXcdGroups) bounds[++x] = (int32_t)sizes.size();
  return lo;
}

bool plan_decode(const int32_t* k_per_seq, int n_seq, int b, int l_d, int h_q, int h_kv,
                 int d, int dtype, int num_splits, int force_rows, int merge, int n_cu, DecodePlan* plan,
                 const char** err, bool ws_allowed) {
  if (n_seq < 1 || l_d < 1 || h_q < 1 || h_kv < 1 || d < 1 || b < 0 || num_splits < 0 ||
      n_cu < 1 || h_q % h_kv != 0 || k_per_seq == nullptr || plan == nullptr) {
    *err = "plan: invalid sizes (need n_seq, l_d, h_q, h_kv, d, n_cu >= 1, b >= 0, "
           "num_splits >= 0, h_q % h_kv == 0)";
    return false;
  }
  const int group = h_q / h_kv;
  const int64_t q_rows = (int64_t)l_d * group;
  if (merge == 0) merge = dtype == 1 ? kDefaultBf16Merge : 1;
  const bool fused = dtype == 1 && (merge == 2 || merge == kFusedBf16Merge);
  DecodePlan p;
  p.n_seq = n_seq;
  p.k_s.resize(n_seq);
  p.n_kv.resize(n_seq);
  p.n_tiles.resize(n_seq);
  int max_tiles = 1;
  for (int s = 0; s < n_seq; ++s) {
    if (k_per_seq[s] < 0) {
      *err = "plan: k_per_seq entries must be >= 0";
      return false;
    }
    const int64_t nkv = (int64_t)k_per_seq[s] * (b + 1) + l_d;
    if (nkv > (int64_t)1 << 30) {
      *err = "plan: too many attended rows";
      return false;
    }
    p.k_s[s] = k_per_seq[s];
    p.n_kv[s] = (int)nkv;
    p.n_tiles[s] = (int)((nkv + kDecodeTile - 1) / kDecodeTile);
    max_tiles = std::max(max_tiles, p.n_tiles[s]);
  }
  auto splits_for = [&](int s, int tps) { return (p.n_tiles[s] + tps - 1) / tps; };
  bool ws_fits = dtype == 1 && ws_allowed;
  for (int s = 0; s < n_seq; ++s) ws_fits = ws_fits && (int64_t)p.k_s[s] * (b + 1) <= kWsMaxPoolRows;
  // the decode without splits, costed like the split plan below (per launch
  // of kMaxSeqPerLaunch sequences, rounds of one workgroup per CU)
  auto ws_cost_us = [&]() {
    const int64_t q_blocks = (q_rows + kDecodeRowsBf16Ws - 1) / kDecodeRowsBf16Ws;
    double t = 0.0;
    for (int s0 = 0; s0 < n_seq; s0 += kMaxSeqPerLaunch) {
      const int s1 = std::min(n_seq, s0 + kMaxSeqPerLaunch);
      int longest = 1;
      for (int s = s0; s < s1; ++s) longest = std::max(longest, (p.n_kv[s] + 31) / 32);
      const double rounds = std::ceil((double)(s1 - s0) * h_kv * q_blocks / n_cu);
      t += rounds * (kWsFixedUs + kWsRoundUs * ((longest + 7) / 8));
    }
    return t;
  };
  // the decode without kv splits: one workgroup per (sequence, kv head, 32
  // query rows) over every kv row, no partials and no workspace
  auto ws_plan = [&]() {
    p.ws = true;
    p.q_rows_per_wg = kDecodeRowsBf16Ws;
    p.q_tiles = (int)((q_rows + kDecodeRowsBf16Ws - 1) / kDecodeRowsBf16Ws);
    p.splits.assign(n_seq, 1);
    p.tiles_per_split = p.n_tiles;
    p.part_off.assign(n_seq, 0);
    p.lse_off.assign(n_seq, 0);
    p.total_workgroups = (int64_t)n_seq * h_kv * p.q_tiles;
    *plan = std::move(p);
    return true;
  };
  if (force_rows == kDecodeRowsBf16Ws) {
    if (dtype != 1 || num_splits > 1 || (merge != 0 && merge != 1)) {
      *err = "plan: the 32-row decode is bf16 only, without splits or a merge option";
      return false;
    }
    if (!ws_fits) {
      *err = "plan: the 32-row decode holds at most 4864 pool rows per sequence, and a pool and response "
             "rows of under 4 GiB each";
      return false;
    }
    return ws_plan();
  }

  // (query rows per workgroup, workgroups resident per CU) candidates
  struct Shape { int rows, resident; };
  const Shape bf16_shapes[2] = {{kDecodeRowsBf16Large, kResidentBf16Large},
                                {kDecodeRowsBf16Small, kResidentBf16Small}};
  const Shape f32_shapes[1] = {{kDecodeRowsF32, kResidentF32}};
  const Shape* shapes = dtype == 1 ? bf16_shapes : f32_shapes;
  int n_shapes = dtype == 1 ? 2 : 1;
  if (force_rows > 0) {          // a forced workgroup shape (the caller checked it exists)
    for (int i = 0; i < n_shapes; ++i)
      if (shapes[i].rows == force_rows) {
        shapes += i;
        break;
      }
    n_shapes = 1;
  }

  p.splits.assign(n_seq, 1);
  p.tiles_per_split.assign(n_seq, 1);
  if (num_splits > 0) {
    p.q_rows_per_wg = shapes[0].rows;
    for (int s = 0; s < n_seq; ++s) {
      const int want = std::min(num_splits, p.n_tiles[s]);
      const int tps = (p.n_tiles[s] + want - 1) / want;
      p.tiles_per_split[s] = tps;
      p.splits[s] = splits_for(s, tps);
    }
  } else {
    double best = 1e300;
    int best_tps = max_tiles, best_rows = shapes[0].rows;
    for (int si = 0; si < n_shapes; ++si) {
      const int64_t q_tiles = (q_rows + shapes[si].rows - 1) / shapes[si].rows;
      const double slots = (double)n_cu * shapes[si].resident;
      for (int tps = max_tiles; tps >= 1; --tps) {
        // the sequences run in launches of kMaxSeqPerLaunch, one after the
        // other: each launch's rounds, longest split and merge add up
        double t = 0.0;
        for (int s0 = 0; s0 < n_seq; s0 += kMaxSeqPerLaunch) {
          const int s1 = std::min(n_seq, s0 + kMaxSeqPerLaunch);
          int64_t n_wg = 0;
          int max_splits = 1, longest = 1;
          for (int s = s0; s < s1; ++s) {
            const int ns = splits_for(s, tps);
            max_splits = std::max(max_splits, ns);
            longest = std::max(longest, std::min(tps, p.n_tiles[s]));
            n_wg += (int64_t)h_kv * q_tiles * ns;
          }
          double rounds = std::ceil((double)n_wg / slots);
          if (fused) {
            // every split of a group on one XCD: rounds of the fullest XCD
            std::vector<int> sizes;
            for (int s = s0; s < s1; ++s)
              for (int64_t k = 0; k < (int64_t)h_kv * q_tiles; ++k) sizes.push_back(splits_for(s, tps));
            int32_t bounds[kXcdGroups + 1];
            const double per_xcd = std::max(1.0, std::floor(slots / kXcdGroups));
            rounds = std::max(rounds, std::ceil((double)xcd_partition(sizes, bounds) / per_xcd));
          }
          t += rounds * (longest + kFixedTiles);
          if (max_splits > 1)
            t += fused ? kFusedMergeBase + kFusedMergePerSplit * max_splits : kMergeBase + kMergePerSplit * max_splits;
        }
        if (t < best - 1e-9) {      // strictly better: ties keep fewer splits, larger tiles
          best = t;
          best_tps = tps;
          best_rows = shapes[si].rows;
        }
      }
    }
    p.q_rows_per_wg = best_rows;
    for (int s = 0; s < n_seq; ++s) {
      p.tiles_per_split[s] = best_tps;
      p.splits[s] = splits_for(s, best_tps);
    }
    // the chosen split plan in microseconds, against the decode without
    // splits (bf16, default merge, nothing forced)
    if (ws_fits && force_rows == 0 && merge == kDefaultBf16Merge) {
      const int64_t q_tiles = (q_rows + best_rows - 1) / best_rows;
      const double tile_us = best_rows == kDecodeRowsBf16Large ? kSplitTileUs : kSplitTileSmallUs;
      double split_us = 0.0;
      for (int s0 = 0; s0 < n_seq; s0 += kMaxSeqPerLaunch) {
        const int s1 = std::min(n_seq, s0 + kMaxSeqPerLaunch);
        int64_t n_wg = 0;
        int max_splits = 1, longest = 1;
        for (int s = s0; s < s1; ++s) {
          max_splits = std::max(max_splits, p.splits[s]);
          longest = std::max(longest, std::min(best_tps, p.n_tiles[s]));
          n_wg += (int64_t)h_kv * q_tiles * p.splits[s];
        }
        split_us += std::ceil((double)n_wg / n_cu) * (kSplitWgUs + tile_us * longest);
        if (max_splits > 1) split_us += kSplitMergeUs + kSplitMergePerSplitUs * max_splits;
      }
      if (ws_cost_us() < split_us) return ws_plan();
    }
  }
  p.q_tiles = (int)((q_rows + p.q_rows_per_wg - 1) / p.q_rows_per_wg);
  const int64_t per_split_wg = (int64_t)h_kv * p.q_tiles;

  p.part_off.assign(n_seq, 0);
  p.lse_off.assign(n_seq, 0);
  int64_t part = 0, lse = 0;
  p.total_workgroups = 0;
  // rows of one split's partial: the output rows (separate merge kernel), or
  // every row of the sequence's workgroups, padding included (in-kernel merge)
  const int64_t split_rows = fused ? per_split_wg * p.q_rows_per_wg : (int64_t)l_d * h_q;
  for (int s = 0; s < n_seq; ++s) {
    p.total_workgroups += per_split_wg * p.splits[s];
    if (p.splits[s] > 1) {
      p.part_off[s] = part;
      p.lse_off[s] = lse;
      part += (int64_t)p.splits[s] * split_rows * d;
      lse += (int64_t)p.splits[s] * split_rows;
    }
  }
  p.part_floats = part;
  p.lse_floats = lse;
  // bf16 partial outputs for a separate merge kernel over bf16 inputs;
  // float32 or bf16 (merge 3) for the in-kernel merge; float32 for the f32 path
  p.fused = fused && part > 0;
  p.fused_bf16 = p.fused && merge == kFusedBf16Merge;
  p.sep_f32 = dtype == 1 && merge == kSeparateF32Merge && part > 0;
  p.part_elem_bytes = dtype == 1 && !p.sep_f32 && (!p.fused || p.fused_bf16) ? 2 : 4;
  if (p.fused) {
    const int64_t groups = (int64_t)std::min(n_seq, kMaxSeqPerLaunch) * h_kv * p.q_tiles;
    p.sync_words = 2 + groups * (1 + p.q_rows_per_wg / 32);
    p.sync_bytes = align256(p.sync_words * 4);
  }
  p.workspace_bytes = part ? p.sync_bytes + align256(part * p.part_elem_bytes) + align256(lse * 4) : 0;
  *plan = std::move(p);
  return true;
}

}  // namespace pdllm
