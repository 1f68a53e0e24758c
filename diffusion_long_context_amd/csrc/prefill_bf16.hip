// Chunk-local bidirectional attention with fused per-key window scoring,
// bf16 inputs, gfx950 MFMA.
//
// What it computes (Prefilling-dLLM summary, Methodology 1: every chunk,
// BOS row first, is attended only within itself, bidirectionally;
// Methodology 2: a chunk's rows are ranked by the cumulative attention weight
// they receive from the query tokens):
//   o_chunk[c,r,h]   = sum_j softmax_j(scale <q_chunk[c,r,h], K[slot,j,g]>) V[slot,j,g]
//   part[c,g,p,j]    = sum over the window rows wave p handled (heads h in
//                      group g) of softmax_j(scale <q_win[w,h], K[slot,j,g]>)
// and the finalize kernel sums part over g, then p, in a fixed order into key_score.
//
// Design for CDNA4: one workgroup of 8 wavefronts per (chunk, kv head).  The
// chunk's whole K and V (both row-major) for that kv head are staged into LDS
// once -- up to 288 rows x 128 d x 2 tensors, about 158 KiB of the 160 KiB --
// and every query row of the G grouped heads streams past it, so
// HBM traffic is one read of Q and the pool slot and one write of O.
// Wavefronts take 32-row blocks round-robin, with the next block's queries
// loaded while the current one computes: chunk-row blocks run the shared
// attention step (attn_tile.h, 32x32x16 MFMA) over 64-row kv steps;
// window-row blocks run S = Q K^T on the 16x16x32 MFMA (which leaves each
// lane one key column), an exact row softmax over all keys, and accumulate
// each key's weight in registers.  Each wave writes its per-key sums as one
// partial row; the finalize kernel adds them over waves and kv heads in a
// fixed order.
#include "attn_tile.h"
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 288;              // slot_rows <= 257, padded to 32
constexpr int kMaxKb = kMaxRows / 16;      // 16-row kv blocks

template <int D>
struct PSmem {
  static constexpr int KP = D + 8;          // K pitch (elements): 8-row 16-byte reads conflict-free
  static constexpr int VP = D + 16;         // V pitch (elements): transposing reads conflict-free
  uint16_t k[kMaxRows * KP];                // both row-major
  uint16_t v[kMaxRows * VP];
  int next_item;                            // dynamic hand-out of chunk-row items
  int chunk_pick;                           // the workgroup's chunk, when chosen by rank
};


// NKB = 16-row kv blocks of the chunk padded to 32 rows (compile-time, so
// every loop over keys is static).  ONE_ROW: the layout has a single row
// past its last 64-row block (R = 64 (NKB / 4) + 1, as for R = C + 1).
template <int D, int NKB, bool ONE_ROW>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(const PrefillArgs a) {
  static_assert(NKB % 2 == 0 && NKB <= kMaxKb, "kv blocks");
  static_assert(!ONE_ROW || NKB % 4 == 2, "a single row past the 64-row blocks");
  __shared__ PSmem<D> sm;
  constexpr int KP = PSmem<D>::KP, VP = PSmem<D>::VP;
  constexpr int DC = D / 32;               // 32-wide d chunks (16x16x32 MFMA)
  constexpr int TPR = D / 8;
  static_assert(kThreads % TPR == 0, "loader mapping");

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // ---- the work item (chunk, kv head).  When only the chunks top-K keeps
  // are scored and a.rank_order is set, workgroups take chunks in
  // descending score order --
  // workgroup (r n_seq + s) h_kv + g takes the chunk of rank r in sequence s
  // (rank_key order, the order top-K selects by) -- so the scored chunks,
  // which carry the window work, all run in the first round of workgroups
  // and no CU draws two of them.  A chunk's work does not depend on which
  // workgroup runs it.  The ranks are counted in LDS (the K and V areas,
  // before the staging), with up to four threads per candidate, each over a
  // share of the keys.
  const int g = blockIdx.x % a.h_kv;
  int c = blockIdx.x / a.h_kv;
  bool scored = true;
  if (a.sel_score != nullptr) {
    const int nps = a.sel_per_seq;
    if (a.rank_order) {
      const int n_seq = a.n_chunks / nps;
      const int r = c / n_seq, sq = c - r * n_seq;
      const float* row = a.sel_score + (int64_t)sq * nps;
      uint64_t* keys = reinterpret_cast<uint64_t*>(&sm.k[0]);
      int* cnt = reinterpret_cast<int*>(&sm.v[0]);
      for (int j = tid; j < nps; j += kThreads) {
        keys[j] = rank_key(row[j], (uint32_t)j);
        cnt[j] = 0;
      }
      __syncthreads();
      static_assert(kPrefillRankChunks <= kThreads, "one thread per candidate at least");
      {
        const int P = nps <= kThreads / 4 ? 4 : nps <= kThreads / 2 ? 2 : 1;   // threads per candidate
        const int nj = kThreads / P;
        const int j = tid % nj, part = tid / nj;
        if (j < nps) {
          const uint64_t mine = keys[j];
          const int lo = part * nps / P, hi = (part + 1) * nps / P;
          int larger = 0;
          for (int i = lo; i < hi; ++i) larger += keys[i] > mine ? 1 : 0;
          atomicAdd(&cnt[j], larger);
        }
      }
      __syncthreads();
      for (int j = tid; j < nps; j += kThreads)
        if (cnt[j] == r) sm.chunk_pick = j;
      __syncthreads();
      c = sq * nps + sm.chunk_pick;        // (the K / V areas' last reads were before the barrier)
      scored = r < a.sel_k[sq];
    } else {
      scored = chunk_scored(a, c);
    }
  }
  const int R = a.slot_rows;               // the layout's rows per chunk
  // rows this chunk holds (a partial last chunk holds fewer): keys and
  // query rows past Rc take no part
  const int Rc = a.chunk_rows != nullptr ? min(max(a.chunk_rows[c], 1), R) : R;
  constexpr int rpad = 16 * NKB;
  const int slot = a.chunk_slot[c];
  const int lr = lane & 15, lj = lane >> 4;  // 16x16 layout (window items)
  const int G = a.group;
  const float sl2 = a.scale_log2;
  const int n_rows_w = a.w * G;
  const int n_wb = (n_rows_w + 31) / 32;
  const uint16_t* qw = static_cast<const uint16_t*>(a.q_win) +
                       (int64_t)(c / a.chunks_per_win) * a.w * a.h_q * D;
  // Window items are 32 (window row, grouped head) pairs, wave w taking
  // w, w + 8, ...; rows past the end clamp to the last row (their weight is
  // zero), so every fetch is unconditional and the memory waits stay exact.
  auto fetch_w = [&](int witem, bf16x8 (&qf)[2][DC]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int x = min(witem * 32 + 16 * b + lr, n_rows_w - 1);
      const int r = x / G, h = g * G + (x - r * G);
      load_q<DC, 32>(qf[b], qw + ((int64_t)r * a.h_q + h) * D + 8 * lj);
    }
  };
  // the first window item's queries load together with the staging
  bf16x8 qw_cur[2][DC];
  if (n_wb > 0) fetch_w(min(wave, n_wb - 1), qw_cur);

  // ---- stage the chunk's K and V (rows >= Rc are zero); every load is issued
  // before the first LDS store so the staging costs one memory round trip
  {
    const uint16_t* pk = static_cast<const uint16_t*>(a.pool_k);
    const uint16_t* pv = static_cast<const uint16_t*>(a.pool_v);
    const int64_t base = (int64_t)slot * a.ps_slot + (int64_t)g * a.ps_head;
    const int d0 = 8 * (tid % TPR);
    constexpr int kRowsPerPass = 4 * (kThreads / TPR);
    constexpr int kPasses = (rpad + kRowsPerPass - 1) / kRowsPerPass;
    const int r_first = 4 * (tid / TPR);
    u32x4 kr[kPasses][4], vr[kPasses][4];
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r_first + ps * kRowsPerPass + i;
        if (r < Rc) {
          const int64_t off = base + (int64_t)r * a.ps_row + d0;
          kr[ps][i] = *reinterpret_cast<const u32x4*>(pk + off);
          vr[ps][i] = *reinterpret_cast<const u32x4*>(pv + off);
        } else {
          kr[ps][i] = vr[ps][i] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r_first + ps * kRowsPerPass + i;
        if (r < rpad) {
          *reinterpret_cast<u32x4*>(&sm.k[r * KP + d0]) = kr[ps][i];
          *reinterpret_cast<u32x4*>(&sm.v[r * VP + d0]) = vr[ps][i];
        }
      }
    if (tid == 0) sm.next_item = kWaves;  // items 0..kWaves-1 go to waves 0..kWaves-1
  }
  __syncthreads();

  const int n_rows_c = Rc * G;
  const int n_cb = (n_rows_c + 31) / 32;
  const uint16_t* qc = static_cast<const uint16_t*>(a.q_chunk) + (int64_t)c * R * a.h_q * D;
  uint16_t* oc = static_cast<uint16_t*>(a.o_chunk) + (int64_t)c * R * a.h_q * D;
  using Attn = WaveAttn<D, KP, VP>;
  constexpr int DC32 = Attn::DC;            // 16-wide d chunks (32x32x16 MFMA)
  const int lc = lane & 31, lh = lane >> 5; // 32x32 layout: query column, half
  const uint16_t* k_lane = &sm.k[lc * KP + 8 * lh];
  const uint16_t* v_lane = &sm.v[v_lane_offset(lane, VP)];

  // Query rows past the end (the last item's tail, or an item number past
  // the last one) are clamped to the last row: those lanes compute the same
  // output as the lane that owns it and store the same bytes to the same
  // address, so loads and stores need no branch and the memory counter
  // waits stay exact (the next item's query prefetch is not waited on
  // together with this item's stores).
  auto row_of = [&](int item) { return min(item * 32 + lc, n_rows_c - 1); };
  auto fetch_c = [&](int item, bf16x8 (&qf)[DC32]) {
    const int x = row_of(item);
    const int r = x / G, h = g * G + (x - r * G);
    load_q<DC32, 16>(qf, qc + ((int64_t)r * a.h_q + h) * D + 8 * lh);
  };
  auto attend = [&](int item, const bf16x8 (&qf)[DC32]) {
    __builtin_amdgcn_sched_barrier(0);     // keep items apart: no cross-item hoisting
    Attn at;
    at.init();
    // 64-row steps over rows [0, 64 (NKB / 4)), masked at Rc; when
    // NKB % 4 == 2 the remaining rows run as one 32-row step, or, when the
    // layout has a single row there (R = C + 1 for C a multiple of 64), as a
    // one-row update.  A step wholly past Rc (a partial chunk) is masked
    // throughout; a one-row update past Rc is skipped.
    //
    // The 64-row steps are software-pipelined: step st's softmax runs with
    // the S^T MFMAs of step st + 1 interleaved (in a fixed, fenced order),
    // then its PV over all four 16-row pieces.  Pieces past Rc hold zero V
    // rows (staged so up to rpad) and p = 0, so they add exactly nothing.
    constexpr int n_full = NKB / 4;
    if constexpr (n_full > 0) {
      f32x16 sc[2][2];
      at.template qk<2>(sc[0], k_lane, qf);
#pragma unroll
      for (int st = 0; st < n_full; ++st) {
        f32x16 (&cur)[2] = sc[st & 1];
        f32x16 (&nxt)[2] = sc[(st + 1) & 1];
        bf16x8 pf[4];
        // the softmax (with the next step's S^T MFMAs) at raised wave
        // priority, the PV MFMAs at the default: a wave in its softmax
        // issues first, so its VALU work fills the other wave's MFMA time
        __builtin_amdgcn_s_setprio(3);
        at.template prep<2>(cur, sl2, max(Rc - st * 64, 0), lh);
        if (st + 1 < n_full)
          at.template exp_qk<2, true, 2>(cur, pf, nxt, k_lane + (st + 1) * 64 * KP, qf, sl2);
        else
          at.template exp_qk<2, false>(cur, pf, nxt, nullptr, qf, sl2);
        __builtin_amdgcn_s_setprio(0);
        at.template pv<2, true>(pf, v_lane + st * 64 * VP);
      }
    }
    if constexpr (NKB % 4 == 2) {
      constexpr int kv0 = 64 * n_full;
      if constexpr (ONE_ROW) {
        if (Rc > kv0) at.one_row(&sm.k[kv0 * KP + 8 * lh], v_lane + kv0 * VP, qf, sl2, lh);
      } else {
        at.template step<1>(k_lane + kv0 * KP, v_lane + kv0 * VP, qf, sl2, max(Rc - kv0, 0), lh);
      }
    }
    const float l = at.row_sum();
    const int x = row_of(item);
    const int r = x / G, h = g * G + (x - r * G);
    store_o_bf16<Attn::DB>(oc + ((int64_t)r * a.h_q + h) * D + 8 * lh, at.acc, 1.f / l);
  };
  // ---- phase 1: window-row items, a fixed round-robin over waves (so the
  // per-key sums are added in a fixed order).  S = Q K^T on the 16x16x32 MFMA
  // leaves lane (lr, lj) the keys 16 kb + lr of rows 4 lj + e, so each key's
  // weight accumulates in registers with no per-item shuffles.
  float colsum[NKB];                       // lane: key 16 kb + lr, summed over its window rows
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) colsum[kb] = 0.f;
  const uint16_t* k16 = &sm.k[lr * KP + 8 * lj];
  // (a chunk that top-K does not select is not scored when only the
  // selected ones are asked for: its waves go straight to the chunk items)
  for (int witem = wave; scored && witem < n_wb; witem += kWaves) {
    const int first = witem * 32;
    bf16x8 qf[2][DC];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qf[b][dc] = qw_cur[b][dc];
    // the next item's queries (this one's again on the last pass) load
    // while this one computes
    fetch_w(min(witem + kWaves, n_wb - 1), qw_cur);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 ninf = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x4 sw[NKB];
      // key blocks in pairs; the scheduling barrier keeps at most one pair's
      // K fragments in registers
#pragma unroll
      for (int kb = 0; kb < NKB; kb += 2) {
        bf16x8 kf[2][DC];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int dc = 0; dc < DC; ++dc)
            kf[u][dc] = *reinterpret_cast<const bf16x8*>(k16 + 16 * (kb + u) * KP + 32 * dc);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          sw[kb + u] = mfma16x16x32(qf[b][0], kf[u][0], zero);
#pragma unroll
          for (int dc = 1; dc < DC; ++dc) sw[kb + u] = mfma16x16x32(qf[b][dc], kf[u][dc], sw[kb + u]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // keys past Rc (only in the last two blocks unless the chunk is partial;
      // the first test is workgroup-uniform)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        if (16 * kb + 15 >= Rc && 16 * kb + lr >= Rc) sw[kb] = ninf;
      float mx[4], sum[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float m = max_f(sw[0][e], sw[1][e]);
#pragma unroll
        for (int kb = 2; kb < NKB; kb += 2) m = max_f(max_f(m, sw[kb][e]), sw[kb + 1][e]);
        mx[e] = -row16_max(m) * sl2;
        sum[e] = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sw[kb][e], sl2, mx[e]));
          sw[kb][e] = p;
          sum[e] += p;
        }
      float wgt[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = row16_sum(sum[e]);
        wgt[e] = first + 16 * b + 4 * lj + e < n_rows_w ? __builtin_amdgcn_rcpf(t) : 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        colsum[kb] = fmaf(sw[kb][3], wgt[3], fmaf(sw[kb][2], wgt[2], fmaf(sw[kb][1], wgt[1],
                          fmaf(sw[kb][0], wgt[0], colsum[kb]))));
    }
  }

  // per-key sums of this wave: across its 4 lane groups, then one row of
  // the partial key scores (the finalize kernel adds the waves and kv heads
  // in a fixed order)
  if (scored) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      colsum[kb] = wave_xor_sum(colsum[kb], 16);
      colsum[kb] = wave_xor_sum(colsum[kb], 32);
    }
    float* part = a.part_score + (((int64_t)c * a.h_kv + g) * a.parts + wave) * R;
    if (lj == 0) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        if (16 * kb + lr < R) part[16 * kb + lr] = colsum[kb];
    }
  }

  // ---- phase 2: chunk-row items, 32 (row, grouped head) pairs each, handed
  // out dynamically (each item's output does not depend on which wave runs
  // it), which evens out the window items and the waves' unequal issue
  // priority; the next item's queries load while the current item computes
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(&sm.next_item, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  // The first pair is peeled so that the loop head sees the same pending
  // memory operations from both paths: the loads of one item's queries,
  // the stores of the item before it, the loads of the next item's queries.
  if (wave < n_cb) {
    bf16x8 qa[DC32], qb[DC32];
    int item = wave;
    fetch_c(item, qa);
    int nxt = grab();
    fetch_c(nxt, qb);
    attend(item, qa);
    if (nxt < n_cb) {
      item = grab();
      fetch_c(item, qa);
      while (true) {
        attend(nxt, qb);
        if (item >= n_cb) break;
        nxt = grab();
        fetch_c(nxt, qb);
        attend(item, qa);
        if (nxt >= n_cb) break;
        item = grab();
        fetch_c(item, qa);
      }
    }
  }
}

// key_score[c][j] = sum over kv heads g = 0 .. h_kv-1 and, inside each, over
// the partial rows p = 0 .. parts-1 (in that order) of part[c][g][p][j].
__global__ __launch_bounds__(256) void score_finalize_kernel(const float* part, int n_chunks,
                                                             int h_kv, int parts, int slot_rows,
                                                             float* key_score) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n_chunks * slot_rows) return;
  const int64_t c = idx / slot_rows, j = idx - c * slot_rows;
  const float* pc = part + c * h_kv * parts * slot_rows + j;
  const int n = h_kv * parts;
  // loads in groups of 16 (all in flight together), added in index order
  constexpr int kGroup = 16;
  float s = 0.f;
  for (int q0 = 0; q0 < n; q0 += kGroup) {
    float x[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) x[u] = q0 + u < n ? pc[(int64_t)(q0 + u) * slot_rows] : 0.f;
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      if (q0 + u < n) s += x[u];
  }
  key_score[idx] = s;
}

template <int D>
int prefill_launch(const PrefillArgs& a, void* stream) {
  const dim3 grid(a.n_chunks * a.h_kv), block(kThreads);
  const hipStream_t st = (hipStream_t)stream;
  // one row past the last 64-row block: the one-row tail instance
  const bool one = a.slot_rows % 64 == 1;
  switch ((a.slot_rows + 31) / 32) {
    case 1: if (one) hipLaunchKernelGGL((prefill_bf16_kernel<D, 2, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((prefill_bf16_kernel<D, 2, false>), grid, block, 0, st, a);
            break;
    case 2: hipLaunchKernelGGL((prefill_bf16_kernel<D, 4, false>), grid, block, 0, st, a); break;
    case 3: if (one) hipLaunchKernelGGL((prefill_bf16_kernel<D, 6, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((prefill_bf16_kernel<D, 6, false>), grid, block, 0, st, a);
            break;
    case 4: hipLaunchKernelGGL((prefill_bf16_kernel<D, 8, false>), grid, block, 0, st, a); break;
    case 5: if (one) hipLaunchKernelGGL((prefill_bf16_kernel<D, 10, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((prefill_bf16_kernel<D, 10, false>), grid, block, 0, st, a);
            break;
    case 6: hipLaunchKernelGGL((prefill_bf16_kernel<D, 12, false>), grid, block, 0, st, a); break;
    case 7: if (one) hipLaunchKernelGGL((prefill_bf16_kernel<D, 14, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((prefill_bf16_kernel<D, 14, false>), grid, block, 0, st, a);
            break;
    case 8: hipLaunchKernelGGL((prefill_bf16_kernel<D, 16, false>), grid, block, 0, st, a); break;
    case 9: if (one) hipLaunchKernelGGL((prefill_bf16_kernel<D, 18, true>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((prefill_bf16_kernel<D, 18, false>), grid, block, 0, st, a);
            break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_prefill_bf16(const PrefillArgs& a, int d, void* stream) {
  if (a.n_chunks == 0) return (int)hipSuccess;
  if (d == 128) return prefill_launch<128>(a, stream);
  if (d == 64) return prefill_launch<64>(a, stream);
  return (int)hipErrorInvalidValue;
}

int launch_score_finalize(const PrefillArgs& a, void* stream) {
  const int64_t n = (int64_t)a.n_chunks * a.slot_rows;
  if (n == 0) return (int)hipSuccess;
  hipLaunchKernelGGL(score_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, a.part_score, a.n_chunks, a.h_kv, a.parts, a.slot_rows,
                     a.key_score);
  return (int)hipGetLastError();
}

}  // namespace pdllm
