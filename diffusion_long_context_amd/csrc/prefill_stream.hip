// Chunk-local bidirectional attention with per-key window scoring for bf16
// chunks whose K and V do not fit on chip (slot_rows up to 4097: chunk sizes
// 512 .. 4096 plus the BOS row), gfx950 MFMA.
//
// Same results as prefill_bf16.hip (Prefilling-dLLM summary, Methodology 1:
// each chunk, BOS row first, is attended only within itself,
// bidirectionally; Methodology 2: a chunk's rows are ranked by the
// cumulative attention weight they receive from the query tokens; the
// method's trade-off study varies the chunk size):
//   o_chunk[c,r,h] = sum_j softmax_j(scale <q_chunk[c,r,h], K[slot,j,g]>) V[slot,j,g]
//   key_score[c,j] = sum_h sum_w softmax_j(scale <q_win[w,h], K[slot,j,g]>)
// computed in three launches instead of one:
//  1. stream_attn_kernel<D, false>: the chunk rows.  A workgroup takes 256
//     (row, grouped head) pairs of one (chunk, kv head); the slot's K and V
//     stream through double-buffered 64-row LDS tiles under the online
//     softmax of attn_tile.h (the tile loop of the decode kernel, with the
//     rows of a tile read straight from the slot instead of a row table).
//  2. stream_attn_kernel<D, true>: the window rows through the same loop
//     with no V: each row's softmax normaliser in log2 units,
//     n2 = m + log2(l), goes to the workspace.
//  3. window_colsum_kernel<D>: per (chunk, kv head, 128-key tile),
//     S = Q_win K^T on the 32x32x16 MFMA with the keys across lanes, so the
//     exact weights p = 2^(s sl2 - n2) (float32) of a key add up inside a
//     lane; one partial row per (chunk, kv head), in a fixed order.
// The finalize kernel (prefill_bf16.hip) then adds the kv heads in order.
#include "attn_tile.h"
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;                  // kv rows per tile
constexpr int kRows = 32 * kWaves;         // query rows per workgroup

template <int D>
struct StreamSmem {
  static constexpr int KP = D + 8;         // K pitch (elements): 8-row 16-byte reads conflict-free
  static constexpr int VP = D + 32;        // V pitch (elements): transposing reads conflict-free
  uint16_t k[2][kTile * KP];               // double-buffered tiles, both row-major
  uint16_t v[2][kTile * VP];
};

template <int D, bool WIN>
__global__ __launch_bounds__(kThreads) void stream_attn_kernel(const PrefillArgs a, int n_qt) {
  __shared__ StreamSmem<D> sm;
  constexpr int KP = StreamSmem<D>::KP, VP = StreamSmem<D>::VP;
  using Attn = WaveAttn<D, KP, VP>;
  constexpr int DC = Attn::DC, DB = Attn::DB;
  constexpr int TPR = D / 8;               // loader threads per kv row (16 B each)
  constexpr int RPT = kTile * TPR / kThreads;   // kv rows per loader thread
  static_assert(RPT == 1 || RPT == 2, "loader mapping");
  constexpr int STAGES = 2;
  constexpr int NK = kTile / 32;

  // ---- work item (chunk, kv head, query tile); query tiles vary fastest,
  // so the workgroups reading one slot's K/V sit on one XCD and share its L2
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = wg % n_qt;
  const int cg = wg / n_qt;
  const int g = cg % a.h_kv, c = cg / a.h_kv;
  const int R = a.slot_rows, G = a.group;  // R: the layout's rows per chunk
  // rows this chunk holds (a partial last chunk holds fewer); past Rc no key
  // or query row takes part
  const int Rc = a.chunk_rows != nullptr ? min(max(a.chunk_rows[c], 1), R) : R;
  const int n_rows = (WIN ? a.w : Rc) * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lc = lane & 31, lj = lane >> 5;
  const int64_t base = (int64_t)a.chunk_slot[c] * a.ps_slot + (int64_t)g * a.ps_head;
  const uint16_t* pk = static_cast<const uint16_t*>(a.pool_k) + base;
  const uint16_t* pv = static_cast<const uint16_t*>(a.pool_v) + base;
  if constexpr (WIN) {
    if (!chunk_scored(a, c)) return;        // a chunk top-K does not select (uniform)
  }

  // ---- queries (B operand of S^T); pairs past the end clamp to the last one
  const int xq = qt * kRows + wave * 32 + lc;
  const int x = min(xq, n_rows - 1);
  const int r = x / G, h = g * G + (x - r * G);
  bf16x8 qf[DC];
  {
    const uint16_t* src = WIN ? static_cast<const uint16_t*>(a.q_win) +
                                    ((int64_t)(c / a.chunks_per_win) * a.w + r) * a.h_q * D
                              : static_cast<const uint16_t*>(a.q_chunk) + ((int64_t)c * R + r) * a.h_q * D;
    load_q<DC, 16>(qf, src + (int64_t)h * D + 8 * lj);
  }

  // ---- tile loader.  A thread owns RPT consecutive kv rows x 8 d values of
  // a tile.  Load unit u carries K of tile u and V of tile u-1 (tile numbers
  // clamped to the slot, rows clamped to its last row, so every load reads
  // valid data); the window pass has no V.
  const int n_tiles = (Rc + kTile - 1) / kTile;
  // a last tile holding a single row (Rc = 64 k + 1, as for C + 1 rows) is a
  // one-row update after the MFMA tiles, not a 64-row tile with 63 masked rows
  const bool one_row = Rc % kTile == 1;
  const int n_mt = one_row ? n_tiles - 1 : n_tiles;   // tiles through the MFMA loop
  const int ld_d0 = 8 * (tid % TPR);
  const int ld_r0 = RPT * (tid / TPR);
  u32x4 kreg[STAGES][RPT], vreg[STAGES][RPT];
  auto load_unit = [&](int set, int u) {
    const int tk = min(u, n_tiles - 1), tv = min(max(u - 1, 0), n_tiles - 1);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int rk = min(tk * kTile + ld_r0 + i, Rc - 1);
      kreg[set][i] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(
          (gptr16)(pk + (int64_t)rk * a.ps_row + ld_d0));
      if constexpr (!WIN) {
        const int rv = min(tv * kTile + ld_r0 + i, Rc - 1);
        vreg[set][i] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(
            (gptr16)(pv + (int64_t)rv * a.ps_row + ld_d0));
      }
    }
  };
  auto store_k = [&](int buf, int set) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<u32x4*>(&sm.k[buf][(ld_r0 + i) * KP + ld_d0]) = kreg[set][i];
  };
  auto store_v = [&](int buf, int set) {
    if constexpr (!WIN) {
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        *reinterpret_cast<u32x4*>(&sm.v[buf][(ld_r0 + i) * VP + ld_d0]) = vreg[set][i];
    }
  };

  Attn at;
  at.init();
  const float sl2 = a.scale_log2;
  const uint16_t* k_base = &sm.k[0][0] + lc * KP + 8 * lj;
  const uint16_t* v_base = &sm.v[0][0] + v_lane_offset(lane, VP);

  // ---- prologue: K and V of tile 0 and K of tile 1 into LDS, units 2 and 3
  // in flight, S^T of tile 0 computed
  load_unit(0, 0);
  load_unit(1, 1);
  store_k(0, 0);
  store_v(0, 0);
  store_k(1, 1);
  load_unit(0, 2);
  load_unit(1, 3);
  __syncthreads();
  f32x16 sc_a[NK], sc_b[NK];
  at.template qk<NK>(sc_a, k_base, qf);
  __syncthreads();                         // K buffer 0 is rewritten in iteration 0

  // ---- main loop.  Iteration u stores unit u+2 (K of tile u+2 into K buffer
  // u & 1, whose tile u was read in iteration u-1; V of tile u+1 into V
  // buffer (u+1) & 1, last read by tile u-1), issues the loads of unit u+4
  // into the staging set just freed, then runs the softmax of tile u with
  // the S^T MFMAs of tile u+1 interleaved, and the PV of tile u.  Every
  // iteration issues exactly one unit's loads and the two halves of the
  // loop body are unconditional, so the wait before a store covers only the
  // loads issued two iterations earlier.  One barrier per tile.
  auto iter = [&](int u, f32x16 (&cur)[NK], f32x16 (&nxt)[NK]) {
    const int set = u % STAGES;
    if (u + 2 < n_tiles) store_k(u & 1, set);
    if (u + 1 < n_tiles) store_v((u + 1) & 1, set);
    load_unit(set, u + 4);
    bf16x8 pf[2 * NK];
    at.template prep<NK>(cur, sl2, Rc - u * kTile, lj);
    if (u + 1 < n_mt)
      at.template exp_qk<NK, true>(cur, pf, nxt, k_base + ((u + 1) & 1) * (kTile * KP), qf, sl2);
    else
      at.template exp_qk<NK, false>(cur, pf, nxt, nullptr, qf, sl2);
    if constexpr (!WIN)
      at.template pv<NK>(pf, v_base + (u & 1) * (kTile * VP), min(2 * NK, (Rc - u * kTile + 15) >> 4));
    __syncthreads();
  };
  {
    int u = 0;
    for (; u + 1 < n_mt; u += 2) {
      iter(u, sc_a, sc_b);
      iter(u + 1, sc_b, sc_a);
    }
    if (u < n_mt) iter(u, sc_a, sc_b);
  }
  // the single-row tile n_mt: its K (and V) went to buffer n_mt & 1 in the
  // prologue or in iterations n_mt - 2 (K) and n_mt - 1 (V), before the last
  // barrier
  if (one_row)
    at.template one_row<!WIN>(&sm.k[n_mt & 1][8 * lj], v_base + (n_mt & 1) * (kTile * VP), qf, sl2, lj);

  // ---- epilogue (lanes lc and lc + 32 hold halves of the same query row)
  const float l = at.row_sum();
  if constexpr (!WIN) {
    // clamped pairs store the same bytes as the pair they copy
    store_o_bf16<DB>(static_cast<uint16_t*>(a.o_chunk) + (((int64_t)c * R + r) * a.h_q + h) * D + 8 * lj,
                     at.acc, 1.f / l);
  } else {
    // rows padded to a multiple of 32; the padding holds +inf (weight 0)
    const int n_pad = (n_rows + 31) & ~31;
    if (lj == 0 && xq < n_pad)
      a.win_norm[((int64_t)c * a.h_kv + g) * n_pad + xq] = xq < n_rows ? at.m_run + __log2f(l) : INFINITY;
  }
}

constexpr int kColKeys = 128;              // keys per window_colsum workgroup
constexpr int kColWaves = 4;

// Per-key window weights of one (chunk, kv head, 128-key tile):
// part[c][g][j] = sum over window rows x (row x / G, head g G + x % G) of
// 2^(scale_log2 <q_win[w,h], K[j]> - win_norm[c][g][x]).
template <int D>
__global__ __launch_bounds__(64 * kColWaves) void window_colsum_kernel(const PrefillArgs a, int n_kt) {
  constexpr int KP = D + 8;
  constexpr int DC = D / 16;
  constexpr int NB = kColKeys / 32;        // 32-key blocks
  constexpr int TPR = D / 8;
  constexpr int kLoads = kColKeys * TPR / (64 * kColWaves);
  __shared__ __attribute__((aligned(16))) uint16_t ks[kColKeys * KP];
  __shared__ float red[kColWaves][kColKeys];

  const int kt = blockIdx.x % n_kt;
  const int cg = blockIdx.x / n_kt;
  const int g = cg % a.h_kv, c = cg / a.h_kv;
  const int R = a.slot_rows, G = a.group;
  const int Rc = a.chunk_rows != nullptr ? min(max(a.chunk_rows[c], 1), R) : R;
  const int n_rows = a.w * G;
  const int n_qb = (n_rows + 31) / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lc = lane & 31, lj = lane >> 5;
  const int j0 = kt * kColKeys;
  if (!chunk_scored(a, c)) return;          // a chunk top-K does not select (uniform)

  // ---- stage the key tile; rows past the chunk clamp to its last row
  // (their sums are written as 0).  All loads go out before the first store.
  {
    const uint16_t* pk = static_cast<const uint16_t*>(a.pool_k) + (int64_t)a.chunk_slot[c] * a.ps_slot +
                         (int64_t)g * a.ps_head;
    u32x4 kr[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = tid + i * 64 * kColWaves;
      const int rr = e / TPR, d0 = 8 * (e - rr * TPR);
      kr[i] = *reinterpret_cast<const u32x4*>(pk + (int64_t)min(j0 + rr, Rc - 1) * a.ps_row + d0);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int e = tid + i * 64 * kColWaves;
      const int rr = e / TPR, d0 = 8 * (e - rr * TPR);
      *reinterpret_cast<u32x4*>(&ks[rr * KP + d0]) = kr[i];
    }
  }
  __syncthreads();

  const uint16_t* qw = static_cast<const uint16_t*>(a.q_win) + (int64_t)(c / a.chunks_per_win) * a.w * a.h_q * D;
  const float* wn = a.win_norm + ((int64_t)c * a.h_kv + g) * (n_qb * 32);
  const uint16_t* k_lane = &ks[lc * KP + 8 * lj];
  const float sl2 = a.scale_log2;
  float colsum[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) colsum[kb] = 0.f;
  // window blocks of 32 rows go to the waves round-robin (a fixed order)
  for (int b = wave; b < n_qb; b += kColWaves) {
    bf16x8 qa[DC];                         // A operand: lane row lc, d = 16 dc + 8 lj ..
    {
      const int x = min(b * 32 + lc, n_rows - 1);
      const int w = x / G, h = g * G + (x - w * G);
      load_q<DC, 16>(qa, qw + ((int64_t)w * a.h_q + h) * D + 8 * lj);
    }
    // lane (lc, lj) receives rows 8 m + 4 lj + t (i = 4 m + t) of key
    // column lc; their normalisers (+inf on padding rows)
    f32x4 nb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) nb[m] = *reinterpret_cast<const f32x4*>(wn + b * 32 + 8 * m + 4 * lj);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      f32x16 s = mfma32x32x16(qa[0], *reinterpret_cast<const bf16x8*>(k_lane + 32 * kb * KP), f32x16{});
#pragma unroll
      for (int dc = 1; dc < DC; ++dc)
        s = mfma32x32x16(qa[dc], *reinterpret_cast<const bf16x8*>(k_lane + 32 * kb * KP + 16 * dc), s);
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) t += __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -nb[i >> 2][i & 3]));
      colsum[kb] += t;
    }
  }
  // lanes lc and lc + 32 hold the same key (different rows); then the waves
  // in order
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    const float v = sum_halves(colsum[kb]);
    if (lj == 0) red[wave][32 * kb + lc] = v;
  }
  __syncthreads();
  if (tid < kColKeys && j0 + tid < R) {    // keys past Rc (a partial chunk) score 0
    float s = red[0][tid];
#pragma unroll
    for (int wv = 1; wv < kColWaves; ++wv) s += red[wv][tid];
    a.part_score[((int64_t)c * a.h_kv + g) * R + j0 + tid] = j0 + tid < Rc ? s : 0.f;
  }
}

template <int D>
int stream_launch(const PrefillArgs& a, void* stream) {
  const hipStream_t st = (hipStream_t)stream;
  const int R = a.slot_rows, G = a.group;
  const int qt_c = (R * G + kRows - 1) / kRows;
  const int qt_w = (a.w * G + kRows - 1) / kRows;
  const int pairs = a.n_chunks * a.h_kv;
  hipLaunchKernelGGL((stream_attn_kernel<D, false>), dim3(pairs * qt_c), dim3(kThreads), 0, st, a, qt_c);
  hipLaunchKernelGGL((stream_attn_kernel<D, true>), dim3(pairs * qt_w), dim3(kThreads), 0, st, a, qt_w);
  const int n_kt = (R + kColKeys - 1) / kColKeys;
  hipLaunchKernelGGL((window_colsum_kernel<D>), dim3(pairs * n_kt), dim3(64 * kColWaves), 0, st, a, n_kt);
  return (int)hipGetLastError();
}

}  // namespace

int launch_prefill_stream(const PrefillArgs& a, int d, void* stream) {
  if (a.n_chunks == 0) return (int)hipSuccess;
  if (d == 128) return stream_launch<128>(a, stream);
  if (d == 64) return stream_launch<64>(a, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace pdllm
