// Chunk-sparse decode attention without KV splits, for bf16 inputs on gfx950.
//
// What it computes is what the split decode computes (Prefilling-dLLM
// summary, Methodology 2 and 3, and "Attention kernel optimization"): every
// decode row (token i, query head h) of a sequence attends, without a mask,
// to the BOS row and the kept rows of each selected chunk -- read in place
// from the non-contiguous chunk pool -- followed by the sequence's response
// rows; the output is the softmax-weighted sum of V and, optionally, the
// natural-log normaliser.
//
// Design for CDNA4, for calls whose query rows are too few to fill the GPU
// with large query tiles (a window of a few hundred tokens over one kv head
// gives a few dozen 256-row tiles):
// * One workgroup per (sequence, kv head, 32 query rows) covers every kv row
//   of the sequence, so no partial output is written and no merge kernel
//   runs.  The 8 wavefronts share the 32 query rows and take disjoint 32-row
//   kv tiles (wave w: the tiles n_t-1-w, n_t-9-w, ..., so the response rows,
//   which need no index lookup, come first).
// * A workgroup reads its kv head's rows once; the workgroups of one
//   (sequence, kv head) sit on one XCD and hit its L2.  At 32 query rows per
//   workgroup every CU streams the whole kv head (about 2 KB of K/V per
//   query row), at about 70 GB/s per CU: bound by the wavefronts' own
//   instruction streams (each tile is stored to and read from LDS by one
//   wavefront), near the CU's load rate for gathered rows (75-94 GB/s),
//   not by the MFMAs.
// * Each wavefront gathers its tiles with coalesced 16-byte loads (four
//   256-byte rows per instruction; the MFMA fragment layout would read 32-byte
//   pieces of 32 rows per instruction, which a CU streams at a third of the
//   rate) into staging registers one tile ahead, and stores them into its own
//   LDS tile: no workgroup barrier in the loop.  S^T = K Q^T and
//   O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 (attn_tile.h).
// * The pool rows' addresses come from a row table built once per workgroup
//   in LDS (element offsets / 8, and per-tile masks of absent kept rows),
//   from the index tables or from rows resolved once per prompt
//   (pdllm_resolve_rows).
//   Loads take a scalar base and a 32-bit byte offset, so the pool and the
//   response rows must each span under 4 GiB (the library checks).
// * At the end the 8 online-softmax states are merged in LDS: reference max
//   M = max_w m_w, O = sum_w 2^(m_w - M) O_w, l = sum_w 2^(m_w - M) l_w.
#include "attn_tile.h"
#include "device_common.h"
#include "pdllm_internal.h"

namespace pdllm {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQRows = kDecodeRowsBf16Ws;    // query rows per workgroup
constexpr int kT = 32;                        // kv rows per wavefront tile
constexpr int kFillPerThread = (kWsMaxPoolRows + kThreads - 1) / kThreads;
constexpr int kMaxTiles = kFillPerThread * kThreads / kT;
static_assert(kQRows == 32, "one query column per lane pair");

template <int D>
struct WsSmem {
  static constexpr int KP = D + 8;            // K pitch (elements): fragment reads conflict-free
  static constexpr int VP = D + 16;           // V pitch (elements): transposing reads
  static constexpr int OS = D / 2 + 4;        // merge buffer: floats per lane (padded)
  struct Tiles {
    uint16_t k[kWaves][kT * KP];
    uint16_t v[kWaves][kT * VP];
  };
  struct Merge {
    float o[kWaves][64][OS];                  // wave w's scaled accumulators, lane-major
    float m[kWaves][32];                      // reference max of each query column (log2 units)
    float l[kWaves][32];                      // row sum of each query column
  };
  static_assert(sizeof(Merge) <= sizeof(Tiles), "the merge reuses the tiles' LDS");
  union alignas(16) {
    Tiles t;
    Merge g;
  } u;
  // pool rows of the sequence: element offset / 8 of (slot, row, kv head),
  // in a permuted order inside each 32-row tile (see row_pos)
  int32_t rows[kWsMaxPoolRows];
  uint32_t amask[kMaxTiles];                  // per tile: bit r = row r is an absent kept row
};

// Loader geometry: 16-byte chunks per row, rows per load instruction, load
// instructions per tile and tensor.
template <int D>
struct Geo {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NU = kT / RPI;
};

// Row r of a tile is loaded by the lanes with lane / CPR == r % RPI, in their
// load u = r / RPI; the table keeps a lane's NU rows next to each other.
template <int D>
__device__ __forceinline__ int row_pos(int v) {
  constexpr int RPI = Geo<D>::RPI, NU = Geo<D>::NU;
  const int r = v & (kT - 1);
  return (v - r) + (r % RPI) * NU + r / RPI;
}

// The work item of workgroup `bid`: items are (sequence, kv head, query
// block) with the query block fastest; XCD x (workgroup b runs on XCD b % 8)
// takes the contiguous item range [x per, (x + 1) per), so the workgroups of
// one (sequence, kv head) share an XCD and its L2.
struct WsItem {
  int si, g, qb;
  bool valid;
};
__device__ __forceinline__ WsItem ws_item(const DecodeArgs& a, int bid) {
  const int per = a.grid_wg / kXcdGroups;
  const int item = (bid % kXcdGroups) * per + bid / kXcdGroups;
  WsItem w;
  w.valid = item < a.total_wg;
  const int per_seq = a.h_kv * a.q_tiles;
  w.si = min(item / per_seq, a.n_seq_launch - 1);
  const int rem = item - w.si * per_seq;
  w.g = rem / a.q_tiles;
  w.qb = rem - w.g * a.q_tiles;
  return w;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void decode_ws_kernel(const DecodeArgs a) {
  __shared__ WsSmem<D> sm;
  using G = Geo<D>;
  constexpr int CPR = G::CPR, RPI = G::RPI, NU = G::NU;
  constexpr int KP = WsSmem<D>::KP, VP = WsSmem<D>::VP, OS = WsSmem<D>::OS;
  using Attn = WaveAttn<D, KP, VP>;
  constexpr int DC = Attn::DC, DB = Attn::DB;

  const WsItem w = ws_item(a, blockIdx.x);
  if (!w.valid) return;                      // whole workgroup: no barrier is skipped by part of it
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lc = lane & 31, lj = lane >> 5;
  const int si = w.si, g = w.g, s = a.seq0 + si;
  const int k_s = a.seq[si].k_s, n_kv = a.seq[si].n_kv;
  const int per = a.b + 1, n_pool = k_s * per;
  const int Gq = a.group, rows_total = a.l_d * Gq;
  const uint16_t* pk = static_cast<const uint16_t*>(a.pool_k);
  const uint16_t* pv = static_cast<const uint16_t*>(a.pool_v);
  const uint16_t* rk = static_cast<const uint16_t*>(a.k_resp);
  const uint16_t* rv = static_cast<const uint16_t*>(a.v_resp);

  // queries: B-operand fragments of S^T for query column lc (rows past the
  // end read the last row and are never stored)
  bf16x8 qf[DC];
  {
    const int x = min(w.qb * kQRows + lc, rows_total - 1);
    const int i = x / Gq, h = g * Gq + (x - i * Gq);
    load_q<DC, 16>(qf, static_cast<const uint16_t*>(a.q) + (((int64_t)s * a.l_d + i) * a.h_q + h) * D + 8 * lj);
  }

  // ---- the tile loader: lane (row group lane / CPR, chunk lane % CPR) loads
  // rows RPI u + lane / CPR of the tile, u = 0 .. NU-1
  const int lrow = lane / CPR, lch = 8 * (lane % CPR);
  const int64_t resp_row = (int64_t)a.h_kv * D;             // elements between response rows
  const int64_t resp0 = ((int64_t)s * a.l_d - n_pool) * resp_row + (int64_t)g * D + lch;
  u32x4 ks[NU], vs[NU];
  auto issue = [&](int tt) {
    const int v0 = kT * tt;
    // K and V of a row sit at the same offset from their bases: when a whole
    // tile comes from one source, each row costs one 32-bit byte offset from
    // a scalar base (the pool and the response rows each span under 4 GiB)
    auto load2 = [&](const uint16_t* kb, const uint16_t* vb, uint32_t off_bytes, int u) __attribute__((always_inline)) {
      ks[u] = *(const __attribute__((address_space(1))) u32x4*)(reinterpret_cast<const char*>(kb) + off_bytes);
      vs[u] = *(const __attribute__((address_space(1))) u32x4*)(reinterpret_cast<const char*>(vb) + off_bytes);
    };
    if (v0 + kT <= n_pool) {                 // pool rows only: the row table
      const uint32_t* e = reinterpret_cast<const uint32_t*>(&sm.rows[v0 + lrow * NU]);
#pragma unroll
      for (int u = 0; u < NU; ++u) load2(pk, pv, (e[u] << 4) + 2u * (uint32_t)lch, u);
    } else if (v0 >= n_pool && v0 + kT <= n_kv) {   // response rows only
      const uint32_t off0 = (uint32_t)(2 * (resp0 + (int64_t)(v0 + lrow) * resp_row));
      const uint32_t step = (uint32_t)(2 * RPI * resp_row);
#pragma unroll
      for (int u = 0; u < NU; ++u) load2(rk, rv, off0 + (uint32_t)u * step, u);
    } else {                                  // mixed, or past the last row (clamped to it)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int v = min(v0 + RPI * u + lrow, n_kv - 1);
        const bool pool = v < n_pool;
        const uint32_t off = pool ? (((uint32_t)sm.rows[row_pos<D>(v)]) << 4) + 2u * (uint32_t)lch
                                  : (uint32_t)(2 * (resp0 + (int64_t)v * resp_row));
        load2(pool ? pk : rk, pool ? pv : rv, off, u);
      }
    }
  };

  const int n_t = (n_kv + kT - 1) / kT;
  int t = n_t - 1 - wave;                    // this wavefront's first tile (may be < 0: none)
  // a first tile of response rows needs no row table: its loads go out now
  const bool early = t >= 0 && kT * t >= n_pool;
  if (early) issue(t);

  // ---- the row table of the pool rows (thread tid: rows tid + 512 i); every
  // load of a batch is issued before the first use
  if (n_pool > 0 && a.rows != nullptr) {    // resolved once (pdllm_resolve_rows): one load a row
    const int32_t* rt = a.rows + (int64_t)s * a.rows_stride;
    const uint32_t head8 = (uint32_t)(((int64_t)g * a.ps_head) >> 3);
    int e[kFillPerThread];
#pragma unroll
    for (int i = 0; i < kFillPerThread; ++i)
      e[i] = *(const __attribute__((address_space(1))) int32_t*)(rt + min(tid + kThreads * i, n_pool - 1));
#pragma unroll
    for (int i = 0; i < kFillPerThread; ++i) {
      const int v = tid + kThreads * i;
      if (v < n_pool) sm.rows[row_pos<D>(v)] = (int32_t)(((uint32_t)e[i] & 0x7fffffffu) + head8);
      const uint64_t m = __ballot(v < n_pool && e[i] < 0);
      if (lane == 0) {
        sm.amask[(v - lane) / kT] = (uint32_t)m;
        sm.amask[(v - lane) / kT + 1] = (uint32_t)(m >> 32);
      }
    }
  } else if (n_pool > 0) {
    const int32_t* sel = a.sel_chunk + (int64_t)s * a.k_max;
    int vv[kFillPerThread], cg[kFillPerThread], rr[kFillPerThread];
#pragma unroll
    for (int i = 0; i < kFillPerThread; ++i) {
      vv[i] = min(tid + kThreads * i, n_pool - 1);
      const int k = vv[i] / per;
      rr[i] = vv[i] - k * per;
      cg[i] = *(const __attribute__((address_space(1))) int32_t*)(sel + k);
    }
    int slot[kFillPerThread], kr[kFillPerThread];
#pragma unroll
    for (int i = 0; i < kFillPerThread; ++i) {
      cg[i] = s * a.n_chunks_per_seq + min(max(cg[i], 0), a.n_chunks_per_seq - 1);
      slot[i] = *(const __attribute__((address_space(1))) int32_t*)(a.chunk_slot + cg[i]);
      const int32_t* kp = a.keep_rows != nullptr && rr[i] > 0 ? a.keep_rows + (int64_t)cg[i] * a.b + rr[i] - 1
                                                               : a.idx_dummy;
      kr[i] = *(const __attribute__((address_space(1))) int32_t*)(kp);
    }
#pragma unroll
    for (int i = 0; i < kFillPerThread; ++i) {
      const int v = tid + kThreads * i;
      const bool absent = rr[i] > 0 && a.keep_rows != nullptr && kr[i] < 0;
      const int row = rr[i] == 0 || absent ? 0 : a.compact ? rr[i] : kr[i];
      const int64_t off = (int64_t)slot[i] * a.ps_slot + (int64_t)row * a.ps_row + (int64_t)g * a.ps_head;
      if (v < n_pool) sm.rows[row_pos<D>(v)] = (int32_t)(off >> 3);
      // rows v of this wave span the tiles 2 (wave + 16 i) and 2 (wave + 16 i) + 1
      const uint64_t m = __ballot(v < n_pool && absent);
      if (lane == 0) {
        sm.amask[(v - lane) / kT] = (uint32_t)m;
        sm.amask[(v - lane) / kT + 1] = (uint32_t)(m >> 32);
      }
    }
  }
  __syncthreads();                           // row table ready
  if (t >= 0 && !early) issue(t);

  Attn at;
  at.init();
  const float sl2 = a.scale_log2;
  uint16_t* const k_tile = &sm.u.t.k[wave][0];
  uint16_t* const v_tile = &sm.u.t.v[wave][0];
  const uint16_t* k_lane = k_tile + lc * KP + 8 * lj;
  const uint16_t* v_lane = v_tile + v_lane_offset(lane, VP);

  while (t >= 0) {                           // wave-uniform
    // this tile's staged rows into the wavefront's LDS tile
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int r = RPI * u + lrow;
      *reinterpret_cast<u32x4*>(k_tile + r * KP + lch) = ks[u];
      *reinterpret_cast<u32x4*>(v_tile + r * VP + lch) = vs[u];
    }
    const int tn = t - kWaves;
    if (tn >= 0) issue(tn);                  // the next tile's loads, in flight during this one
    const uint32_t am = kT * t < n_pool ? sm.amask[t] : 0u;
    f32x16 sc[1];
    bf16x8 pf[2];
    at.template qk<1>(sc, k_lane, qf);
    __builtin_amdgcn_s_setprio(3);
    at.template prep<1>(sc, sl2, n_kv - kT * t, lj, 0, (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)am));
    at.template exp_qk<1, false>(sc, pf, sc, nullptr, qf, sl2);
    __builtin_amdgcn_s_setprio(0);
    at.template pv<1>(pf, v_lane);
    t = tn;
  }

  // ---- merge the wavefronts' states (every query column is in every wave)
  const float lw = at.row_sum();
  __syncthreads();                           // every tile loop has ended: the tiles' LDS is reused
  if (lane < 32) {
    sm.u.g.m[wave][lc] = at.m_run;
    sm.u.g.l[wave][lc] = lw;
  }
  __syncthreads();
  float mx = kNoMax;
#pragma unroll
  for (int x = 0; x < kWaves; ++x) mx = max_f(mx, sm.u.g.m[x][lc]);
  {
    const float alpha = __builtin_amdgcn_exp2f(at.m_run - mx);
    float* dst = &sm.u.g.o[wave][lane][0];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * q) =
            f32x4{at.acc[db][4 * q] * alpha, at.acc[db][4 * q + 1] * alpha, at.acc[db][4 * q + 2] * alpha,
                  at.acc[db][4 * q + 3] * alpha};
  }
  __syncthreads();
  if (wave < 2 * DB) {                       // wave 2 db + p: registers 8 p .. 8 p + 7 of block db
    const int db = wave >> 1, p = wave & 1;
    float l = 0.f;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) {
      l += __builtin_amdgcn_exp2f(sm.u.g.m[x][lc] - mx) * sm.u.g.l[x][lc];
      const float* src = &sm.u.g.o[x][lane][16 * db + 8 * p];
      lo += *reinterpret_cast<const f32x4*>(src);
      hi += *reinterpret_cast<const f32x4*>(src + 4);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int x = w.qb * kQRows + lc;
    if (x < rows_total) {
      const int i = x / Gq, h = g * Gq + (x - i * Gq);
      const uint32_t x0 = pack_bf16x2(lo[0] * inv, lo[1] * inv), x1 = pack_bf16x2(lo[2] * inv, lo[3] * inv);
      const uint32_t y0 = pack_bf16x2(hi[0] * inv, hi[1] * inv), y1 = pack_bf16x2(hi[2] * inv, hi[3] * inv);
      const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
      uint16_t* orow = static_cast<uint16_t*>(a.o) + (((int64_t)s * a.l_d + i) * a.h_q + h) * D + 8 * lj;
      *reinterpret_cast<u32x4*>(orow + 32 * db + 16 * p) = u32x4{s0[0], s1[0], s0[1], s1[1]};
      if (wave == 0 && lj == 0 && a.lse != nullptr)
        a.lse[((int64_t)s * a.h_q + h) * a.l_d + i] = mx * kLn2 + logf(l);
    }
  }
}

}  // namespace

int launch_decode_ws(const DecodeArgs& a, int d, void* stream) {
  if (a.grid_wg == 0) return (int)hipSuccess;
  const hipStream_t st = (hipStream_t)stream;
  if (d == 128)
    hipLaunchKernelGGL((decode_ws_kernel<128>), dim3(a.grid_wg), dim3(kThreads), 0, st, a);
  else if (d == 64)
    hipLaunchKernelGGL((decode_ws_kernel<64>), dim3(a.grid_wg), dim3(kThreads), 0, st, a);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace pdllm
