// Device-side helpers of the gfx950 kernels: vector types, MFMA wrappers,
// bf16 conversion, wave reductions and the XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdllm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Pointers known to be in device global memory (loads through them are
// global_load, which does not share the LDS wait counter as flat loads do).
typedef __attribute__((address_space(1))) const uint16_t* gptr16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16) on one wavefront.
// Lane l supplies A row (l % 16) and B column (l % 16), each with the eight
// k values of lane group l / 16; it receives D column (l % 16), rows
// 4 (l / 16) .. 4 (l / 16) + 3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo, (__bf16)hi});
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// max(a, b) as v_maximum3_f32.  fmaxf (IEEE maxNum) makes the compiler
// quiet each operand it cannot prove canonical first -- every MFMA result
// and every lane-permuted value -- with one extra VALU op per operand; the
// IEEE 754-2019 maximum needs none.  The two differ only on NaN operands
// (maximum returns the NaN), which the softmax inputs never hold.
__device__ __forceinline__ float max_f(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float wave_xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

// Lane v of the same 16-lane DPP row picked by CTRL (quad_perm, row mirrors).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
// Butterfly over the 16 lanes of a DPP row: xor 1, xor 2 (quad permutes),
// then lane i with 7 - i (half mirror) and with 15 - i (mirror).  Each step
// pairs lanes that already hold equal partial results, so every lane of the
// row ends with the same bits.
__device__ __forceinline__ float row16_max(float v) {
  v = max_f(v, dpp_row<0xB1>(v));
  v = max_f(v, dpp_row<0x4E>(v));
  v = max_f(v, dpp_row<0x141>(v));
  return max_f(v, dpp_row<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_row<0xB1>(v);
  v += dpp_row<0x4E>(v);
  v += dpp_row<0x141>(v);
  return v + dpp_row<0x140>(v);
}

// Selection order as an integer key: a float score becomes an order-
// preserving 32-bit key (-0 and +0 share one, NaN gets the lowest), and
// candidate i gets (key << 32) | ~i, so that equal scores rank the lower
// index first and all keys differ.  i outranks j iff key_i > key_j.
__device__ __forceinline__ uint64_t rank_key(float x, uint32_t index) {
  uint32_t u = __float_as_uint(x);
  uint32_t key;
  if (x != x) {
    key = 0u;                               // NaN: after every number
  } else {
    if (x == 0.f) u = 0u;                   // -0 == +0
    key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - index);
}

// Whether candidate c of row[0..n) is among the k best (fewer than k
// candidates outrank it), the rule top-K selects by.  Called by a whole
// wavefront; the result is wave-uniform.
__device__ __forceinline__ bool in_top_k(const float* row, int n, int c, int k) {
  const int lane = threadIdx.x & 63;
  const uint64_t mine = rank_key(row[c], (uint32_t)c);
  int larger = 0;
  // four loads per lane in flight before the comparisons (one memory round
  // trip per 256 candidates)
  for (int j0 = lane; j0 < n; j0 += 256) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = j0 + 64 * u < n ? row[j0 + 64 * u] : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      larger += j0 + 64 * u < n && rank_key(v[u], (uint32_t)(j0 + 64 * u)) > mine ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) larger += __shfl_xor(larger, off, 64);
  return __builtin_amdgcn_readfirstlane(larger) < k;
}

// Whether chunk c of a prefill launch takes part in the window scoring: every
// chunk, or (a.sel_score set) the chunks top-K selects -- chunk c is chunk
// c % sel_per_seq of sequence c / sel_per_seq.  Wave-uniform.
template <class Args>
__device__ __forceinline__ bool chunk_scored(const Args& a, int c) {
  if (a.sel_score == nullptr) return true;
  const int s = c / a.sel_per_seq;
  return in_top_k(a.sel_score + (int64_t)s * a.sel_per_seq, a.sel_per_seq, c - s * a.sel_per_seq, a.sel_k[s]);
}

// The kernel's argument block (its only argument, passed by value) read
// through the argument segment pointer, hidden from the optimiser so that
// loads through it are issued where they are written.
template <class T>
using KernArgs = __attribute__((address_space(4))) const T*;
template <class T>
__device__ __forceinline__ KernArgs<T> kernarg() {
  KernArgs<T> p = (KernArgs<T>)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(p));
  return p;
}

// A compile-time flag passed to a generic lambda (instantiates it twice).
template <bool B>
struct BoolConst {
  static constexpr bool value = B;
};
template <int N>
struct IntConst {
  static constexpr int value = N;
};
// f(IntConst<I>{}), ..., f(IntConst<N - 1>{}) in order
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntConst<I>{});
    static_for<I + 1, N>(f);
  }
}

// Kernel arguments reach a wavefront through the scalar cache, and a
// workgroup's first read of each 64-byte line of them misses it.  Code that
// branches on one argument before it reads the next pays one miss per step.
// warm_args reads one dword every 64 bytes of [BEGIN, END) of an argument
// block, and its last dword (so every line the range overlaps, whatever the
// block's alignment), all in flight together, and waits for them once: the
// later reads of those lines hit the cache.
template <int BEGIN, int END, class T>
__device__ __forceinline__ void warm_args(const T& a) {
  static_assert(BEGIN % 4 == 0 && END % 4 == 0 && BEGIN < END && END <= (int)sizeof(T), "argument range");
  const char* p = reinterpret_cast<const char*>(&a);
  constexpr int N = (END - BEGIN - 4) / 64 + 2;
  int v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int o = BEGIN + 64 * i;
    v[i] = *reinterpret_cast<const int*>(p + (i + 1 < N ? o : END - 4));
  }
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"s"(v[i]));
}

// A wave-uniform 64-bit value (e.g. read from LDS) moved to scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// The last index i in [0, n) with key(i) <= v, for a non-decreasing key
// with key(0) <= v (binary search; wave-uniform arguments stay scalar).
template <class F>
__device__ __forceinline__ int last_index_le(int n, int v, F key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (key(mid) <= v)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Workgroup ids are dispatched round-robin over the 8 XCDs (id % 8).  Remap
// them so that each XCD receives one contiguous range of logical work items;
// neighbouring items share K/V tiles, which then stay in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int kXcd = 8;
  const int per = n / kXcd, rem = n % kXcd;
  const int x = bid % kXcd, k = bid / kXcd;
  return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

}  // namespace pdllm
