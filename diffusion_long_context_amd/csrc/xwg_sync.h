// Data exchange between the workgroups of one launch that run on one XCD of
// gfx950, through that XCD's L2.
//
// The CUs of an XCD share its L2; their vector L1 caches are write-through
// and are invalidated when a kernel starts.  A workgroup publishes results
// to the other workgroups of its XCD by storing them (they reach the L2),
// waiting until its stores have completed (vmcnt(0)), and then adding to a
// counter with a relaxed agent-scope atomic, which every CU sees.  A reader
// acts only after it has seen the count it waits for, and loads the results
// with plain loads: they hit the L2, and no L1 line of theirs can be stale,
// because no CU reads a published line before its reader does.  No cache is
// written back or invalidated (the L2-wide write-back / invalidate that an
// agent-scope fence compiles to is not needed inside one XCD).
#pragma once

#include "device_common.h"

namespace pdllm {

// A raw buffer resource over `base` (byte offsets below 2 GiB, bounds-checked).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ void store_l2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 0);
}
__device__ __forceinline__ void store_l2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 0);
}
__device__ __forceinline__ void store_l2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
}
__device__ __forceinline__ u32x4 load_l2_b128(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
__device__ __forceinline__ u32x2 load_l2_b64(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
}
__device__ __forceinline__ float load_l2_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// Wait until this thread's vector memory operations, stores included, have
// completed (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ int counter_add(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int counter_load(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void counter_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace pdllm
