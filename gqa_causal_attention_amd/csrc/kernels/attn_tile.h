// LDS helpers shared by the matrix-core attention kernels (forward prefill
// and backward): direct-to-LDS loads, the transposing 16-bit LDS read and a
// workgroup barrier that publishes LDS writes.
#pragma once
#include "common.h"

namespace gqa {

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (lds is wave-uniform).  The builtin only exists for the device pass.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
#else
  return s16x4{};
#endif
}

// The same read through inline asm.  Before the builtin form the compiler
// waits for every outstanding global load (vmcnt 0), the direct-to-LDS loads
// of the next tile included; the asm form leaves that wait out, and its
// result is not tracked: wait for it (lgkm_wait) and tie() it before use.
__device__ __forceinline__ s16x4 lds_read_tr16_nowait(const void* p) {
  s16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p));
  return v;
}
// Wait until at most N LDS / scalar-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
// Makes v look redefined here, so its uses stay behind a preceding lgkm_wait.
__device__ __forceinline__ void tie(s16x4& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gqa
