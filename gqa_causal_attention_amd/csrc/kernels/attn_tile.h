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

__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gqa
