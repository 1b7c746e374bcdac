// Small device utilities: a non-finite scan of a weight tensor (run once when
// a block is created: the mojolearn page rejects non-finite weights before any
// computation) and a per-row length bump.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void nonfinite_kernel(const T* __restrict__ p, int64_t n, int* flag) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    bad |= !__builtin_isfinite(to_f32(p[i]));
  if (bad) *flag = 1;
}

__global__ void bump_kernel(int* lengths, int n, int by) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) lengths[i] += by;
}

}  // namespace

hipError_t launch_count_nonfinite(const void* p, int elem, int64_t n, int* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  if (elem == kBF16)
    hipLaunchKernelGGL(nonfinite_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const bf16*>(p), n, flag);
  else
    hipLaunchKernelGGL(nonfinite_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const float*>(p), n, flag);
  return hipGetLastError();
}

hipError_t launch_bump_lengths(int* lengths, int n, int by, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(bump_kernel, dim3((n + 255) / 256), dim3(256), 0, s, lengths, n, by);
  return hipGetLastError();
}

}  // namespace gqa
