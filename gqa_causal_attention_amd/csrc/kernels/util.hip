// Small device utilities: a non-finite scan of a weight tensor (run once when
// a block is created: the mojolearn page rejects non-finite weights before any
// computation), the optional non-finite count over a state's cached keys and
// values (the same page's check of cache values, a debug option here since it
// reads the whole cache), a per-row length bump, and the zeroing of the padding positions
// of a ragged prefill (mojolearn TransformerBlock.forward `lengths`: padding
// positions output exactly +0.0).
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

// Non-finite values among the used slots of a state's cache: row b, kv head j
// (blockIdx.y = b * KV + j) holds min(lengths[b], cap) used slots (slots 0 ..
// lengths[b] - 1, or every slot of a full window ring) of hd values in k and
// in v.  Each thread tests its elements of both and adds how many were inf or
// NaN to *count (one atomic per thread that found any; a debug pass, plain
// element loads).
template <typename T>
__global__ __launch_bounds__(256) void cache_nonfinite_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                              const int* __restrict__ lengths, int KV, int cap,
                                                              int hd, int* count) {
  const int b = blockIdx.y / KV;
  const int64_t slab = (int64_t)blockIdx.y * cap * hd;
  const int used = min(max(lengths[b], 0), cap);
  const int64_t n = (int64_t)used * hd;
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    bad += !__builtin_isfinite(to_f32(k[slab + i]));
    bad += !__builtin_isfinite(to_f32(v[slab + i]));
  }
  if (bad) atomicAdd(count, bad);
}

__global__ void bump_kernel(int* lengths, int n, int by) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) lengths[i] += by;
}

// Rows first .. first + count - 1 of y [B, L, d]: positions t >= n[row - first]
// get +0.0.  Grid: (elements per row / 256, count).
constexpr int kPadRows = 256;
struct PadLens {
  int32_t n[kPadRows];
};
__global__ __launch_bounds__(256) void zero_padding_kernel(float* y, PadLens lens, int first, int L, int d) {
  const int r = blockIdx.y;
  const int64_t per_row = (int64_t)L * d;
  const int64_t start = (int64_t)lens.n[r] * d;
  float* row = y + (int64_t)(first + r) * per_row;
  for (int64_t i = start + (int64_t)blockIdx.x * 256 + threadIdx.x; i < per_row; i += (int64_t)gridDim.x * 256)
    row[i] = 0.0f;
}

}  // namespace

hipError_t launch_zero_padding(float* y, const int32_t* lengths_host, int B, int L, int d, hipStream_t s) {
  for (int first = 0; first < B; first += kPadRows) {
    const int count = B - first < kPadRows ? B - first : kPadRows;
    PadLens lens{};
    int maxpad = 0;
    for (int r = 0; r < count; ++r) {
      lens.n[r] = lengths_host[first + r];
      if (L - lens.n[r] > maxpad) maxpad = L - lens.n[r];
    }
    if (maxpad == 0) continue;
    const int64_t blocks = std::min<int64_t>(((int64_t)maxpad * d + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_padding_kernel, dim3((unsigned)blocks, (unsigned)count), dim3(256), 0, s, y, lens, first,
                       L, d);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Packed ragged rows: row tables written from host values passed by value
// (first row `first`, `count` rows), the gather of the real tokens of x
// [B, L, d] into packed rows, and the scatter back with +0.0 padding.
struct RowTableChunk {
  int32_t start[kPadRows];
  int32_t len[kPadRows];
};
__global__ __launch_bounds__(256) void row_tables_kernel(RowTableChunk c, int first, int count, int* row_start,
                                                         int* row_len) {
  const int i = threadIdx.x;
  if (i < count) {
    row_start[first + i] = c.start[i];
    row_len[first + i] = c.len[i];
  }
}
// grid (token blocks of 4, B): 64 threads per token row, float4 pieces
__global__ __launch_bounds__(256) void gather_rows_kernel(const float* __restrict__ x, float* __restrict__ xp,
                                                          const int* row_start, const int* row_len, int L, int d) {
  const int b = blockIdx.y, t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= row_len[b]) return;
  const float4* src = reinterpret_cast<const float4*>(x + ((int64_t)b * L + t) * d);
  float4* dst = reinterpret_cast<float4*>(xp + ((int64_t)row_start[b] + t) * d);
  for (int i = threadIdx.x & 63; i < d / 4; i += 64) dst[i] = src[i];
}
__global__ __launch_bounds__(256) void scatter_rows_kernel(const float* __restrict__ xp, float* __restrict__ y,
                                                           const int* row_start, const int* row_len, int L, int d) {
  const int b = blockIdx.y, t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= L) return;
  float4* dst = reinterpret_cast<float4*>(y + ((int64_t)b * L + t) * d);
  if (t < row_len[b]) {
    const float4* src = reinterpret_cast<const float4*>(xp + ((int64_t)row_start[b] + t) * d);
    for (int i = threadIdx.x & 63; i < d / 4; i += 64) dst[i] = src[i];
  } else {
    for (int i = threadIdx.x & 63; i < d / 4; i += 64) dst[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

hipError_t launch_row_tables(const int32_t* lengths_host, int B, int* row_start, int* row_len, hipStream_t s) {
  int64_t acc = 0;
  for (int first = 0; first < B; first += kPadRows) {
    const int count = B - first < kPadRows ? B - first : kPadRows;
    RowTableChunk c{};
    for (int r = 0; r < count; ++r) {
      c.start[r] = (int32_t)acc;
      c.len[r] = lengths_host[first + r];
      acc += lengths_host[first + r];
    }
    hipLaunchKernelGGL(row_tables_kernel, dim3(1), dim3(256), 0, s, c, first, count, row_start, row_len);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gather_rows(const float* x, float* xp, const int* row_start, const int* row_len, int B, int L, int d,
                              hipStream_t s) {
  if (B <= 0 || L <= 0 || d % 4 != 0) return B <= 0 || L <= 0 ? hipSuccess : hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((L + 3) / 4), (unsigned)B), dim3(256), 0, s, x, xp,
                     row_start, row_len, L, d);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const float* xp, float* y, const int* row_start, const int* row_len, int B, int L,
                               int d, hipStream_t s) {
  if (B <= 0 || L <= 0 || d % 4 != 0) return B <= 0 || L <= 0 ? hipSuccess : hipErrorInvalidValue;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)((L + 3) / 4), (unsigned)B), dim3(256), 0, s, xp, y,
                     row_start, row_len, L, d);
  return hipGetLastError();
}

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

hipError_t launch_cache_nonfinite(const void* k, const void* v, const int* lengths, int elem, int B, int KV,
                                  int cap, int hd, int* count, hipStream_t s) {
  if (B <= 0 || (int64_t)B * KV > 65535) return hipErrorInvalidValue;
  const int64_t per = (int64_t)cap * hd;
  const unsigned bx = (unsigned)std::min<int64_t>(std::max<int64_t>((per + 255) / 256, 1), 64);
  if (elem == kBF16)
    hipLaunchKernelGGL(cache_nonfinite_kernel<bf16>, dim3(bx, (unsigned)(B * KV)), dim3(256), 0, s,
                       static_cast<const bf16*>(k), static_cast<const bf16*>(v), lengths, KV, cap, hd, count);
  else
    hipLaunchKernelGGL(cache_nonfinite_kernel<float>, dim3(bx, (unsigned)(B * KV)), dim3(256), 0, s,
                       static_cast<const float*>(k), static_cast<const float*>(v), lengths, KV, cap, hd, count);
  return hipGetLastError();
}

hipError_t launch_bump_lengths(int* lengths, int n, int by, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(bump_kernel, dim3((n + 255) / 256), dim3(256), 0, s, lengths, n, by);
  return hipGetLastError();
}

}  // namespace gqa
