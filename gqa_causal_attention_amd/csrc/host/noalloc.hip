// The decode step for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation):
// gqa_block_step with the workspace taken from a fixed device array of this
// library instead of a caller-supplied buffer.
//
// `scratch` below is a file-scope device array.  In host code its name is
// only a host-side stand-in, never a device address: its device address is
// obtained once per device with hipGetSymbolAddress and kept per device, and
// only that address is ever handed to the step.  Every call on one GPU shares
// that GPU's array and finds the previous call's contents in it (nothing the
// step reads from its workspace is assumed to start at zero: every value is
// written before it is read within the call).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../../include/gqa_block.h"

namespace gqa_host {
int report(int code, const char* fmt, ...);  // sets the thread's last-error text (block.cpp)
}

constexpr size_t kScratchBytes = (size_t)64 << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch` (set up on the
// first call on each device, with that device current).
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gqa_host::report(GQA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return gqa_host::report(GQA_ERR_HIP, "device %d is beyond the %d devices this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return gqa_host::report(GQA_ERR_HIP, "hipGetSymbolAddress of the step scratch failed: %s",
                              hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_block_step_noalloc(gqa_block* blk, gqa_state* st, const float* x_dev, float* y_dev, int32_t B,
                           void* hip_stream) {
  if (!blk) return gqa_host::report(GQA_ERR_ARG, "block is NULL");
  if (!st) return gqa_host::report(GQA_ERR_STATE, "step requires a state");
  size_t need = 0;
  if (int r = gqa_workspace_bytes(blk, B, 1, &need)) return r;
  if (need > kScratchBytes)
    return gqa_host::report(GQA_ERR_WORKSPACE,
                            "a step of %d rows needs %zu bytes of workspace, beyond the %zu-byte scratch of the "
                            "no-allocation step",
                            B, need, kScratchBytes);
  void* ws = nullptr;
  if (int r = scratch_of_current_device(&ws)) return r;
  return gqa_block_step(blk, st, x_dev, y_dev, B, ws, kScratchBytes, hip_stream);
}

}  // extern "C"
