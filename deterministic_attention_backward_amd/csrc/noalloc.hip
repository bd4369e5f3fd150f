// Allocation-free variant of attn_bwd_deterministic: the backward's workspace
// (fp32 dQ accumulator, per-row softmax terms, hand-off flags, Symmetric
// Shift's parking area) lives in a static device array of this library
// instead of a caller's buffer, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation).
//
// Each device the library runs on holds its own copy of `scratch` until the
// process ends. Host code never passes `scratch` itself to a kernel (in host
// code the name is a host-side stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and kept per device.
//
// Nothing in the scratch array has to start at zero: the pre-pass of every
// call resets the hand-off flags, tickets and head slots, and the first
// contributor of every dQ element stores rather than adds. All calls on one
// device share that device's array, so calls that overlap in time on one
// device (different streams, or different host threads) race and must not
// be issued.
#include "../../include/attn_det.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(ATTN_NOALLOC_SCRATCH_MIB) << 20;

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)
std::mutex g_scratch_mutex;

// The device address of this device's copy of `scratch` (looked up on the
// first call on each device, with that device current).
int scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd_deterministic_noalloc(const void* q, const void* k, const void* v, const void* o,
                                              const void* dout, const float* lse, int mask, int schedule, void* dq,
                                              void* dk, void* dv, int B, int H, int S, int D, float scale,
                                              int tile_request, void* stream) {
  // Every argument is checked on the host first: the shared validation stops
  // at the missing workspace (ATTN_ERR_WORKSPACE) before any HIP call when
  // the arguments themselves are valid. Then a problem whose workspace does
  // not fit the static array is refused, still before any HIP call.
  const int pre = attn::run_bwd(q, k, v, o, dout, lse, mask, schedule, dq, dk, dv, B, H, H, S, D, scale,
                                tile_request, nullptr, 0, stream, true);
  if (pre != ATTN_ERR_WORKSPACE) return pre;
  if (attn_bwd_workspace_size(B, H, S, D, mask, schedule, tile_request) > kScratchBytes)
    return ATTN_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int st = scratch_for_current_device(&ws);
  if (st != ATTN_OK) return st;
  return attn::run_bwd(q, k, v, o, dout, lse, mask, schedule, dq, dk, dv, B, H, H, S, D, scale, tile_request, ws,
                       kScratchBytes, stream, true);
}
