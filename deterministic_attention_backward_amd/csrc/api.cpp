// C ABI of libattn_det.so: argument validation (pure host, before any HIP
// call), workspace sizing, tile choice, schedule export and kernel dispatch.
#include "../../include/attn_det.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "launch.hpp"
#include "schedule.hpp"

using namespace attn;

namespace {

constexpr uint32_t kDefaultWaitLimit = 1u << 21;
uint32_t g_wait_limit = kDefaultWaitLimit;
int g_poison = 0;
int g_dq_protocol = DQ_AUTO;
hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;

constexpr int kMaxDevices = 64;
int g_num_cu[kMaxDevices];  // 0 = not queried yet

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int choose_tile(int S, int D, int tile_request) {
  if (S <= 0 || (D != 64 && D != 128)) return 0;
  if (tile_request == 64 || tile_request == 128) return tile_request;
  if (tile_request != 0) return 0;
  return S <= 256 ? 64 : 128;
}

struct Shape {
  int T, BR, N, S_pad, n_qsub;
  long long BH;
  bool grouped;  // fewer K/V heads than query heads
};

// Shape checks shared by the backward entry points; returns a status.
int check_shape(int B, int H, int Hkv, int S, int D, int mask, int schedule, int tile_request, bool deterministic,
                Shape* sh) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || S <= 0 || D <= 0) return ATTN_ERR_INVALID_ARG;
  if (H % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (mask != ATTN_MASK_FULL && mask != ATTN_MASK_CAUSAL) return ATTN_ERR_INVALID_ARG;
  if (schedule < ATTN_SCHED_NAIVE || schedule > ATTN_SCHED_SYMMETRIC_SHIFT) return ATTN_ERR_INVALID_ARG;
  if (tile_request != 0 && tile_request != 64 && tile_request != 128) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  const int T = choose_tile(S, D, tile_request);
  const long long N = (static_cast<long long>(S) + T - 1) / T;
  const long long BH = static_cast<long long>(B) * H;
  const int BR = bwd_sub_rows(D, T);
  // index arithmetic on the device uses 32-bit unit and counter indices
  if (BH * align64(N * (T / BR) * dq_waves(T)) >= (1ll << 31) || BH * N * T * D >= (1ll << 40))
    return ATTN_ERR_UNSUPPORTED;
  if (deterministic) {
    if (schedule == ATTN_SCHED_SYMMETRIC_SHIFT && (mask != ATTN_MASK_CAUSAL || (N % 2) != 0))
      return ATTN_ERR_UNSUPPORTED;
  }
  sh->T = T;
  sh->BR = BR;
  sh->N = static_cast<int>(N);
  sh->S_pad = static_cast<int>(N * T);
  sh->n_qsub = static_cast<int>(N * (T / BR));
  sh->BH = BH;
  sh->grouped = Hkv != H;
  return ATTN_OK;
}

WsLayout layout_for(const Shape& sh, int D, int schedule, bool deterministic) {
  const bool park = deterministic && schedule == ATTN_SCHED_SYMMETRIC_SHIFT;
  return ws_layout(sh.BH, sh.S_pad, D, sh.n_qsub, sh.T, park, sh.grouped);
}

int num_cu_current(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  if (g_num_cu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return ATTN_ERR_HIP;
    g_num_cu[dev] = n;
  }
  *out = g_num_cu[dev];
  return ATTN_OK;
}

}  // namespace

namespace attn {

int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
            int mask, int schedule, void* dq, void* dk, void* dv, int B, int H, int Hkv, int S, int D, float scale,
            int tile_request, void* workspace, size_t workspace_bytes, void* stream, bool deterministic) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  Shape sh;
  const int st = check_shape(B, H, Hkv, S, D, mask, schedule, tile_request, deterministic, &sh);
  if (st != ATTN_OK) return st;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_ERR_ALIGNMENT;
  const WsLayout lay = layout_for(sh, D, schedule, deterministic);
  if (!workspace || workspace_bytes < lay.total) return ATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_ALIGNMENT;

  int num_cu = 0;
  if (num_cu_current(&num_cu) != ATTN_OK) return ATTN_ERR_HIP;
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.ws = static_cast<char*>(workspace);
  a.lay = lay;
  a.B = B; a.H = H; a.Hkv = Hkv; a.S = S; a.D = D;
  a.T = sh.T; a.BR = sh.BR; a.N = sh.N; a.S_pad = sh.S_pad; a.n_qsub = sh.n_qsub;
  a.scale = scale;
  a.causal = mask == ATTN_MASK_CAUSAL;
  // The atomic variant has no order to keep: it walks Shift's order, so that
  // at every step the workers of a head add into different dQ tiles.
#ifndef ATTN_ATOMIC_WALK
#define ATTN_ATOMIC_WALK ATTN_SCHED_SHIFT
#endif
  a.sched = deterministic ? schedule : ATTN_ATOMIC_WALK;
  a.atomic = deterministic ? 0 : 1;
  a.wait_limit = g_wait_limit;
  a.poison = g_poison;
  a.dq_protocol = g_dq_protocol;
  a.ev_before = g_ev_before;
  a.ev_after = g_ev_after;
  const hipError_t e = launch_bwd(a, num_cu, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidConfiguration) return ATTN_ERR_UNSUPPORTED;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace attn

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_ALIGNMENT: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_TIMEOUT: return "dQ ordering wait timed out";
    case ATTN_ERR_SCRATCH_LIMIT: return "problem too large for the allocation-free entry point's static scratch";
    default: return "unknown status";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S, int D,
             float scale, int mask, void* stream) {
  return attn_fwd_gqa(q, k, v, o, lse, B, H, H, S, D, scale, mask, stream);
}

int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int S,
                 int D, float scale, int mask, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || !std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (H % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (mask != ATTN_MASK_FULL && mask != ATTN_MASK_CAUSAL) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if (static_cast<long long>(B) * H > 65535 || static_cast<long long>(B) * H * S * D >= (1ll << 40))
    return ATTN_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return ATTN_ERR_ALIGNMENT;
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Hkv = Hkv; a.S = S; a.D = D;
  a.causal = mask == ATTN_MASK_CAUSAL;
  a.scale = scale;
  return launch_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd_tile(int S, int D, int tile_request) {
  if (S <= 0 || D <= 0) return ATTN_ERR_INVALID_ARG;
  if (tile_request != 0 && tile_request != 64 && tile_request != 128) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  return choose_tile(S, D, tile_request);
}

size_t attn_bwd_workspace_size(int B, int H, int S, int D, int mask, int schedule, int tile_request) {
  return attn_bwd_gqa_workspace_size(B, H, H, S, D, mask, schedule, tile_request);
}

size_t attn_bwd_gqa_workspace_size(int B, int H, int Hkv, int S, int D, int mask, int schedule, int tile_request) {
  Shape sh;
  if (check_shape(B, H, Hkv, S, D, mask, schedule, tile_request, true, &sh) != ATTN_OK) {
    // the non-deterministic call accepts any schedule value; size it as NAIVE
    if (check_shape(B, H, Hkv, S, D, mask, ATTN_SCHED_NAIVE, tile_request, true, &sh) != ATTN_OK) return 0;
    return layout_for(sh, D, ATTN_SCHED_NAIVE, true).total;
  }
  return layout_for(sh, D, schedule, true).total;
}

int attn_bwd_deterministic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, int mask, int schedule, void* dq, void* dk, void* dv, int B, int H,
                           int S, int D, float scale, int tile_request, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return run_bwd(q, k, v, o, dout, lse, mask, schedule, dq, dk, dv, B, H, H, S, D, scale, tile_request, workspace,
                 workspace_bytes, stream, true);
}

int attn_bwd_deterministic_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, int mask, int schedule, void* dq, void* dk, void* dv, int B, int H,
                               int Hkv, int S, int D, float scale, int tile_request, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return run_bwd(q, k, v, o, dout, lse, mask, schedule, dq, dk, dv, B, H, Hkv, S, D, scale, tile_request,
                 workspace, workspace_bytes, stream, true);
}

int attn_bwd_nondeterministic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, int mask, void* dq, void* dk, void* dv, int B, int H, int S, int D,
                              float scale, int tile_request, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return run_bwd(q, k, v, o, dout, lse, mask, ATTN_SCHED_NAIVE, dq, dk, dv, B, H, H, S, D, scale, tile_request,
                 workspace, workspace_bytes, stream, false);
}

int attn_bwd_nondeterministic_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                  const float* lse, int mask, void* dq, void* dk, void* dv, int B, int H, int Hkv,
                                  int S, int D, float scale, int tile_request, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return run_bwd(q, k, v, o, dout, lse, mask, ATTN_SCHED_NAIVE, dq, dk, dv, B, H, Hkv, S, D, scale, tile_request,
                 workspace, workspace_bytes, stream, false);
}

int attn_bwd_check(const void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < 64 * sizeof(int)) return ATTN_ERR_INVALID_ARG;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return ATTN_ERR_HIP;
  int flag = 0;
  const char* base = static_cast<const char*>(workspace);
  if (hipMemcpy(&flag, base + sizeof(int), sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
    return ATTN_ERR_HIP;
  return flag ? ATTN_ERR_TIMEOUT : ATTN_OK;
}

int attn_schedule_plan(int n_tiles, int mask, int schedule, int32_t* out, size_t out_len, size_t* needed) {
  if (n_tiles <= 0 || n_tiles > 65536) return ATTN_ERR_INVALID_ARG;
  if (mask != ATTN_MASK_FULL && mask != ATTN_MASK_CAUSAL) return ATTN_ERR_INVALID_ARG;
  if (schedule < ATTN_SCHED_NAIVE || schedule > ATTN_SCHED_SYMMETRIC_SHIFT) return ATTN_ERR_INVALID_ARG;
  const bool causal = mask == ATTN_MASK_CAUSAL;
  if (schedule == ATTN_SCHED_SYMMETRIC_SHIFT && (!causal || n_tiles % 2)) return ATTN_ERR_UNSUPPORTED;
  const int nw = sched_workers(n_tiles, schedule);
  size_t n_tasks = 0;
  for (int w = 0; w < nw; ++w) n_tasks += static_cast<size_t>(sched_num_tasks(n_tiles, causal, schedule, w));
  const size_t want = 2 + 5 * n_tasks;
  if (needed) *needed = want;
  if (!out) return ATTN_OK;
  if (out_len < want) return ATTN_ERR_INVALID_ARG;
  size_t pos = 0;
  out[pos++] = nw;
  out[pos++] = static_cast<int32_t>(n_tasks);
  for (int w = 0; w < nw; ++w) {
    const int nt = sched_num_tasks(n_tiles, causal, schedule, w);
    for (int t = 0; t < nt; ++t) {
      const Task tk = sched_task(n_tiles, causal, schedule, w, t);
      out[pos++] = w;
      out[pos++] = t;
      out[pos++] = tk.q;
      out[pos++] = tk.kv;
      out[pos++] = sched_rank(n_tiles, causal, schedule, tk.q, tk.kv);
    }
  }
  return ATTN_OK;
}

void attn_set_timing_events(void* before, void* after) {
  if (before && after) {
    g_ev_before = static_cast<hipEvent_t>(before);
    g_ev_after = static_cast<hipEvent_t>(after);
  } else {
    g_ev_before = g_ev_after = nullptr;
  }
}

int attn_debug_set_dq_protocol(int protocol) {
  if (protocol < DQ_AUTO || protocol > DQ_XCD_LOCAL) return ATTN_ERR_INVALID_ARG;
  g_dq_protocol = protocol;
  return ATTN_OK;
}

void attn_debug_set_wait_limit(uint32_t iterations, int poison_counter) {
  g_wait_limit = iterations ? iterations : kDefaultWaitLimit;
  g_poison = poison_counter ? 1 : 0;
}

}  // extern "C"
