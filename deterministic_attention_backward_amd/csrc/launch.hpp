// Internal interface between the C-ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Workgroups that may hold a Symmetric Shift parking slot at once; the
// persistent grid never exceeds this.
constexpr int kMaxGrid = 512;

// Unit queues for XCD-local placement: one per XCD id (gfx950 reports 0..7).
constexpr int kMaxQueues = 16;

// dQ hand-off protocols (attn_debug_set_dq_protocol)
enum { DQ_AUTO = 0, DQ_DEVICE = 1, DQ_XCD_LOCAL = 2 };

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Byte layout of the backward workspace (every region 256-byte aligned):
//   header   int32[64]: [0] unit ticket, [1] timeout flag, [2] next head to
//            claim, [16 + q] unit ticket of XCD queue q
//   heads    int32[kMaxQueues][heads_row]: head claimed by each local head slot
//            of a queue (rows padded to 256 bytes: one queue per cache line set)
//   flags    int32[BH][flag_stride]: per (head, query sub-tile, dQ wave) the
//            number of contributions that wave has handed over (rows padded to
//            256 bytes, so no two heads share a cache line)
//   lse2     fp32[BH * S_pad]: lse * log2(e), +inf on padding rows
//   delta    fp32[BH * S_pad]: rowsum(dO * O), 0 on padding rows
//   dq_ws    fp32[BH * S_pad * D]: dQ accumulator
//   park     fp32[kMaxGrid * 2 * T * D * 2]: Symmetric Shift only; per workgroup,
//            one slot per KV tile of its pair, each holding dK and dV
//   dkv      fp32[2][BH * S_pad * D]: grouped-query heads only; each query
//            head's dK (scaled) and dV, summed over the group afterwards
struct WsLayout {
  size_t header, heads, flags, lse2, delta, dq_ws, park, dkv, total;
  long long heads_row, flag_stride;  // int32 elements per queue row / per head
};

// dQ waves per workgroup for a KV tile edge T (one per 32 keys)
inline int dq_waves(int T) { return T / 32; }

inline long long align64(long long x) { return (x + 63) & ~63ll; }

inline WsLayout ws_layout(long long BH, int S_pad, int D, int n_qsub, int T, bool park, bool grouped) {
  WsLayout w;
  w.heads_row = align64(BH);
  w.flag_stride = align64((long long)n_qsub * dq_waves(T));
  size_t off = 0;
  w.header = off;   off += align256(64 * sizeof(int));
  w.heads = off;    off += align256(size_t(kMaxQueues) * w.heads_row * sizeof(int));
  w.flags = off;    off += align256(size_t(BH) * w.flag_stride * sizeof(int));
  w.lse2 = off;     off += align256(size_t(BH) * S_pad * sizeof(float));
  w.delta = off;    off += align256(size_t(BH) * S_pad * sizeof(float));
  w.dq_ws = off;    off += align256(size_t(BH) * S_pad * D * sizeof(float));
  w.park = off;     off += park ? align256(size_t(kMaxGrid) * 2 * T * D * 2 * sizeof(float)) : 0;
  w.dkv = off;      off += grouped ? 2 * align256(size_t(BH) * S_pad * D * sizeof(float)) : 0;
  w.total = off;
  return w;
}

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float* lse;
  void *dq, *dk, *dv;
  char* ws;
  WsLayout lay;
  int B, H, Hkv, S, D, T, BR, N, S_pad, n_qsub;  // Hkv: K/V heads (H / Hkv query heads share one)
  float scale;
  int causal, sched, atomic;
  uint32_t wait_limit;
  int poison;
  int dq_protocol;                 // DQ_AUTO / DQ_DEVICE / DQ_XCD_LOCAL
  hipEvent_t ev_before, ev_after;  // optional: recorded around the main kernel
};

struct FwdArgs {
  const void *q, *k, *v;
  void* o;
  float* lse;
  int B, H, Hkv, S, D, causal;
  float scale;
};

// Sub-tile height (query rows per MFMA pass) the backward uses for (D, T).
inline int bwd_sub_rows(int D, int T) { return (D == 64 && T == 128) ? 128 : 64; }

hipError_t launch_bwd(const BwdArgs& a, int num_cu, hipStream_t stream);

// The backward entry points' common path (api.cpp): validates every argument
// on the host before any HIP call, then launches on `stream`. Returns a status.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, int mask,
            int schedule, void* dq, void* dk, void* dv, int B, int H, int Hkv, int S, int D, float scale,
            int tile_request, void* workspace, size_t workspace_bytes, void* stream, bool deterministic);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

}  // namespace attn
