// Attention backward kernels for gfx950: pre-pass, main tile kernel with the
// ordered dQ reduction, and the dQ conversion pass of the atomic variant.
//
// Gradient (per head, scale c, from the given O and LSE):
//   P = exp(c Q K^T - LSE)   dV = P^T dO   dP = dO V^T   Delta = rowsum(dO * O)
//   dS = P * (dP - Delta)    dQ = c dS K   dK = c dS^T Q
//
// Work decomposition (DASH, Dutch and Japanese technical summaries §2.1: all
// work of one KV tile stays on one processor so that its accumulators stay in
// registers): a persistent grid of workgroups takes "units" from a ticket
// counter; a unit is one worker of one head (one KV tile, two for Symmetric
// Shift). The unit walks its tasks (query tile i, KV tile j) in the order the
// schedule fixes, accumulates dK_j/dV_j in MFMA accumulators and, per query
// sub-tile, hands its dQ partial to the fp32 dQ workspace in the schedule's
// order: wait until the sub-tile's counter equals r(i, j), add, then (one
// sub-tile later, when the adds have long completed) increment the counter.
// The last contributor of a sub-tile writes bf16 dq itself; a post-pass
// checks the call's failure flag (and converts the atomic variant's sums).
#include "../../include/attn_det.h"
#include "common.hpp"
#include "launch.hpp"
#include "lds.hpp"
#include "schedule.hpp"

namespace attn {

// --------------------------------------------------------------------------------------
// pre-pass: Delta = rowsum(dO * O) in fp32, LSE in base 2, hand-off flags and tickets reset.

struct PreParams {
  const bf16 *o, *dout;
  const float* lse;
  float *lse2, *delta, *dq_ws;
  int *flags, *header, *heads;
  long long n_heads;    // entries of the head table
  long long rows;       // BH * S_pad
  int S, S_pad;
  long long n_flags;
  long long dq_ws_elems;  // > 0: zero the dQ accumulator (atomic variant)
};

// Control words shared between XCDs (tickets, head claims, the hand-off flags of
// the cross-XCD protocol) are only touched by atomic read-modify-writes at
// device scope, so every access meets the others at the same place. A read is
// an atomic OR with a zero the compiler cannot see: an RMW whose operand is a
// known identity (add 0, or 0) is folded into an atomic load, which the cache
// hierarchy serves like any other load and which then need not observe the
// RMWs other waves perform on the word.
__device__ __forceinline__ void ctl_set(int* w, int v) {
  (void)__hip_atomic_exchange(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ctl_read(int* w) {
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  return __hip_atomic_fetch_or(w, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Number of bounded waits that ran out since the last read (all launches of
// this process on this device); read and cleared by attn_debug_wait_timeouts.
// header[1] marks the call itself as failed: its post-passes write NaN outputs.
__device__ int g_wait_timeouts;

__device__ __forceinline__ void note_timeout(int* header) {
  ctl_set(&header[1], 1);
  atomicAdd(&g_wait_timeouts, 1);
}

template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(PreParams p) {
  constexpr int LPR = D / 8;  // lanes per row, 8 bf16 each
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nthreads = (long long)gridDim.x * blockDim.x;
  const int sub = threadIdx.x % LPR;
  // Control words (hand-off flags, tickets, head table) start at 0 (head slots at
  // -1). The main kernel launches after this kernel has completed, which makes
  // these values visible to every XCD.
  for (long long i = gtid; i < p.n_flags; i += nthreads) ctl_set(&p.flags[i], 0);
  if (gtid < 64) ctl_set(&p.header[gtid], 0);
  for (long long i = gtid; i < p.n_heads; i += nthreads) ctl_set(&p.heads[i], -1);
  for (long long base = gtid / LPR; base < p.rows; base += nthreads / LPR) {
    const long long bh = base / p.S_pad;
    const int s = (int)(base % p.S_pad);
    float acc = 0.0f;
    if (s < p.S) {
      const long long off = (bh * p.S + s) * D + sub * 8;
      const bf16x8 ov = *(const bf16x8*)(p.o + off);
      const bf16x8 dv = *(const bf16x8*)(p.dout + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)ov[e] * (float)dv[e];
    }
    // fixed butterfly over the LPR lanes of this row: the same order every run
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, LPR);
    if (sub == 0) {
      p.delta[base] = (s < p.S) ? acc : 0.0f;
      p.lse2[base] = (s < p.S) ? p.lse[bh * p.S + s] * 1.4426950408889634f : __builtin_inff();
    }
  }
  for (long long i = gtid * 4; i < p.dq_ws_elems; i += nthreads * 4)
    *(f32x4*)(p.dq_ws + i) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// --------------------------------------------------------------------------------------
// main kernel
//
// A workgroup holds one KV tile of T keys and runs two kinds of waves, one of
// each per SIMD:
//   tile waves (T/32): wave a owns keys 32a..32a+31. Its registers hold those
//     keys' K rows (B operand of S = Q K^T; at D = 64 also the V rows of
//     dP = dO V^T, which at D = 128 the wave reads from its own LDS rows) and
//     their dK and dV accumulators (transposed: four consecutive features of
//     one key per register quad) for the whole run of tasks on the tile. Per query
//     sub-tile of BR rows it computes S, dP, P and dS, writes dS^T to LDS and
//     accumulates dV += P^T dO and dK += dS^T Q, reading the staged Q and dO
//     rows both row-wise (A operands) and transposed (B operands, through the
//     transposing LDS read).
//   dQ waves (T/32): stage the query sub-tiles (Q, dO, LSE, Delta) from HBM into
//     LDS with DMA loads (no registers involved) and, one sub-tile behind the
//     tile waves, compute dQ = dS K from the dS^T the tile waves left in LDS
//     (K columns held in registers) and hand the partial over to the fp32 dQ
//     workspace in the schedule's order.
// Two workgroup barriers per sub-tile order the hand-over between the roles
// (X: the dQ waves are done with the previous dS^T; Y: the tile waves are done
// with the sub-tile and the next one has landed). The staged rows are
// double-buffered; dS^T is single-buffered and protected by the two barriers.

struct MainParams {
  const bf16 *q, *k, *v;
  const bf16* dout;
  bf16 *dk, *dv;
  const float *lse2, *delta;
  float *dq_ws, *park;
  bf16* dq;
  int *flags, *header, *heads;
  int S, S_pad, N, n_qsub, n_workers, n_units, sched, BH;
  int ilv;  // heads whose workers share each run of XCD-queue tickets (1: one head after another)
  int H, group;  // query heads per batch; query heads per K/V head
  float* dkv;    // group > 1: per query head fp32 dK (scaled), then dV, [BH][S_pad][D] each
  int flag_stride, heads_row;  // int32 elements per head of flags / per queue row of heads
  int poison_flag;             // >= 0: the wait on this flag can never succeed (exercises the bound)
  float scale, scale_log2;
  uint32_t wait_limit;
};

// XCD-local words (hand-off flags, head slots, the dQ accumulator): plain
// stores, which pass the CU's write-through L1 and land in the XCD's L2, and
// agent-scope loads, which skip the L1 and are served by that L2. Every access
// of such a word within a launch comes from one XCD, so its L2 is the single
// place where they all meet. (A plain load may be served by a stale L1 line,
// and an L1 invalidate at workgroup scope does not drop it.)
__device__ __forceinline__ void l2_store(int* w, int v) {
  asm volatile("" ::: "memory");
  *w = v;
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ int l2_load(int* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at base + byte_off through a buffer resource (base wave-uniform,
// byte_off < bytes), as an agent-scope load served by the XCD's L2.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 l2_load16(const float* base, unsigned bytes, unsigned byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(base, bytes), (int)byte_off, 0, 16 /* sc1 */));
}

// Words shared by workgroups on different XCDs: system-scope accesses (sc0 sc1
// cache policy), which are written through to and read from the device-wide
// coherence point instead of an XCD's L2. The dword forms are the relaxed
// system-scope atomic load and store; the 16-byte forms use the same policy
// on buffer loads and stores. Measured on the box: workgroups on two XCDs
// handing a 4 KB region back and forth this way (flag after a completed
// store) never read a stale value in 1000 hand-overs.
__device__ __forceinline__ void sys_store(int* w, int v) {
  __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ int sys_load(int* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ f32x4 sys_load16(const float* base, unsigned bytes, unsigned byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(base, bytes), (int)byte_off, 0, 17 /* sc0 sc1 */));
}
__device__ __forceinline__ void sys_store16(float* base, unsigned bytes, unsigned byte_off, f32x4 v) {
  typedef unsigned u32v4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32v4, v), rsrc(base, bytes), (int)byte_off, 0, 17);
}

// Workgroup barrier over LDS only: this wave's LDS operations complete
// (lgkmcnt(0)) before it arrives; its global loads and stores stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Profiling build (-DATTN_PROFILE_WAIT=1): per workgroup, the cycles the waves
// spend waiting, read back with attn_debug_wait_profile:
//   [0] tile waves at the two hand-over barriers  [1] tile waves in total
//   [2] dQ waves waiting for their dQ turn         [3] dQ waves at the barriers
//   [4] dQ waves in total                          [5] sub-tiles handed off
//   [6] tile waves switching KV tiles: a segment's set-up (K/V loads, parked
//       accumulators restored, first sub-tile staged, three barriers) and
//       tear-down (accumulators parked or dK/dV stored)
//   [7] segments run                               [8] tile waves claiming units
#ifndef ATTN_PROFILE_WAIT
#define ATTN_PROFILE_WAIT 0
#endif
constexpr bool kProfileWait = ATTN_PROFILE_WAIT != 0;
constexpr int kProfSlots = 9;
__device__ unsigned long long g_wait_prof[kMaxGrid][kProfSlots];
// Profiling build: dQ ordering checks. A wave that waits for its turn must
// never see its flag beyond its rank (someone handed over out of order), and
// a wave that hands over must find its flag still at its own rank (nobody
// else advanced it). Violations are counted here (attn_debug_order_violations).
__device__ unsigned g_order_violations;
static int g_last_grid = 0;

struct WaitClock {
  unsigned long long turn = 0, bar = 0, seg = 0, nseg = 0, claim = 0;
};
__device__ __forceinline__ unsigned long long wclock() {
  if constexpr (kProfileWait) return __builtin_amdgcn_s_memtime();
  return 0;
}

// How a unit hands its dQ partials over.
enum {
  MODE_ATOMIC = 0,  // non-deterministic: fp32 atomic adds in whatever order they land
  MODE_DEVICE = 1,  // deterministic: system-scope read-modify-writes, serialised by the hand-off flags
  MODE_XCD = 2      // deterministic: all workers of a head on one XCD, plain RMW via its L2
};

template <int D_, int T_, int BR_>
struct Geo {
  static constexpr int D = D_, T = T_, BR = BR_;
  static constexpr int NA = T / 32;            // tile waves
  static constexpr int NB = NA;                // dQ waves
  static constexpr int NTA = NA * 64, NTB = NB * 64, NT = NTA + NTB;
  static constexpr int DP = D + 8;             // padded K and V rows (bf16 elements)
  static constexpr int RB = 2 * D;             // staged Q/dO row (bytes, swizzled chunks)
  static constexpr int SP = BR + 4;            // transposed dS rows
  static constexpr int KC = D / 16;            // k-chunks over the features
  static constexpr int ND = D / 32;            // 32-wide feature blocks
  static constexpr int MB = BR / 32;           // 32-row query blocks per sub-tile
  static constexpr int NSUB = T / BR;          // sub-tiles per task
  static constexpr int TC = T / 16;            // k-chunks over the keys
  static constexpr int QBW = MB * ND / NB;     // dQ blocks per dQ wave: one row block, QBW feature blocks
  // staging: LDS DMA pieces of 1 KB (64 lanes x 16 bytes), Q then dO
  static constexpr int PIECES = 2 * BR * RB / 1024;
  static constexpr int PPW = PIECES / NA;      // per tile wave
  // LDS regions (bytes)
  static constexpr int RM_BYTES = 2 * BR * RB + 2 * BR * 4;  // one staging buffer: Q, dO, LSE, Delta
  static constexpr int KT_OFF = 2 * RM_BYTES;
  static constexpr int KT_BYTES = T * DP * 2;                // K rows, read transposed by the dQ waves
  static constexpr int DS_OFF = KT_OFF + KT_BYTES;
  static constexpr int DS_BYTES = T * SP * 2;
  // D = 128: the tile waves keep V in LDS (row-major, each wave reads only the
  // rows it wrote) so that K, dK and dV fit their registers without spilling
  static constexpr bool V_LDS = D >= 128;
  static constexpr int SV_OFF = DS_OFF + DS_BYTES;
  static constexpr int SV_BYTES = V_LDS ? T * DP * 2 : 0;
  static constexpr int UNIT_OFF = SV_OFF + SV_BYTES;
  static constexpr int LDS_BYTES = UNIT_OFF + 16;
  static_assert(QBW >= 1 && QBW * NB == MB * ND && QBW <= ND && ND % QBW == 0, "dQ block split");
  static_assert(PPW >= 1 && PIECES % NA == 0 && T % BR == 0 && BR % 64 == 0 && NA >= 2, "staging split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(V_LDS || T * DP * 2 <= RM_BYTES, "D = 64: V rows and staged dV fit a staging buffer");
};

template <class G>
struct Lds {
  char* base;
  __device__ __forceinline__ char* q(int b) const { return base + b * G::RM_BYTES; }
  __device__ __forceinline__ char* o(int b) const { return q(b) + G::BR * G::RB; }
  __device__ __forceinline__ float* lse(int b) const { return (float*)(base + b * G::RM_BYTES + 2 * G::BR * G::RB); }
  __device__ __forceinline__ float* dl(int b) const { return lse(b) + G::BR; }
  __device__ __forceinline__ bf16* kt() const { return (bf16*)(base + G::KT_OFF); }
  __device__ __forceinline__ bf16* dst() const { return (bf16*)(base + G::DS_OFF); }
  __device__ __forceinline__ bf16* v() const { return (bf16*)(base + G::SV_OFF); }
  __device__ __forceinline__ int* unit() const { return (int*)(base + G::UNIT_OFF); }
};

// A run of consecutive tasks of one unit on the same KV tile (wave-uniform).
struct Seg {
  int bh, wk, t0, n;  // head, worker, first task, sub-tiles in the run
  int kv, slot;       // KV tile and its parking slot
  bool restore;       // accumulators parked earlier in this unit: reload them
  bool keep;          // the tile comes back later in this unit: park at the end
  bool passes;        // sub-tiles in passes: every task's first sub-tile, then every task's second
  // The i-th sub-tile of the run: its task (index into the unit's task list) and
  // its sub-tile within the task's query tile. In passes, each sub-tile still
  // receives its dQ contributions in the schedule's order of tasks (the order
  // is per query tile, so per sub-tile), while the sub-tiles a workgroup's
  // neighbours touch within one step shrink to half a query tile each: the
  // running sums and staged rows of a step fit the XCD's L2.
  template <int NSUB>
  __device__ __forceinline__ int task(int i) const {
    if (NSUB == 2 && passes) return t0 + (i < n / 2 ? i : i - n / 2);
    return t0 + i / NSUB;
  }
  template <int NSUB>
  __device__ __forceinline__ int half(int i) const {
    if (NSUB == 2 && passes) return i < n / 2 ? 0 : 1;
    return i % NSUB;
  }
};

// ---- tile waves


template <class G, bool CAUSAL, int MODE>
struct TileRole {
  static constexpr int KC = G::KC, ND = G::ND, MB = G::MB, NSUB = G::NSUB;
  const MainParams& p;
  Lds<G> L;
  int tid, lane, a, l32, hh;
  // staged-row addressing (see swz): row-wise reads of row l32, chunk 2c + hh at
  // a_base + 32 (c ^ sw1); transposed reads (TrLane) at tl.base[part] + 64 (n ^ tl.hi)
  int a_base, sw1;
  TrLane tl;
  static constexpr bool VL = G::V_LDS;
  bf16x8 Kr[KC], Vr[VL ? 1 : KC];
  f32x16 dKa[ND], dVa[ND];
  bf16x8 dsb[2];  // dS of the current sub-tile's first row block, packed, carried over barrier X
  WaitClock* wc = nullptr;  // profiling build only

  __device__ __forceinline__ TileRole(const MainParams& p_, Lds<G> L_) : p(p_), L(L_) {
    tid = threadIdx.x;
    lane = tid & 63;
    a = __builtin_amdgcn_readfirstlane(tid >> 6);
    l32 = lane & 31;
    hh = lane >> 5;
    const int sw = swz<G::D>(l32);
    a_base = l32 * G::RB + 16 * ((hh ^ sw) & 1);
    sw1 = sw >> 1;
    tl.init<G::D>(lane);
  }

  __device__ __forceinline__ void park(const Seg& sg, bool load) {
    float* base = p.park + ((size_t)blockIdx.x * 2 + sg.slot) * (size_t)(2 * ND * 16 * G::NTA);
#pragma unroll
    for (int n = 0; n < ND; ++n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float* x = base + (size_t)((n * 16 + i) * G::NTA + tid);
        float* y = base + (size_t)(((ND + n) * 16 + i) * G::NTA + tid);
        if (load) {
          dKa[n][i] = *x;
          dVa[n][i] = *y;
        } else {
          *x = dKa[n][i];
          *y = dVa[n][i];
        }
      }
    }
  }

  __device__ __forceinline__ void seg_begin(const Seg& sg) {
    const int S = p.S;
    // K/V head of this query head (grouped-query attention: group consecutive query heads share one)
    const int kvh = (sg.bh / p.H) * (p.H / p.group) + (sg.bh % p.H) / p.group;
    const bf16* kh = p.k + (size_t)kvh * S * G::D;
    const bf16* vh = p.v + (size_t)kvh * S * G::D;
    // This wave's 32 K and V rows, loaded along the rows (each instruction
    // reads whole rows: full cache lines) into the K-row region (which the
    // dQ waves read transposed) and the V-row region (D = 64: a staging
    // buffer the dQ waves fill only later), then this wave's K operand is
    // read back in the MFMA layout. Keys past the end are read as copies of
    // the last key (they are masked).
    constexpr int LPR = G::D / 8, RPI = 64 / LPR, NR = 32 / RPI;  // lanes per row, rows per instruction
    int lrow = lane / LPR, lcol = 8 * (lane % LPR);
    asm volatile("" : "+v"(lrow), "+v"(lcol));
    const int key0 = sg.kv * G::T + 32 * a;
    bf16x8 kq[NR], vq[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const unsigned off = 2u * (unsigned)(min(key0 + RPI * r + lrow, S - 1) * G::D + lcol);
      kq[r] = *at_bytes((const bf16x8*)kh, off);
      vq[r] = *at_bytes((const bf16x8*)vh, off);
    }
    bf16* kt = L.kt();
    bf16* vs = VL ? L.v() : (bf16*)L.q(1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      *(bf16x8*)&kt[(32 * a + RPI * r + lrow) * G::DP + lcol] = kq[r];
      *(bf16x8*)&vs[(32 * a + RPI * r + lrow) * G::DP + lcol] = vq[r];
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are in LDS
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      Kr[c] = *(const bf16x8*)&kt[(32 * a + l32) * G::DP + 16 * c + 8 * hh];
      if constexpr (!VL) Vr[c] = *(const bf16x8*)&vs[(32 * a + l32) * G::DP + 16 * c + 8 * hh];
    }
    if (sg.restore) {
      park(sg, true);
    } else {
#pragma unroll
      for (int n = 0; n < ND; ++n) {
        dKa[n] = zero16();
        dVa[n] = zero16();
      }
    }
  }
  __device__ __forceinline__ void seg_kd(const Seg&) {}
  __device__ __forceinline__ void seg_stage(const Seg&) {}

  // S and dP of row block m (raw scores)
  __device__ __forceinline__ void mma(int m, int buf, f32x16& s, f32x16& dp) {
    // (the lane constants are re-read here so that the compiler computes the
    // swizzled addresses where they are used instead of keeping them all live)
    int ab = a_base, s1 = sw1;
    asm volatile("" : "+v"(ab), "+v"(s1));
    const char* Q = L.q(buf) + 32 * m * G::RB + ab;
    const char* O = L.o(buf) + 32 * m * G::RB + ab;
    const bf16* V = &L.v()[(32 * a + l32) * G::DP + 8 * hh];
    s = zero16();
    dp = zero16();
    // operands one k-chunk ahead; the scheduling fences keep at most two
    // chunks of operands live (the resident K/dK/dV leave little room)
    bf16x8 qa[2], oa[2], vb[2];
    qa[0] = *(const bf16x8*)(Q + (s1 << 5));
    oa[0] = *(const bf16x8*)(O + (s1 << 5));
    if constexpr (VL) vb[0] = *(const bf16x8*)&V[0];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (c + 1 < KC) {
        const int co = ((c + 1) ^ s1) << 5;
        qa[(c + 1) & 1] = *(const bf16x8*)(Q + co);
        oa[(c + 1) & 1] = *(const bf16x8*)(O + co);
        if constexpr (VL) vb[(c + 1) & 1] = *(const bf16x8*)&V[16 * (c + 1)];
      }
      s = mfma32(qa[c & 1], Kr[c], s);
      dp = mfma32(oa[c & 1], VL ? vb[c & 1] : Vr[VL ? 0 : c], dp);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Row block m: S and dP (their MFMAs interleaved, mma()), then P in place;
  // then dV^T += dO^T P with dS = P (dP - Delta) computed between those MFMAs
  // (16 / ND scores per feature block), so that this vector work runs while
  // they do; then dS^T to LDS and dK^T += Q^T dS. Only the packed dS of row
  // block 0 is carried over barrier X. The dV and dK products take the
  // staged dO and Q rows through the transposing read as their A operands
  // (trB: 8 queries in the order of the C-matrix rows the lane holds, 4 hh +
  // 0..3 and 8 + 4 hh + 0..3) and P or dS, packed, as their B operands, so the
  // accumulators hold dV^T and dK^T blocks: a lane owns four consecutive
  // features of one key per register quad.

  // P = exp2(S scale log2(e) - LSE log2(e)) in place. The exponent is one
  // explicit fused multiply-add, so its rounding (and with it every bit
  // downstream) does not depend on how the compiler schedules this code. A
  // causal mask compiles a masked and an unmasked path (the mask test per
  // score would cost every tile); the other masks test only the key (the
  // ragged last KV tile), one path for all tiles, in which need_mask false
  // lets every key pass.
  template <bool MASK>
  __device__ __forceinline__ void probs_path(int m, int buf, int q_base, int kv_base, bool need_mask, f32x16& sc) {
    const float* Ls = L.lse(buf) + 32 * m + 4 * hh;
    const int key_g = kv_base + 32 * a + l32;
    const bool key_ok = key_g < p.S || !need_mask;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 L4 = *(const f32x4*)&Ls[8 * g];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int i = 4 * g + b;
        const float pv = fast_exp2(__builtin_fmaf(sc[i], p.scale_log2, -L4[b]));
        if constexpr (MASK) {
          const int q_g = q_base + 32 * m + 8 * g + 4 * hh + b;
          sc[i] = key_ok && (!CAUSAL || key_g <= q_g) ? pv : 0.0f;
        } else {
          sc[i] = pv;
        }
      }
    }
  }
  __device__ __forceinline__ void probs(int m, int buf, int q_base, int kv_base, bool need_mask, f32x16& sc) {
    if constexpr (CAUSAL) {
      if (need_mask) probs_path<true>(m, buf, q_base, kv_base, true, sc);
      else probs_path<false>(m, buf, q_base, kv_base, false, sc);
    } else {
      probs_path<true>(m, buf, q_base, kv_base, need_mask, sc);
    }
  }

  __device__ __forceinline__ void dvalues(int m, int buf, const f32x16& sc, f32x16& dpr, bf16x8& d0, bf16x8& d1) {
    const bf16x8 pb0 = pack8(sc, 0), pb1 = pack8(sc, 8);
    int tb[2] = {tl.base[0], tl.base[1]}, th = tl.hi;
    asm volatile("" : "+v"(tb[0]), "+v"(tb[1]), "+v"(th));
    const char* OB = L.o(buf) + 32 * m * G::RB;
    const float* Ds = L.dl(buf) + 32 * m + 4 * hh;
    bf16x8 ov[2][2];
    {
      const int nx = th << 6;
      ov[0][0] = trB<G::RB>(OB, 0, tb, nx);
      ov[0][1] = trB<G::RB>(OB, 1, tb, nx);
    }
    // Delta of the four row quads: one quad ahead at D = 128 (one quad per
    // feature block), all four at once at D = 64 (two per feature block)
    constexpr int QN = 4 / ND;
    f32x4 D4[4];
#pragma unroll
    for (int g = 0; g < (ND == 4 ? 1 : 4); ++g) D4[g] = *(const f32x4*)&Ds[8 * g];
#pragma unroll
    for (int n = 0; n < ND; ++n) {
      if (n + 1 < ND) {
        const int nx = ((n + 1) ^ th) << 6;
        ov[(n + 1) & 1][0] = trB<G::RB>(OB, 0, tb, nx);
        ov[(n + 1) & 1][1] = trB<G::RB>(OB, 1, tb, nx);
        if constexpr (ND == 4) D4[n + 1] = *(const f32x4*)&Ds[8 * (n + 1)];
      }
      dVa[n] = mfma32(ov[n & 1][0], pb0, dVa[n]);
      dVa[n] = mfma32(ov[n & 1][1], pb1, dVa[n]);
      // dS of row quads QN n .. QN n + QN - 1 of the block
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const int g = QN * n + q;
#pragma unroll
        for (int b = 0; b < 4; ++b) dpr[4 * g + b] = sc[4 * g + b] * (dpr[4 * g + b] - D4[g][b]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    d0 = pack8(dpr, 0);
    d1 = pack8(dpr, 8);
  }

  __device__ __forceinline__ void dkeys(int m, int buf, bf16x8 d0, bf16x8 d1) {
    bf16* drow = &L.dst()[(32 * a + l32) * G::SP + 32 * m + 4 * hh];  // four consecutive queries per write
    *(bf16x4*)(drow + 0) = __builtin_shufflevector(d0, d0, 0, 1, 2, 3);
    *(bf16x4*)(drow + 8) = __builtin_shufflevector(d0, d0, 4, 5, 6, 7);
    *(bf16x4*)(drow + 16) = __builtin_shufflevector(d1, d1, 0, 1, 2, 3);
    *(bf16x4*)(drow + 24) = __builtin_shufflevector(d1, d1, 4, 5, 6, 7);
    int tb[2] = {tl.base[0], tl.base[1]}, th = tl.hi;
    asm volatile("" : "+v"(tb[0]), "+v"(tb[1]), "+v"(th));
    const char* QB = L.q(buf) + 32 * m * G::RB;
    bf16x8 qv[2][2];
    {
      const int nx = th << 6;
      qv[0][0] = trB<G::RB>(QB, 0, tb, nx);
      qv[0][1] = trB<G::RB>(QB, 1, tb, nx);
    }
#pragma unroll
    for (int n = 0; n < ND; ++n) {
      if (n + 1 < ND) {
        const int nx = ((n + 1) ^ th) << 6;
        qv[(n + 1) & 1][0] = trB<G::RB>(QB, 0, tb, nx);
        qv[(n + 1) & 1][1] = trB<G::RB>(QB, 1, tb, nx);
      }
      dKa[n] = mfma32(qv[n & 1][0], d0, dKa[n]);
      dKa[n] = mfma32(qv[n & 1][1], d1, dKa[n]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // a row block up to (not including) its dS write and dK products
  __device__ __forceinline__ void block_front(int m, int buf, int q_base, int kv_base, bool need_mask, bf16x8& d0,
                                              bf16x8& d1) {
    f32x16 sc, dpr;
    mma(m, buf, sc, dpr);
    probs(m, buf, q_base, kv_base, need_mask, sc);
    dvalues(m, buf, sc, dpr, d0, d1);
  }

  __device__ __forceinline__ void where(const Seg& sg, int i, int& q_base, int& kv_base, bool& need_mask) {
    const Task task = sched_task(p.N, CAUSAL, p.sched, sg.wk, sg.task<NSUB>(i));
    q_base = task.q * G::T + sg.half<NSUB>(i) * G::BR;
    kv_base = sg.kv * G::T;
    need_mask = (CAUSAL && task.q == sg.kv) || (kv_base + G::T > p.S);
  }

  __device__ __forceinline__ void part1(const Seg& sg, int i) {
    int q_base, kv_base;
    bool need_mask;
    where(sg, i, q_base, kv_base, need_mask);
    block_front(0, i & 1, q_base, kv_base, need_mask, dsb[0], dsb[1]);
  }

  __device__ __forceinline__ void part2(const Seg& sg, int i) {
    int q_base, kv_base;
    bool need_mask;
    where(sg, i, q_base, kv_base, need_mask);
    // (row block 0's dS is written only now: the dQ waves read the previous
    // sub-tile's before barrier X)
    dkeys(0, i & 1, dsb[0], dsb[1]);
#pragma unroll
    for (int m = 1; m < MB; ++m) {
      bf16x8 d0, d1;
      block_front(m, i & 1, q_base, kv_base, need_mask, d0, d1);
      dkeys(m, i & 1, d0, d1);
    }
  }

  __device__ __forceinline__ void seg_end(const Seg& sg) {
    if (sg.keep) {
      park(sg, false);
      return;
    }
    // accumulator quad g of block n: features 32 n + 8 g + 4 hh + 0..3 of key l32
    const int key = sg.kv * G::T + 32 * a + l32;
    if (p.dkv) {  // grouped-query heads: this query head's share, summed over the group later
      float* pk = p.dkv + (size_t)sg.bh * p.S_pad * G::D + (size_t)key * G::D + 4 * hh;  // key < S_pad
      float* pv = pk + (size_t)p.BH * p.S_pad * G::D;
#pragma unroll
      for (int n = 0; n < ND; ++n) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 kq, vq;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kq[e] = dKa[n][4 * g + e] * p.scale;
            vq[e] = dVa[n][4 * g + e];
          }
          *(f32x4*)(pk + 32 * n + 8 * g) = kq;
          *(f32x4*)(pv + 32 * n + 8 * g) = vq;
        }
      }
      return;
    }
    // bf16 dK and dV through LDS: this wave's own 32 rows of the K-row region
    // (idle once the dQ waves have read K^T) take dK, and its rows of the
    // V-row region (D = 128) or of staging buffer 1 (D = 64: the buffer its V
    // rows came in through; idle until the next segment's second sub-tile,
    // staged three barriers later, whereas the DMA of the next segment's first
    // sub-tile into buffer 0 may already be in flight) take dV, written as the
    // accumulators hold them (four features of one key per lane). Both are written first, which frees the accumulator
    // registers; then they are read back along the rows, so that each store
    // instruction writes whole rows (full cache lines) instead of a 16-byte
    // piece of 32 rows.
    // (per-lane base offsets made opaque here, so that the compiler does not
    // hoist them out of the segment loop and keep them in spilled registers)
    int wofs = (32 * a + l32) * G::DP + 4 * hh, rofs = (32 * a + lane / (G::D / 8)) * G::DP + 8 * (lane % (G::D / 8));
    asm volatile("" : "+v"(wofs), "+v"(rofs));
    bf16* stg_k = L.kt();
    bf16* stg_v = G::V_LDS ? L.v() : (bf16*)L.q(1);
#pragma unroll
    for (int n = 0; n < ND; ++n) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = to_bf16(dKa[n][4 * g + e] * p.scale);
          v4[e] = to_bf16(dVa[n][4 * g + e]);
        }
        *(bf16x4*)(stg_k + wofs + 32 * n + 8 * g) = k4;
        *(bf16x4*)(stg_v + wofs + 32 * n + 8 * g) = v4;
        __builtin_amdgcn_sched_barrier(0);  // convert and write one quad at a time (registers)
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are written
    constexpr int LPR = G::D / 8, RPI = 64 / LPR;  // lanes per row, rows per instruction
    const int key0 = sg.kv * G::T + 32 * a;
    const size_t out0 = ((size_t)sg.bh * p.S + key0) * G::D;  // wave-uniform
    int grow = lane / LPR;                                      // this lane's row of the first instruction
    unsigned gofs = (unsigned)(grow * G::D + 8 * (lane % LPR)) * 2u;
    asm volatile("" : "+v"(grow), "+v"(gofs));
#pragma unroll
    for (int r = 0; r < 32 / RPI; ++r) {
      const bf16x8 k8 = *(const bf16x8*)(stg_k + rofs + RPI * r * G::DP);
      const bf16x8 v8 = *(const bf16x8*)(stg_v + rofs + RPI * r * G::DP);
      if (key0 + grow + RPI * r < p.S) {
        *at_bytes((bf16x8*)(p.dk + out0), gofs + (unsigned)(RPI * r * G::D * 2)) = k8;
        *at_bytes((bf16x8*)(p.dv + out0), gofs + (unsigned)(RPI * r * G::D * 2)) = v8;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// ---- dQ waves

template <class G, bool CAUSAL, int MODE>
struct DqRole {
  static constexpr bool ATOMIC = MODE == MODE_ATOMIC;
  static constexpr bool XCD = MODE == MODE_XCD;
  static constexpr int QBW = G::QBW, TC = G::TC, NSUB = G::NSUB, BR = G::BR, D = G::D;
  const MainParams& p;
  Lds<G> L;
  int tb, lane, b, l32, hh, mb, nb0;
  bf16x8 Kd[QBW][TC];   // B operand of dQ: this wave's feature columns, all keys of the tile
  bf16x8 dsA[TC];       // A operand of dQ: dS rows of this wave's row block
  // Full-mask Shift with the XCD-local hand-off: the running sums of a
  // sub-tile are loaded in the next interval's part1, after the staging DMA
  // (which then no longer queues behind them); where contributors wait on
  // each other's turns (the other schedules, the causal mask, the device-wide
  // hand-off) the loads go right after the turn, as early as they can.
  bool late_loads = false;
  int pend = -1;      // flag this wave still owes a hand-over on
  int pend_val = 0;   // the value it will write there
  WaitClock* wc = nullptr;  // profiling build only

  __device__ __forceinline__ DqRole(const MainParams& p_, Lds<G> L_) : p(p_), L(L_) {
    tb = threadIdx.x - G::NTA;
    lane = tb & 63;
    b = __builtin_amdgcn_readfirstlane(tb >> 6);
    l32 = lane & 31;
    hh = lane >> 5;
    constexpr int per_row = G::ND / QBW;
    mb = b / per_row;
    nb0 = QBW * (b % per_row);
    late_loads = XCD && !CAUSAL && p.sched == SCHED_SHIFT;
  }

  // LDS DMA of query rows q0 .. q0 + BR - 1 of head bh into staging buffer
  // buf. Each instruction fills 1 KB of the buffer, lane L the 16 bytes at
  // offset 16 L, so lane L fetches the chunk that the swizzle puts there. Rows
  // past the end of the sequence are read as copies of the last row (the masks
  // give them P = 0 exactly). LSE and Delta: one dword per lane.
  __device__ __forceinline__ void stage(int bh, int q0, int buf) {
    constexpr int CPR = G::D / 8, RPP = 64 / CPR, HALF = G::PIECES / 2;
    const int S = p.S;
    const bf16* qh = p.q + (size_t)bh * S * G::D;
    const bf16* oh = p.dout + (size_t)bh * S * G::D;
    // row r = RPP pr + rl: swz(r) = swz(RPP pr) ^ swz(rl) (disjoint bits)
    int rl = lane / CPR, lx = (lane % CPR) ^ swz<G::D>(lane / CPR);
    asm volatile("" : "+v"(rl), "+v"(lx));
#pragma unroll
    for (int k = 0; k < G::PPW; ++k) {
      const int piece = b * G::PPW + k;  // wave-uniform
      const bool is_o = piece >= HALF;
      const int pr = is_o ? piece - HALF : piece;
      const unsigned off =
          (unsigned)(min(q0 + pr * RPP + rl, S - 1) * G::RB + 16 * (lx ^ swz<G::D>(pr * RPP)));
      char* dst = (is_o ? L.o(buf) : L.q(buf)) + pr * 1024;
      __builtin_amdgcn_global_load_lds(at_bytes(is_o ? oh : qh, off), (__attribute__((address_space(3))) void*)dst, 16, 0,
                                       0);
    }
    if (b < 2) {
      const float* src = (b == 0 ? p.lse2 : p.delta) + (size_t)bh * p.S_pad;  // uniform
      float* dst = b == 0 ? L.lse(buf) : L.dl(buf);
#pragma unroll
      for (int k = 0; k < G::BR / 64; ++k)
        __builtin_amdgcn_global_load_lds(at_bytes(src, 4u * (unsigned)(q0 + 64 * k + lane)),
                                         (__attribute__((address_space(3))) void*)(dst + 64 * k), 4, 0, 0);
    }
  }
  // the DMA issued by this wave (and every older vector memory operation) has completed
  // (the wait is a builtin, not inline asm, so that the compiler knows the
  // staged rows have landed and puts no waits of its own before LDS reads)
  __device__ __forceinline__ static void stage_wait() { wait_vmem(); }

  __device__ __forceinline__ int sub_row0(const Seg& sg, int i) const {
    const Task t = sched_task(p.N, CAUSAL, p.sched, sg.wk, sg.task<NSUB>(i));
    return t.q * G::T + sg.half<NSUB>(i) * BR;
  }

  __device__ __forceinline__ void read_ds() {
    const int grp = lane >> 4, gi = lane & 15;
    const bf16* base =
        &L.dst()[(8 * (grp >> 1) + (gi >> 2)) * G::SP + 32 * mb + 16 * (grp & 1) + 4 * (gi & 3)];
#pragma unroll
    for (int c = 0; c < TC; ++c)
      dsA[c] = cat44(lds_read_tr(base + 16 * c * G::SP), lds_read_tr(base + (16 * c + 4) * G::SP));
  }

  // A hand-off flag as one wave-uniform value. XCD-local: every contributor of
  // the tile runs on this XCD, so its L2 holds the flag; across XCDs: a
  // system-scope load.
  __device__ __forceinline__ int flag_read(int* f) const {
    return __builtin_amdgcn_readfirstlane(XCD ? l2_load(f) : sys_load(f));
  }

  // Once every dQ update this wave issued has completed, tell the next
  // contributor of the same blocks that it may go ahead.
  __device__ __forceinline__ void release() {
    if (!ATOMIC && pend >= 0) {
      // (profiling build: the counter is read before the wait below, so its
      // latency hides behind that of the stores)
      int now = 0;
      if constexpr (kProfileWait) now = XCD ? l2_load(&p.flags[pend]) : sys_load(&p.flags[pend]);
      wait_vmem();
      if constexpr (kProfileWait) {
        if (__builtin_amdgcn_readfirstlane(now) != pend_val - 1 && lane == 0) atomicAdd(&g_order_violations, 1u);
      }
      if (lane == 0) {
        if (XCD) l2_store(&p.flags[pend], pend_val);
        else sys_store(&p.flags[pend], pend_val);
      }
      pend = -1;
    }
  }

  __device__ __forceinline__ void seg_begin(const Seg& sg) { stage(sg.bh, sub_row0(sg, 0), 0); }

  __device__ __forceinline__ void seg_kd(const Seg&) {
    // K^T columns through the transpose read from the row-major K rows: lane i
    // of a 16-lane group gets four consecutive keys of feature column cb + i
    const bf16* kt = L.kt();
    const int grp = lane >> 4, gi = lane & 15;
#pragma unroll
    for (int j = 0; j < QBW; ++j) {
      const int cb = 32 * (nb0 + j) + 16 * (grp & 1) + 4 * (gi & 3);
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        const bf16* r0 = &kt[(16 * c + 8 * (grp >> 1) + (gi >> 2)) * G::DP + cb];
        Kd[j][c] = cat44(lds_read_tr(r0), lds_read_tr(r0 + 4 * G::DP));
      }
    }
  }

  // Sub-tile 0 has landed. (Sub-tile 1 is staged inside the loop, by part1 of
  // sub-tile 0: no DMA is then in flight where the loop is entered, so the
  // compiler needs no wait of its own before the loop's LDS reads.)
  __device__ __forceinline__ void seg_stage(const Seg&) { stage_wait(); }

  // The hand-off of sub-tile j runs in three steps (part1 and part2 below say
  // in which intervals):
  //   acquire: where the partial goes; wait for the turn; start the loads of
  //            the running sum;
  //   commit:  add and store (or the atomic RMWs; the last contributor writes
  //            bf16 dq instead);
  //   release: once the stores have completed, hand over to the next
  //            contributor (write its value into this wave's flag).
  f32x16 acc[QBW], prev[QBW];
  int h_flag = 0, h_r = 0;
  bool h_last = true;
  float* h_row = nullptr;
  bf16* h_dq = nullptr;  // the sub-tile's first row of dq
  int h_rows = 0;        // its rows within the sequence

  // The dQ products take their operands in the order (K columns, dS rows), so
  // each 32 x 32 accumulator holds a block of dQ^T: lane l owns query row
  // l mod 32 and, per register quad g, the four consecutive feature columns
  // 8g + 4 (l / 32) + 0..3 (four bf16 of dq are one 8-byte piece of a row).
  // The accumulator is stored in the MFMA's own register order: per query
  // sub-tile, 32 x 32 blocks (row block mb, feature block nb) of 1024 floats.
  // Every contributor of a block holds it in the same lanes, so
  //  - deterministic modes, "quad-major": accumulators 4g..4g+3 of lane l at
  //    (g * 64 + l) * 4: each 16-byte access of a wave covers 1 KB;
  //  - the atomic variant, "element-major": accumulator e of lane l at
  //    e * 64 + l: each atomic instruction covers 256 contiguous bytes.
  __device__ __forceinline__ unsigned blk_base(int j) const { return 4096u * (unsigned)(mb * G::ND + nb0 + j); }
  __device__ __forceinline__ unsigned elem_off(int j, int e) const { return blk_base(j) + 4u * (64 * e + lane); }
  __device__ __forceinline__ unsigned quad_off(int j, int g) const { return blk_base(j) + 16u * (64 * g + lane); }

  // dQ partial of sub-tile j from the dS rows in registers
  __device__ __forceinline__ void dq_mma() {
#pragma unroll
    for (int x = 0; x < QBW; ++x) {
      acc[x] = zero16();
#pragma unroll
      for (int c = 0; c < TC; ++c) acc[x] = mfma32(Kd[x][c], dsA[c], acc[x]);
    }
  }

  // where sub-tile j's partial goes; wait for its turn; start the running-sum loads
  __device__ __forceinline__ void acquire(const Seg& sg, int j) {
    const Task t = sched_task(p.N, CAUSAL, p.sched, sg.wk, sg.task<NSUB>(j));
    // this wave's flag for the sub-tile: dQ wave b of every contributor updates
    // the same blocks of the accumulator, so it waits only for wave b of the
    // previous contributor
    h_flag = sg.bh * p.flag_stride + (t.q * NSUB + sg.half<NSUB>(j)) * G::NB + b;
    h_r = ATOMIC ? 0 : sched_rank(p.N, CAUSAL, p.sched, t.q, sg.kv);
    h_last = ATOMIC ? true : (h_r == sched_contributors(p.N, CAUSAL, t.q) - 1);
    const int q0 = t.q * G::T + sg.half<NSUB>(j) * BR;
    h_row = p.dq_ws + ((size_t)sg.bh * p.S_pad + q0) * D;  // uniform
    h_dq = p.dq + ((size_t)sg.bh * p.S + q0) * D;
    h_rows = p.S - q0;
    if (ATOMIC || h_r == 0) return;
    // wait until the previous contributor's wave b has handed over (flag == r)
    const int target = h_r + (h_flag == p.poison_flag ? 0x40000000 : 0);
    const unsigned long long w0 = wclock();
    int* const fl = &p.flags[h_flag];
    int seen = flag_read(fl);
    uint32_t it = 0;
    while (seen != target) {
      if constexpr (kProfileWait) {
        if (seen > target) {  // handed over past this contributor's rank
          if (lane == 0) atomicAdd(&g_order_violations, 1u);
          break;
        }
      }
      if (++it >= p.wait_limit) {
        if (lane == 0) note_timeout(p.header);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      seen = flag_read(fl);
    }
    if constexpr (kProfileWait) wc->turn += wclock() - w0;
    if (!late_loads) load_sums();
  }
  // start the loads of the acquired sub-tile's running sum (none for its first
  // contributor or the atomic variant)
  __device__ __forceinline__ void load_sums() {
    if (ATOMIC || h_r == 0) return;
    // XCD-local: every contributor of this tile runs on this XCD, so its L2
    // holds the accumulator coherently for all of them: read the running sum
    // there. Across XCDs: read it from the device-wide coherence point.
#pragma unroll
    for (int x = 0; x < QBW; ++x) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = XCD ? l2_load16(h_row, 4u * BR * D, quad_off(x, g))
                            : sys_load16(h_row, 4u * BR * D, quad_off(x, g));
#pragma unroll
        for (int k = 0; k < 4; ++k) prev[x][4 * g + k] = v[k];
      }
    }
  }

  __device__ __forceinline__ void commit() {
    if (ATOMIC) {
#pragma unroll
      for (int x = 0; x < QBW; ++x) {
#pragma unroll
        for (int e = 0; e < 16; ++e) atomicAdd(at_bytes(h_row, elem_off(x, e)), acc[x][e]);
      }
      return;
    }
    if (h_last) {
      // The sub-tile's final sum: its last contributor writes dq = bf16(scale x
      // sum) into dq itself (the conversion the post-pass does for the atomic
      // variant), and no fp32 sum: quad g of block x is the 8-byte piece of
      // row 32 mb + l32 at feature column 32 (nb0 + x) + 8g + 4hh.
      // (one opaque per-lane base and constant offsets)
      int lrow = 32 * mb + l32;
      unsigned lofs = 2u * (unsigned)(lrow * D + 32 * nb0 + 4 * hh);
      asm volatile("" : "+v"(lrow), "+v"(lofs));
      if (lrow < h_rows) {
#pragma unroll
        for (int x = 0; x < QBW; ++x) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 b;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              b[k] = to_bf16((h_r > 0 ? prev[x][4 * g + k] + acc[x][4 * g + k] : acc[x][4 * g + k]) * p.scale);
            *at_bytes((bf16x4*)h_dq, lofs + 2u * (unsigned)(32 * x + 8 * g)) = b;
          }
        }
      }
      return;
    }
    if (XCD) {
      // (the first contributor stores its partial as it is)
#pragma unroll
      for (int x = 0; x < QBW; ++x) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = h_r > 0 ? prev[x][4 * g + k] + acc[x][4 * g + k] : acc[x][4 * g + k];
          *at_bytes((f32x4*)h_row, quad_off(x, g)) = v;
        }
      }
    } else {
      // Across XCDs: system-scope stores of the new running sum (written
      // through to the device-wide coherence point); the first contributor
      // stores its partial as it is.
#pragma unroll
      for (int x = 0; x < QBW; ++x) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = h_r > 0 ? prev[x][4 * g + k] + acc[x][4 * g + k] : acc[x][4 * g + k];
          sys_store16(h_row, 4u * BR * D, quad_off(x, g), v);
        }
      }
    }
    asm volatile("" ::: "memory");
    pend = h_flag;  // (not the last contributor: the next one waits for this)
    pend_val = h_r + 1;
  }

  // The hand-off of sub-tile j is spread over two intervals so that the
  // tile waves never wait at barrier X for dQ work and every memory latency
  // has time to pass:
  //   interval j+1, before X: dS of j to registers (the tile waves overwrite
  //            dS^T after X); after X: dQ = dS K, wait for the turn, start the
  //            running-sum loads;
  //   interval j+2, after X:  add and store; hand over once the stores have
  //            completed, which the dQ MFMAs of j+1 leave time for.
  // Before X a dQ wave only reads the previous sub-tile's dS out of LDS and
  // issues the DMA of the next sub-tile's rows. A wave hands sub-tile j over before it waits for its turn on j+1, so each
  // wait depends only on hand-overs that no later wait of their wave precedes:
  // with cyclic schedules (Shift, Symmetric Shift) this is what keeps the waits
  // free of cycles.
  // The dQ waves also stage the query rows: sub-tile i+1 goes into the other
  // buffer (its last readers passed the previous barrier Y) while sub-tile i
  // is computed, and has landed before barrier Y.
  __device__ __forceinline__ void part1(const Seg& sg, int i) {
    if (i > 0) read_ds();
    if (i + 1 < sg.n) stage(sg.bh, sub_row0(sg, i + 1), (i + 1) & 1);
    if (late_loads && i > 1) load_sums();  // sub-tile i-2, acquired in the previous part2
  }

  __device__ __forceinline__ void part2(const Seg& sg, int i) {
    // sub-tile i+1's rows and the running sums of i-2 (loaded an interval
    // ago). Waited for on every path, also where nothing was staged, so that
    // the compiler sees no DMA in flight at the loop head and puts no wait of
    // its own before the next dS reads (which would hold them, and the DMA
    // issued after them, until the running-sum loads of this interval arrive).
    stage_wait();
    if (i > 1) commit();              // sub-tile i-2
    if (i > 0) dq_mma();              // sub-tile i-1
    release();                        // sub-tile i-2
    if (i > 0) acquire(sg, i - 1);    // sub-tile i-1
  }

  __device__ __forceinline__ void seg_end(const Seg& sg) {
    read_ds();                        // dS of the last sub-tile
    if (sg.n > 1) {
      if (late_loads) load_sums();
      commit();                       // sub-tile n-2
    }
    dq_mma();                         // sub-tile n-1
    release();
    acquire(sg, sg.n - 1);
    if (late_loads) load_sums();
    commit();
    release();
  }
};

// ---- the shared unit / segment / sub-tile skeleton (identical barrier sequence for both roles)

#ifndef ATTN_SUBTILE_PASSES
#define ATTN_SUBTILE_PASSES 1
#endif
constexpr bool PASSES = ATTN_SUBTILE_PASSES != 0;

#ifndef ATTN_HEAD_INTERLEAVE
#define ATTN_HEAD_INTERLEAVE 0  // 0: by the rule below; otherwise that many heads
#endif

// Heads interleaved in an XCD queue for naive and Descending: 4, 2 or 1, the
// most that keeps heads x workers within 256 on a causal mask and within 64
// on a full one. (Interleaved runs on the 4k and 8k causal and the 2k, 4k and
// 16k full shapes: more heads at once fill the gaps of the serial dQ chains;
// past that bound the running sums of the heads in flight no longer stay in
// the XCD's L2 between contributors, and the 16k full mask slows down.)
inline int head_interleave(bool causal, int n_workers) {
  if (ATTN_HEAD_INTERLEAVE > 0) return ATTN_HEAD_INTERLEAVE;
  const int cap = causal ? 256 : 64;
  int g = 4;
  while (g > 1 && g * n_workers > cap) g /= 2;
  return g;
}

#ifndef ATTN_ATOMIC_XCD_QUEUE
#define ATTN_ATOMIC_XCD_QUEUE 1
#endif

// A head slot of an XCD queue once its run's first ticket has published it
// (p.BH, and the call marked failed, if the wait bound runs out first).
__device__ __forceinline__ int wait_slot(const MainParams& p, int* slot) {
  int v;
  uint32_t it = 0;
  while ((v = l2_load(slot)) < 0) {
    if (++it >= p.wait_limit) {
      note_timeout(p.header);
      return p.BH;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return v;
}

template <class G, bool CAUSAL, int MODE, class Role>
__device__ __forceinline__ void run_units(const MainParams& p, const Lds<G>& L, Role& role) {
  // Per-XCD queues: the XCD-local hand-off needs every contributor of a head
  // on one XCD; the atomic variant uses them too, so that a head's atomic
  // adds land in one XCD's L2 (it never waits, so any placement is safe).
  constexpr bool XCD = MODE == MODE_XCD || (MODE == MODE_ATOMIC && ATTN_ATOMIC_XCD_QUEUE != 0);
  int xq = 0;  // this workgroup's XCD, the queue it takes units from
  if (XCD) {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    xq = (int)(x & (kMaxQueues - 1));
  }
  // The unit a workgroup runs next: [0] head, [1] worker, [2] how many units
  // thread 0 has published (LDS starts undefined).
  int* sUnit = L.unit();
  if (threadIdx.x == 0) sUnit[2] = 0;
  lds_barrier();
  int seq = 0;
  WaitClock wclk;
  if constexpr (kProfileWait) role.wc = &wclk;
  const unsigned long long t_start = wclock();
  unsigned long long n_sub = 0;
  for (;;) {
    const unsigned long long c0 = wclock();
    ++seq;
    // Thread 0 claims the next unit as soon as its own wave has finished the
    // previous one and publishes it through LDS; the other waves wait only
    // for that word, not at a barrier, so the tile waves claim and load the
    // next K/V tile while the dQ waves still hand the last sub-tile over
    // (they meet at the segment's first barrier). One slot suffices: thread 0
    // reaches the next claim only after the segment's barriers, which every
    // wave passes after reading this unit.
    if (threadIdx.x == 0) {
      if (!XCD) {
        const int u = atomicAdd(&p.header[0], 1);
        sUnit[0] = u < p.n_units ? u / p.n_workers : p.BH;
        sUnit[1] = u % p.n_workers;
      } else {
        // Units of one head are consecutive tickets of one XCD's queue or,
        // with ilv > 1, ilv heads take turns within each run of ilv x workers
        // tickets (worker 0 of each, then worker 1 of each, ...): where a
        // worker waits only on the workers before it (naive, Descending),
        // workgroups freed together then start on several heads at once
        // instead of lining up behind one head's hand-offs. The first ticket
        // of a run claims the run's ilv heads (an atomic shared by all XCDs)
        // once the queue's previous run has claimed, so the heads of a queue
        // only grow along it, and publishes the first of them through this
        // XCD's L2 for the run's other tickets. Each wait here is for a lower
        // ticket of the same queue, held by a running workgroup that
        // publishes right after its atomic, so it ends. A ticket whose slot
        // lies past the last head takes another ticket; a run that starts
        // past it ends the queue for every later ticket as well.
        int head, wk;
        for (;;) {
          const int k = atomicAdd(&p.header[16 + xq], 1);
          const int span = p.ilv * p.n_workers, grp = k / span, rem = k - grp * span;
          wk = rem / p.ilv;
          int first = p.BH;  // the run's first head
          if (grp < p.BH) {
            int* slot = &p.heads[xq * p.heads_row + grp];
            if (rem == 0) {
              if (grp == 0 || wait_slot(p, slot - 1) < p.BH) first = min(atomicAdd(&p.header[2], p.ilv), p.BH);
              l2_store(slot, first);
            } else {
              first = wait_slot(p, slot);
            }
          }
          head = first >= p.BH ? p.BH : first + rem % p.ilv;
          if (head < p.BH || first >= p.BH) break;  // a unit, or the end of the queue
        }
        sUnit[0] = head;
        sUnit[1] = wk;
      }
      __hip_atomic_store(&sUnit[2], seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&sUnit[2], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) != seq)
      __builtin_amdgcn_s_sleep(1);
    if constexpr (kProfileWait) wclk.claim += wclock() - c0;
    const int bh = __builtin_amdgcn_readfirstlane(sUnit[0]);
    // Causal Shift: dQ tile i receives KV tiles i, i-1, ..., 0 in that order,
    // so worker j waits on worker j+1 at every step. Dealing a head's workers
    // last KV tile first starts every predecessor before its successor; in
    // ascending order the workers of a head that start one after another (as
    // a previous head's shortest units drain) line up on the same dQ tiles
    // and their hand-offs serialise.
    const int wk_pos = __builtin_amdgcn_readfirstlane(sUnit[1]);
    const int wk = (CAUSAL && p.sched == SCHED_SHIFT && MODE != MODE_ATOMIC) ? p.n_workers - 1 - wk_pos : wk_pos;
    if (bh >= p.BH) break;
    const int ntasks = sched_num_tasks(p.N, CAUSAL, p.sched, wk);

    // the (at most two) KV tiles of this unit and the last task on each
    int tileA = -1, lastA = -1, lastB = -1;
    for (int t = 0; t < ntasks; ++t) {
      const int kv = sched_task(p.N, CAUSAL, p.sched, wk, t).kv;
      if (tileA < 0 || kv == tileA) {
        tileA = kv;
        lastA = t;
      } else {
        lastB = t;
      }
    }
    bool parkedA = false, parkedB = false;
    for (int t0 = 0; t0 < ntasks;) {
      const int kv = sched_task(p.N, CAUSAL, p.sched, wk, t0).kv;
      int t1 = t0 + 1;
      while (t1 < ntasks && sched_task(p.N, CAUSAL, p.sched, wk, t1).kv == kv) ++t1;
      Seg sg;
      sg.bh = bh;
      sg.wk = wk;
      sg.t0 = t0;
      sg.n = (t1 - t0) * G::NSUB;
      sg.kv = kv;
      const bool isA = kv == tileA;
      sg.slot = isA ? 0 : 1;
      sg.restore = isA ? parkedA : parkedB;
      sg.keep = (isA ? lastA : lastB) >= t1;
      // passes over the sub-tiles: Shift on a full mask, where every worker of a
      // head is on a different query tile at every step (measured: 6-9% faster
      // there; neutral to 2.5% slower for naive and Descending, much slower for
      // Shift on a causal mask, whose workers walk runs of different lengths)
      sg.passes = PASSES && !CAUSAL && p.sched == SCHED_SHIFT;
      if (isA) parkedA = sg.keep;
      else parkedB = sg.keep;

      const unsigned long long s0 = wclock();
      role.seg_begin(sg);  // tile waves: K/V, K^T to LDS, accumulators; dQ waves: load sub-tile 0
      lds_barrier();
      role.seg_kd(sg);     // dQ waves: K columns from LDS
      lds_barrier();
      role.seg_stage(sg);  // dQ waves: sub-tile 0 has landed
      lds_barrier();
      const unsigned long long s1 = wclock();
      // (sg.n >= 1: the body runs at least once, which also tells the
      // compiler that the accumulators loaded in seg_begin have arrived by
      // seg_end, so the epilogue's stores need no waits for them)
      int i = 0;
      do {
        role.part1(sg, i);
        const unsigned long long b0 = wclock();
        lds_barrier();  // X
        const unsigned long long b1 = wclock();
        role.part2(sg, i);
        const unsigned long long b2 = wclock();
        lds_barrier();  // Y
        if constexpr (kProfileWait) {
          wclk.bar += (b1 - b0) + (wclock() - b2);
          ++n_sub;
        }
      } while (++i < sg.n);
      const unsigned long long s2 = wclock();
      role.seg_end(sg);    // tile waves: park or write dK/dV; dQ waves: last sub-tile's dQ
      if constexpr (kProfileWait) {
        wclk.seg += (s1 - s0) + (wclock() - s2);
        ++wclk.nseg;
      }
      t0 = t1;
    }
  }
  if constexpr (kProfileWait) {
    const unsigned long long total = wclock() - t_start;
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0 && blockIdx.x < kMaxGrid) {
      if (wave == 0) {
        g_wait_prof[blockIdx.x][0] = wclk.bar;
        g_wait_prof[blockIdx.x][1] = total;
        g_wait_prof[blockIdx.x][6] = wclk.seg;
        g_wait_prof[blockIdx.x][7] = wclk.nseg;
        g_wait_prof[blockIdx.x][8] = wclk.claim;
      } else if (wave == G::NA) {
        g_wait_prof[blockIdx.x][2] = wclk.turn;
        g_wait_prof[blockIdx.x][3] = wclk.bar;
        g_wait_prof[blockIdx.x][4] = total;
        g_wait_prof[blockIdx.x][5] = n_sub;
      }
    }
  }
}

template <int D, int T, int BR, bool CAUSAL, int MODE>
__global__ void __launch_bounds__(T / 16 * 64) bwd_main_kernel(MainParams p) {
  using G = Geo<D, T, BR>;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  const Lds<G> L{smem};
  if ((int)(threadIdx.x >> 6) < G::NA) {
    TileRole<G, CAUSAL, MODE> role(p, L);
    run_units<G, CAUSAL, MODE>(p, L, role);
  } else {
    DqRole<G, CAUSAL, MODE> role(p, L);
    run_units<G, CAUSAL, MODE>(p, L, role);
  }
}

// --------------------------------------------------------------------------------------
// post-pass: the failure check; for the atomic variant dq = bf16(scale * dQ accumulator)

// A tripped wait bound (header[1], set by the main kernel) makes the call's
// results unusable: the dQ order may have been broken. The passes after the
// main kernel then write NaN into every output instead of values, so the
// failure shows in the gradients themselves, with no host synchronisation.
__device__ __forceinline__ bool call_failed(const int* header) {
  return __hip_atomic_load(&header[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__device__ __forceinline__ void fill_nan(bf16* x, long long n, long long t0, long long nthreads) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(bf16, (unsigned short)0x7FC0);
  for (long long i = t0; i < n / 8; i += nthreads) *(bf16x8*)(x + 8 * i) = v;
}

template <int D>
__global__ void __launch_bounds__(256) bwd_post_kernel(const float* dq_ws, bf16* dq, bf16* dk, bf16* dv,
                                                       const int* header, long long BH, int S, int S_pad,
                                                       int convert, float scale, long long kv_elems) {
  // Fills dq, dk and dv with NaN if the main kernel gave up a wait. Else, for
  // the atomic variant (convert != 0; the deterministic modes write dq in the
  // main kernel), converts its sums: dq_ws holds, per 32 query rows of a
  // head, D / 32 blocks of 32 x 32 in MFMA register order (element-major within
  // a block, see the dQ waves), contiguous. A workgroup takes one such row
  // block: each thread converts the accumulators 4g..4g+3 of one lane (four
  // features of one row) into an LDS tile, then writes whole rows, 16 bytes
  // per thread.
  constexpr int ND = D / 32, NQ = 32 * D / 4 / 256, NC = 32 * D / 8 / 256, TP = D + 8;
  __shared__ __attribute__((aligned(16))) bf16 tile[32 * TP];
  const long long t0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nthreads = (long long)gridDim.x * blockDim.x;
  if (call_failed(header)) {
    fill_nan(dq, BH * S * D, t0, nthreads);
    fill_nan(dk, kv_elems, t0, nthreads);
    fill_nan(dv, kv_elems, t0, nthreads);
    return;
  }
  if (!convert) return;  // (the deterministic modes: the main kernel wrote dq)
  const int rbh = S_pad / 32;  // row blocks per head
  for (long long rb = blockIdx.x; rb < BH * rbh; rb += gridDim.x) {  // workgroup-uniform
    const long long bh = rb / rbh;
    const int r0 = (int)(rb - bh * rbh) * 32;
    const float* src = dq_ws + (bh * S_pad + r0) * D;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = threadIdx.x + 256 * j;  // f32x4 q of the row block: block q / 256, quad g, lane
      const int blk = q >> 8, g = (q >> 6) & 3, lane = q & 63;
      f32x4 v;
      // (element-major: the atomic variant's layout)
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = src[blk * 1024 + (4 * g + k) * 64 + lane];
      // (blocks of dQ^T: lane l holds row l mod 32, features 8g + 4 (l / 32) + 0..3)
      const int row = lane & 31, col = 32 * blk + 8 * g + 4 * (lane >> 5);
      bf16x4 b;
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = to_bf16(v[k] * scale);
      *(bf16x4*)&tile[row * TP + col] = b;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = threadIdx.x + 256 * j;
      const int row = c / (D / 8), part = c % (D / 8);
      if (r0 + row < S) *(bf16x8*)(dq + (bh * S + r0 + row) * D + 8 * part) = *(const bf16x8*)&tile[row * TP + 8 * part];
    }
    __syncthreads();  // (the next row block reuses the tile)
  }
  static_assert(ND * 32 == D && NQ * 256 * 4 == 32 * D && NC * 256 * 8 == 32 * D, "row block split");
}

// --------------------------------------------------------------------------------------
// launcher

// --------------------------------------------------------------------------------------
// grouped-query epilogue: dK, dV of K/V head hk = the sum over its G query heads
// hk G, ..., hk G + G - 1, added in that order (a fixed order: deterministic)

__global__ void __launch_bounds__(256) bwd_gqa_reduce_kernel(const float* dkv, bf16* dk, bf16* dv, const int* header,
                                                             int H, int Hkv, int S, int S_pad, int D, long long BH) {
  const int G = H / Hkv;
  const long long quads = (long long)(BH / H) * Hkv * S * (D / 4);  // output elements / 4
  const long long part = BH * S_pad * D;                             // floats per tensor of dkv
  const long long nthreads = (long long)gridDim.x * blockDim.x;
  const long long t0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (call_failed(header)) {  // the post-pass has written NaN into dq; dk and dv follow
    fill_nan(dk, quads * 4, t0, nthreads);
    fill_nan(dv, quads * 4, t0, nthreads);
    return;
  }
  for (long long t = t0; t < quads; t += nthreads) {
    const long long e = t * 4;                   // output element: ((b Hkv + hk) S + s) D + d
    const long long row = e / D;                 // (b Hkv + hk) S + s
    const int d = (int)(e - row * D);
    const long long bk = row / S;                // b Hkv + hk
    const int s = (int)(row - bk * S);
    const long long b = bk / Hkv, hk = bk - b * Hkv;
    const long long h0 = b * H + hk * G;         // first query head of the group
    f32x4 ak = {0.0f, 0.0f, 0.0f, 0.0f}, av = ak;
    for (int g = 0; g < G; ++g) {
      const long long src = ((h0 + g) * S_pad + s) * D + d;
      const f32x4 xk = *(const f32x4*)(dkv + src);
      const f32x4 xv = *(const f32x4*)(dkv + part + src);
      ak += xk;
      av += xv;
    }
    bf16x4 ok, ov;
    for (int k = 0; k < 4; ++k) {
      ok[k] = to_bf16(ak[k]);
      ov[k] = to_bf16(av[k]);
    }
    *(bf16x4*)(dk + e) = ok;
    *(bf16x4*)(dv + e) = ov;
  }
}

template <int D, int T, int BR, bool CAUSAL, int MODE>
static hipError_t launch_main(const MainParams& mp, int grid, hipStream_t stream) {
  g_last_grid = grid;
  hipLaunchKernelGGL((bwd_main_kernel<D, T, BR, CAUSAL, MODE>), dim3((unsigned)grid), dim3(T / 16 * 64), 0, stream,
                     mp);
  return hipGetLastError();
}

template <int D, int T, int BR, bool CAUSAL>
static hipError_t launch_mask(const MainParams& mp, bool atomic, int num_cu, int protocol, hipStream_t stream) {
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, bwd_main_kernel<D, T, BR, CAUSAL, MODE_DEVICE>, T / 16 * 64, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  long long grid = (long long)num_cu * per_cu;
  if (grid > kMaxGrid) grid = kMaxGrid;
  if (grid > mp.n_units) grid = mp.n_units;
  // Cyclic dQ waits (Shift, Symmetric Shift) need every worker of a head
  // resident at once; the persistent grid must hold at least one head.
  const bool cyclic = mp.sched == SCHED_SHIFT || mp.sched == SCHED_SYMMETRIC_SHIFT;
  if (!atomic && cyclic && grid < mp.n_workers) return hipErrorInvalidConfiguration;
  // XCD-local hand-off: workgroup g runs on XCD g % 8 (gfx950, 8 XCDs per
  // device in SPX mode), so each XCD holds grid / 8 of the persistent
  // workgroups. Cyclic schedules need all workers of a head resident there.
  const int n_xcd = (num_cu >= 64 && num_cu % 8 == 0) ? 8 : 1;
  const long long per_xcd = grid / n_xcd;
  const bool xcd = !atomic && protocol != DQ_DEVICE && (!cyclic || mp.n_workers <= per_xcd);
  if (atomic) return launch_main<D, T, BR, CAUSAL, MODE_ATOMIC>(mp, (int)grid, stream);
  if (xcd) return launch_main<D, T, BR, CAUSAL, MODE_XCD>(mp, (int)grid, stream);
  return launch_main<D, T, BR, CAUSAL, MODE_DEVICE>(mp, (int)grid, stream);
}

template <int D, int T, int BR>
static hipError_t dispatch_mask(const MainParams& mp, bool causal, bool atomic, int num_cu, int protocol,
                                hipStream_t s) {
  return causal ? launch_mask<D, T, BR, true>(mp, atomic, num_cu, protocol, s)
                : launch_mask<D, T, BR, false>(mp, atomic, num_cu, protocol, s);
}

hipError_t launch_bwd(const BwdArgs& a, int num_cu, hipStream_t stream) {
  const long long BH = (long long)a.B * a.H;
  int* header = (int*)(a.ws + a.lay.header);
  int* flags = (int*)(a.ws + a.lay.flags);
  float* lse2 = (float*)(a.ws + a.lay.lse2);
  float* delta = (float*)(a.ws + a.lay.delta);
  float* dq_ws = (float*)(a.ws + a.lay.dq_ws);
  float* park = (float*)(a.ws + a.lay.park);
  int* heads = (int*)(a.ws + a.lay.heads);

  PreParams pp;
  pp.o = (const bf16*)a.o;
  pp.dout = (const bf16*)a.dout;
  pp.lse = a.lse;
  pp.lse2 = lse2;
  pp.delta = delta;
  pp.dq_ws = dq_ws;
  pp.flags = flags;
  pp.header = header;
  pp.heads = heads;
  pp.n_heads = (long long)kMaxQueues * a.lay.heads_row;
  pp.rows = BH * a.S_pad;
  pp.S = a.S;
  pp.S_pad = a.S_pad;
  pp.n_flags = BH * a.lay.flag_stride;
  pp.dq_ws_elems = a.atomic ? BH * a.S_pad * a.D : 0;
  if (a.S_pad % 32 != 0) return hipErrorInvalidValue;  // (S_pad = tiles x T; the post-pass takes 32 rows at a time)
  {
    const long long want = (pp.rows * (a.D / 8) + 255) / 256;
    const unsigned grid = (unsigned)(want < 4096 ? (want < 1 ? 1 : want) : 4096);
    if (a.D == 64) hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(grid), dim3(256), 0, stream, pp);
    else hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(grid), dim3(256), 0, stream, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  MainParams mp;
  mp.q = (const bf16*)a.q;
  mp.k = (const bf16*)a.k;
  mp.v = (const bf16*)a.v;
  mp.dout = (const bf16*)a.dout;
  mp.dk = (bf16*)a.dk;
  mp.dv = (bf16*)a.dv;
  mp.lse2 = lse2;
  mp.delta = delta;
  mp.dq_ws = dq_ws;
  mp.park = park;
  mp.flags = flags;
  mp.flag_stride = (int)a.lay.flag_stride;
  mp.heads_row = (int)a.lay.heads_row;
  // poisoning: the last dQ wave's flag of the last query sub-tile of the last head
  mp.poison_flag = (!a.atomic && a.poison) ? (int)((BH - 1) * a.lay.flag_stride + (long long)a.n_qsub * dq_waves(a.T) - 1) : -1;
  mp.header = header;
  mp.heads = heads;
  mp.dq = (bf16*)a.dq;
  mp.BH = (int)BH;
  mp.H = a.H;
  mp.group = a.H / a.Hkv;
  mp.dkv = mp.group > 1 ? (float*)(a.ws + a.lay.dkv) : nullptr;
  mp.S = a.S;
  mp.S_pad = a.S_pad;
  mp.N = a.N;
  mp.n_qsub = a.n_qsub;
  mp.sched = a.atomic ? SCHED_NAIVE : a.sched;
  mp.n_workers = sched_workers(a.N, mp.sched);
  mp.n_units = (int)(BH * mp.n_workers);
  mp.ilv = (!a.atomic && (mp.sched == SCHED_NAIVE || mp.sched == SCHED_DESCENDING)) ? head_interleave(a.causal != 0, mp.n_workers) : 1;
  mp.scale = a.scale;
  mp.scale_log2 = a.scale * 1.4426950408889634f;
  mp.wait_limit = a.wait_limit;

  hipError_t e = hipErrorInvalidValue;
  const bool causal = a.causal != 0, atomic = a.atomic != 0;
  if (a.ev_before && a.ev_after) {
    e = hipEventRecord(a.ev_before, stream);
    if (e != hipSuccess) return e;
  }
  if (a.D == 128 && a.T == 128) e = dispatch_mask<128, 128, 64>(mp, causal, atomic, num_cu, a.dq_protocol, stream);
  else if (a.D == 128 && a.T == 64) e = dispatch_mask<128, 64, 64>(mp, causal, atomic, num_cu, a.dq_protocol, stream);
  else if (a.D == 64 && a.T == 128) e = dispatch_mask<64, 128, 128>(mp, causal, atomic, num_cu, a.dq_protocol, stream);
  else if (a.D == 64 && a.T == 64) e = dispatch_mask<64, 64, 64>(mp, causal, atomic, num_cu, a.dq_protocol, stream);
  if (e != hipSuccess) return e;
  if (a.ev_before && a.ev_after) {
    e = hipEventRecord(a.ev_after, stream);
    if (e != hipSuccess) return e;
  }

  {
    // (deterministic modes: a check of the failure flag, and the NaN fill if set)
    const long long want = atomic ? BH * (a.S_pad / 32) : 1024;  // row blocks
    const unsigned g = (unsigned)(want < 16384 ? (want < 1 ? 1 : want) : 16384);
    // (grouped heads: dk and dv are written by the group sum below, which checks the flag itself)
    const long long kv_elems = mp.group > 1 ? 0 : BH * a.S * a.D;
    if (a.D == 64)
      hipLaunchKernelGGL(bwd_post_kernel<64>, dim3(g), dim3(256), 0, stream, dq_ws, (bf16*)a.dq, (bf16*)a.dk,
                         (bf16*)a.dv, (const int*)header, BH, a.S, a.S_pad, atomic ? 1 : 0, a.scale, kv_elems);
    else
      hipLaunchKernelGGL(bwd_post_kernel<128>, dim3(g), dim3(256), 0, stream, dq_ws, (bf16*)a.dq, (bf16*)a.dk,
                         (bf16*)a.dv, (const int*)header, BH, a.S, a.S_pad, atomic ? 1 : 0, a.scale, kv_elems);
    e = hipGetLastError();
  }
  if (e == hipSuccess && mp.group > 1) {
    const long long want = ((long long)a.B * a.Hkv * a.S * (a.D / 4) + 255) / 256;
    const unsigned g = (unsigned)(want < 8192 ? (want < 1 ? 1 : want) : 8192);
    hipLaunchKernelGGL(bwd_gqa_reduce_kernel, dim3(g), dim3(256), 0, stream, (const float*)mp.dkv, (bf16*)a.dk,
                       (bf16*)a.dv, (const int*)header, a.H, a.Hkv, a.S, a.S_pad, a.D, BH);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace attn

extern "C" int attn_debug_wait_profile(uint64_t* out, int max_workgroups) {
  if (!attn::kProfileWait) return ATTN_ERR_UNSUPPORTED;
  if (!out || max_workgroups <= 0) return ATTN_ERR_INVALID_ARG;
  static unsigned long long rows[attn::kMaxGrid][attn::kProfSlots];
  if (hipDeviceSynchronize() != hipSuccess) return ATTN_ERR_HIP;
  if (hipMemcpyFromSymbol(rows, HIP_SYMBOL(attn::g_wait_prof), sizeof(rows)) != hipSuccess) return ATTN_ERR_HIP;
  const int n = attn::g_last_grid < max_workgroups ? attn::g_last_grid : max_workgroups;
  for (int g = 0; g < n; ++g)
    for (int k = 0; k < attn::kProfSlots; ++k) out[attn::kProfSlots * g + k] = rows[g][k];
  return n;
}

extern "C" int attn_debug_order_violations(int reset) {
  if (!attn::kProfileWait) return ATTN_ERR_UNSUPPORTED;
  if (hipDeviceSynchronize() != hipSuccess) return ATTN_ERR_HIP;
  unsigned n = 0;
  if (hipMemcpyFromSymbol(&n, HIP_SYMBOL(attn::g_order_violations), sizeof(n)) != hipSuccess) return ATTN_ERR_HIP;
  if (reset) {
    const unsigned zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(attn::g_order_violations), &zero, sizeof(zero)) != hipSuccess)
      return ATTN_ERR_HIP;
  }
  return n > 0x7fffffffu ? 0x7fffffff : (int)n;
}

extern "C" int attn_debug_wait_timeouts(int reset) {
  if (hipDeviceSynchronize() != hipSuccess) return ATTN_ERR_HIP;
  int n = 0;
  if (hipMemcpyFromSymbol(&n, HIP_SYMBOL(attn::g_wait_timeouts), sizeof(n)) != hipSuccess) return ATTN_ERR_HIP;
  if (reset) {
    const int zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(attn::g_wait_timeouts), &zero, sizeof(zero)) != hipSuccess) return ATTN_ERR_HIP;
  }
  return n;
}
