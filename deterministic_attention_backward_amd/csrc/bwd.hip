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
// sub-tile later, when the adds have long completed) increment the counter. A
// post-pass converts the fp32 accumulator to bf16 dq.
#include "common.hpp"
#include "launch.hpp"
#include "schedule.hpp"

namespace attn {

// --------------------------------------------------------------------------------------
// pre-pass: Delta = rowsum(dO * O) in fp32, LSE in base 2, counters and ticket reset.

struct PreParams {
  const bf16 *o, *dout;
  const float* lse;
  float *lse2, *delta, *dq_ws;
  int *counters, *header, *heads;
  long long n_heads;    // entries of the head table
  long long rows;       // BH * S_pad
  int S, S_pad;
  long long n_counters;
  long long dq_ws_elems;  // > 0: zero the dQ accumulator (atomic variant)
  int poison;
};

template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(PreParams p) {
  constexpr int LPR = D / 8;  // lanes per row, 8 bf16 each
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nthreads = (long long)gridDim.x * blockDim.x;
  const int sub = threadIdx.x % LPR;
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
  // every counter starts at 0; the optional poison value (an unreachable turn,
  // used to exercise the wait bound) is written by the thread that owns that slot
  for (long long i = gtid; i < p.n_counters; i += nthreads)
    p.counters[i] = (p.poison && i == p.n_counters - 1) ? 0x40000000 : 0;
  if (gtid < 64) p.header[gtid] = 0;
  for (long long i = gtid; i < p.n_heads; i += nthreads) p.heads[i] = -1;
  for (long long i = gtid * 4; i < p.dq_ws_elems; i += nthreads * 4)
    *(f32x4*)(p.dq_ws + i) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// --------------------------------------------------------------------------------------
// main kernel
//
// Workgroup = T/32 waves; wave w owns keys 32w..32w+31 of the current KV tile.
// Registers hold, for the whole unit: this wave's K and V rows as the B
// operands of S = Q K^T and dP = dO V^T, the K columns it needs as the B
// operand of dQ = dS K, and the dK/dV accumulators. Per query sub-tile
// (BR rows) LDS holds Q and dO twice: row-major (A operands of S and dP) and
// transposed with the queries of every 16-row group permuted so that one
// 16-byte read yields a lane's eight k-values of the dV/dK B operand in the
// order the P/dS accumulators supply them. dS goes to LDS transposed (one
// 8-byte write per accumulator quad) and comes back through the gfx950
// transpose read as the A operand of dQ.

struct MainParams {
  const bf16 *q, *k, *v;
  const bf16* dout;
  bf16 *dk, *dv;
  const float *lse2, *delta;
  float *dq_ws, *park;
  bf16* dq;
  int *counters, *header, *heads;
  int S, S_pad, N, n_qsub, n_workers, n_units, sched, BH;
  float scale, scale_log2;
  uint32_t wait_limit;
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// supplies the address of a 4-element row chunk and receives element i % 4 of
// the chunks supplied by lanes 4e + i / 4, e = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// quads of each 16-query group in transposed LDS rows are stored in the order 0, 2, 1, 3
__device__ __forceinline__ int quad_pos(int qg) { return 16 * (qg >> 2) + 4 * ((qg & 1) * 2 + ((qg >> 1) & 1)); }

// How a unit hands its dQ partials over.
enum {
  MODE_ATOMIC = 0,  // non-deterministic: fp32 atomic adds in whatever order they land
  MODE_DEVICE = 1,  // deterministic: device-scope atomic RMWs serialised by the counters
  MODE_XCD = 2      // deterministic: all workers of a head on one XCD, plain RMW via its L2
};

template <int D, int T, int BR, bool CAUSAL, int MODE>
__global__ void __launch_bounds__(T / 32 * 64, 1) bwd_main_kernel(MainParams p) {
  constexpr bool ATOMIC = MODE == MODE_ATOMIC;
  constexpr bool XCD = MODE == MODE_XCD;
  constexpr int NW = T / 32;
  constexpr int NT = NW * 64;
  constexpr int DP = D + 8;        // row-major Q/dO rows (bf16 elements)
  constexpr int BRP = BR + 8;      // transposed Q/dO rows
  constexpr int TP = T + 8;        // transposed K rows
  constexpr int SP = BR + 4;       // transposed dS rows
  constexpr int KC = D / 16;       // k-chunks over the feature dimension
  constexpr int ND = D / 32;       // 32-wide feature blocks
  constexpr int MB = BR / 32;      // 32-row query blocks per sub-tile
  constexpr int NSUB = T / BR;     // query sub-tiles per task
  constexpr int QBW = MB * ND / NW;             // dQ 32x32 blocks per wave
  constexpr int NCOL = ND >= NW ? ND / NW : 1;  // ... in this many feature columns
  constexpr int NROW = QBW / NCOL;              // ... and this many query rows
  constexpr int TC = T / 16;       // k-chunks over the keys
  constexpr int GROUPS = (BR / 4) * (D / 8);  // staging pieces: 4 rows x 8 features
  constexpr int GPT = GROUPS / NT;
  static_assert(QBW * NW == MB * ND && GROUPS % NT == 0 && T % BR == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) bf16 sQ[BR * DP];
  __shared__ __attribute__((aligned(16))) bf16 sO[BR * DP];
  __shared__ __attribute__((aligned(16))) bf16 sQT[D * BRP];
  __shared__ __attribute__((aligned(16))) bf16 sOT[D * BRP];
  __shared__ __attribute__((aligned(16))) bf16 sKT[D * TP];
  __shared__ __attribute__((aligned(16))) bf16 sdST[T * SP];
  __shared__ __attribute__((aligned(16))) float sL[BR];
  __shared__ __attribute__((aligned(16))) float sDl[BR];
  __shared__ int sUnit[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int S = p.S;

  bf16x8 Kr[KC], Vr[KC];           // B operands of S and dP (this wave's keys)
  // B operand of dQ (all keys, this wave's columns): registers, except in the
  // XCD-local mode, which needs those registers for the in-flight running sums
  // and reads the operand from the K^T tile in LDS instead.
  constexpr bool KD_REG = !XCD;
  bf16x8 Kd[KD_REG ? NCOL : 1][KD_REG ? TC : 1];
  f32x16 dKa[ND], dVa[ND];
  u32x4 stq[GPT][4], sto[GPT][4];  // staged next sub-tile
  float stl = 0.0f, std_ = 0.0f;

  auto col_of = [&](int kc) { return ND >= NW ? w * NCOL + kc : w % ND; };
  auto row_of = [&](int kr) { return ND >= NW ? kr : w / ND + kr * (NW / ND); };

  // Rows past the end of the sequence are read as copies of the last row: the
  // masks give them P = 0 exactly, so a finite duplicate contributes nothing.
  auto stage_load = [&](int bh, int qrow0) {
    const bf16* qh = p.q + (size_t)bh * S * D;     // uniform head bases
    const bf16* oh = p.dout + (size_t)bh * S * D;
#pragma unroll
    for (int g = 0; g < GPT; ++g) {
      const int gi = tid + g * NT;
      const int qg = gi % (BR / 4), dg = gi / (BR / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = min(qrow0 + qg * 4 + rr, S - 1);
        const unsigned off = 2u * (unsigned)(row * D + dg * 8);
        stq[g][rr] = *at_bytes((const u32x4*)qh, off);
        sto[g][rr] = *at_bytes((const u32x4*)oh, off);
      }
    }
    if (tid < BR) {
      const float* lh = p.lse2 + (size_t)bh * p.S_pad;
      const float* dh = p.delta + (size_t)bh * p.S_pad;
      stl = *at_bytes(lh, 4u * (unsigned)(qrow0 + tid));
      std_ = *at_bytes(dh, 4u * (unsigned)(qrow0 + tid));
    }
  };

  auto stage_store = [&]() {
#pragma unroll
    for (int g = 0; g < GPT; ++g) {
      const int gi = tid + g * NT;
      const int qg = gi % (BR / 4), dg = gi / (BR / 4);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        *(u32x4*)&sQ[(qg * 4 + rr) * DP + dg * 8] = stq[g][rr];
        *(u32x4*)&sO[(qg * 4 + rr) * DP + dg * 8] = sto[g][rr];
      }
      const int pos = quad_pos(qg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 tq, to;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          tq[rr] = __builtin_bit_cast(bf16x8, stq[g][rr])[e];
          to[rr] = __builtin_bit_cast(bf16x8, sto[g][rr])[e];
        }
        *(bf16x4*)&sQT[(dg * 8 + e) * BRP + pos] = tq;
        *(bf16x4*)&sOT[(dg * 8 + e) * BRP + pos] = to;
      }
    }
    if (tid < BR) {
      sL[tid] = stl;
      sDl[tid] = std_;
    }
  };

  // K/V of KV tile kv into registers (and K^T through LDS for the dQ operand)
  auto load_kv = [&](int bh, int kv) {
    const int key = min(kv * T + 32 * w + l32, S - 1);  // keys past the end are masked
    const bf16* kh = p.k + (size_t)bh * S * D;
    const bf16* vh = p.v + (size_t)bh * S * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const unsigned off = 2u * (unsigned)(key * D + 16 * c + 8 * hh);
      Kr[c] = *at_bytes((const bf16x8*)kh, off);
      Vr[c] = *at_bytes((const bf16x8*)vh, off);
#pragma unroll
      for (int e = 0; e < 8; ++e) sKT[(16 * c + 8 * hh + e) * TP + 32 * w + l32] = Kr[c][e];
    }
    __syncthreads();
    if (KD_REG) {
#pragma unroll
      for (int kc = 0; kc < NCOL; ++kc) {
#pragma unroll
        for (int c = 0; c < TC; ++c)
          Kd[KD_REG ? kc : 0][KD_REG ? c : 0] = *(const bf16x8*)&sKT[(32 * col_of(kc) + l32) * TP + 16 * c + 8 * hh];
      }
    }
  };

  auto finalize_kv = [&](int bh, int kv) {
#pragma unroll
    for (int n = 0; n < ND; ++n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kv * T + 32 * w + 8 * (i / 4) + 4 * hh + (i % 4);
        if (key < S) {
          const size_t off = ((size_t)bh * S + key) * D + 32 * n + l32;
          p.dk[off] = to_bf16(dKa[n][i] * p.scale);
          p.dv[off] = to_bf16(dVa[n][i]);
        }
      }
    }
  };

  // Symmetric Shift parking: one slot per (workgroup, tile of the pair)
  auto park_acc = [&](int slot, bool load) {
    float* base = p.park + ((size_t)blockIdx.x * 2 + slot) * (size_t)(2 * ND * 16 * NT);
#pragma unroll
    for (int n = 0; n < ND; ++n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float* a = base + (size_t)((n * 16 + i) * NT + tid);
        float* b = base + (size_t)(((ND + n) * 16 + i) * NT + tid);
        if (load) {
          dKa[n][i] = *a;
          dVa[n][i] = *b;
        } else {
          *a = dKa[n][i];
          *b = dVa[n][i];
        }
      }
    }
    wait_vmem();
  };

  int xq = 0;  // this workgroup's XCD, the queue it takes units from
  if (XCD) {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    xq = (int)(x & (kMaxQueues - 1));
  }

  for (;;) {
    __syncthreads();
    if (tid == 0) {
      if (!XCD) {
        const int u = atomicAdd(&p.header[0], 1);
        sUnit[0] = u < p.n_units ? u / p.n_workers : p.BH;
        sUnit[1] = u % p.n_workers;
      } else {
        // Units of one head are consecutive tickets of one XCD's queue; the
        // ticket of a head's first worker claims the next unclaimed head and
        // publishes it for the others (lower tickets are held by running
        // workgroups, so the wait below always ends).
        const int k = atomicAdd(&p.header[16 + xq], 1);
        const int i = k / p.n_workers, wk = k % p.n_workers;
        int head = p.BH;
        if (i < p.BH) {
          int* slot = &p.heads[xq * p.BH + i];
          if (wk == 0) {
            head = min(atomicAdd(&p.header[2], 1), p.BH);
            __hip_atomic_store(slot, head, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            uint32_t it = 0;
            while ((head = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < 0) {
              if (++it >= p.wait_limit) {
                __hip_atomic_store(&p.header[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                head = p.BH;
                break;
              }
              __builtin_amdgcn_s_sleep(2);
            }
          }
        }
        sUnit[0] = head;
        sUnit[1] = wk;
      }
    }
    __syncthreads();
    const int bh = sUnit[0];
    const int wk = sUnit[1];
    if (bh >= p.BH) break;
    const int ntasks = sched_num_tasks(p.N, CAUSAL, p.sched, wk);
    const int total = ntasks * NSUB;

    // the (at most two) KV tiles of this unit and the last task of each
    int tileA = -1, tileB = -1, lastA = -1, lastB = -1;
    for (int t = 0; t < ntasks; ++t) {
      const int kv = sched_task(p.N, CAUSAL, p.sched, wk, t).kv;
      if (tileA < 0 || kv == tileA) {
        tileA = kv;
        lastA = t;
      } else {
        tileB = kv;
        lastB = t;
      }
    }
    int cur_kv = -1;
    bool parkedA = false, parkedB = false;
    int pend = -1;  // counter whose increment is still owed (its RMWs are in flight)

    {
      const Task t0 = sched_task(p.N, CAUSAL, p.sched, wk, 0);
      stage_load(bh, t0.q * T);
      stage_store();
      if (total > 1) {
        const Task t1 = sched_task(p.N, CAUSAL, p.sched, wk, 1 / NSUB);
        stage_load(bh, t1.q * T + (1 % NSUB) * BR);
      }
    }

    for (int idx = 0; idx < total; ++idx) {
      const int t = idx / NSUB;
      const int sidx = idx % NSUB;
      const Task task = sched_task(p.N, CAUSAL, p.sched, wk, t);
      const int qi = task.q, kj = task.kv;

      if (kj != cur_kv) {
        if (cur_kv >= 0) {
          const bool isA = (cur_kv == tileA);
          if (t <= (isA ? lastA : lastB)) {
            park_acc(isA ? 0 : 1, false);
            if (isA) parkedA = true; else parkedB = true;
          } else {
            finalize_kv(bh, cur_kv);
          }
        }
        __syncthreads();
        load_kv(bh, kj);
        const bool isA = (kj == tileA);
        if (isA ? parkedA : parkedB) {
          park_acc(isA ? 0 : 1, true);
          if (isA) parkedA = false; else parkedB = false;
        } else {
#pragma unroll
          for (int n = 0; n < ND; ++n) {
            dKa[n] = zero16();
            dVa[n] = zero16();
          }
        }
        cur_kv = kj;
      }

      const int q_base = qi * T + sidx * BR;
      const int kv_base = kj * T;
      __syncthreads();  // staged sub-tile visible

      // ---- S = Q K^T, dP = dO V^T, P, dS; dV += P^T dO, dK += dS^T Q
      const int key_g = kv_base + 32 * w + l32;
      const bool key_ok = key_g < S;
      const bool need_mask = (CAUSAL && qi == kj) || (kv_base + T > S);
#pragma unroll 1
      for (int m = 0; m < MB; ++m) {
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const bf16x8 qa = *(const bf16x8*)&sQ[(32 * m + l32) * DP + 16 * c + 8 * hh];
          const bf16x8 oa = *(const bf16x8*)&sO[(32 * m + l32) * DP + 16 * c + 8 * hh];
          s = mfma32(qa, Kr[c], s);
          dp = mfma32(oa, Vr[c], dp);
        }
        if (need_mask) {  // diagonal tile of a causal mask, or the ragged last KV tile
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 L4 = *(const f32x4*)&sL[32 * m + 8 * a + 4 * hh];
            const f32x4 D4 = *(const f32x4*)&sDl[32 * m + 8 * a + 4 * hh];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int i = 4 * a + b;
              const int q_g = q_base + 32 * m + 8 * a + 4 * hh + b;
              float pv = fast_exp2(s[i] * p.scale_log2 - L4[b]);
              const bool vis = key_ok && (!CAUSAL || key_g <= q_g);
              pv = vis ? pv : 0.0f;
              s[i] = pv;
              dp[i] = pv * (dp[i] - D4[b]);
            }
          }
        } else {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 L4 = *(const f32x4*)&sL[32 * m + 8 * a + 4 * hh];
            const f32x4 D4 = *(const f32x4*)&sDl[32 * m + 8 * a + 4 * hh];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int i = 4 * a + b;
              const float pv = fast_exp2(s[i] * p.scale_log2 - L4[b]);
              s[i] = pv;
              dp[i] = pv * (dp[i] - D4[b]);
            }
          }
        }
        const bf16x8 pb0 = pack8(s, 0), pb1 = pack8(s, 8);
        const bf16x8 db0 = pack8(dp, 0), db1 = pack8(dp, 8);
        // dS^T: four consecutive queries per 8-byte write
        bf16* drow = &sdST[(32 * w + l32) * SP + 32 * m + 4 * hh];
        *(bf16x4*)(drow + 0) = __builtin_shufflevector(db0, db0, 0, 1, 2, 3);
        *(bf16x4*)(drow + 8) = __builtin_shufflevector(db0, db0, 4, 5, 6, 7);
        *(bf16x4*)(drow + 16) = __builtin_shufflevector(db1, db1, 0, 1, 2, 3);
        *(bf16x4*)(drow + 24) = __builtin_shufflevector(db1, db1, 4, 5, 6, 7);
#pragma unroll
        for (int n = 0; n < ND; ++n) {
          const int ro = (32 * n + l32) * BRP + 32 * m + 8 * hh;
          dVa[n] = mfma32(pb0, *(const bf16x8*)&sOT[ro], dVa[n]);
          dVa[n] = mfma32(pb1, *(const bf16x8*)&sOT[ro + 16], dVa[n]);
          dKa[n] = mfma32(db0, *(const bf16x8*)&sQT[ro], dKa[n]);
          dKa[n] = mfma32(db1, *(const bf16x8*)&sQT[ro + 16], dKa[n]);
        }
      }
      wait_vmem();      // this wave's earlier dQ RMWs and staging loads have completed
      __syncthreads();  // dS^T complete; staged Q/dO no longer read; all earlier RMWs done

      if (!ATOMIC && pend >= 0 && tid == 0)
        __hip_atomic_fetch_add(&p.counters[pend], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pend = -1;
      if (idx + 1 < total) {
        stage_store();
        if (!XCD && idx + 2 < total) {  // prefetch now: it lands during the dQ phase and the next S/dP
          const Task n2 = sched_task(p.N, CAUSAL, p.sched, wk, (idx + 2) / NSUB);
          stage_load(bh, n2.q * T + ((idx + 2) % NSUB) * BR);
        }
      }

      // ---- dQ partial of this sub-tile and its ordered hand-off
      const int cidx = bh * p.n_qsub + qi * NSUB + sidx;
      const int r = ATOMIC ? 0 : sched_rank(p.N, CAUSAL, p.sched, qi, kj);
      const bool last = ATOMIC ? true : (r == sched_contributors(p.N, CAUSAL, qi) - 1);
      int seen = r;
      if (!ATOMIC && r > 0 && tid == 0)  // poll early
        seen = __hip_atomic_load(&p.counters[cidx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      float* wsrow = p.dq_ws + ((size_t)bh * p.S_pad + q_base) * D;  // uniform

      // Turn-taking: wait until the previous contributor's update is complete.
      auto wait_turn = [&]() {
        if (tid == 0) {
          uint32_t it = 0;
          while (seen != r) {
            if (++it >= p.wait_limit) {
              __hip_atomic_store(&p.header[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
            seen = __hip_atomic_load(&p.counters[cidx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        __syncthreads();
      };
      auto dq_block = [&](int kc, int mb) {
        f32x16 acc = zero16();
        const int grp = lane >> 4, gi = lane & 15;
        const bf16* base = &sdST[(8 * (grp >> 1) + (gi >> 2)) * SP + 32 * mb + 16 * (grp & 1) + 4 * (gi & 3)];
#pragma unroll
        for (int c = 0; c < TC; ++c) {
          const bf16x8 a = cat44(lds_read_tr(base + 16 * c * SP), lds_read_tr(base + (16 * c + 4) * SP));
          const bf16x8 kb = KD_REG ? Kd[KD_REG ? kc : 0][KD_REG ? c : 0]
                                   : *(const bf16x8*)&sKT[(32 * col_of(kc) + l32) * TP + 16 * c + 8 * hh];
          acc = mfma32(a, kb, acc);
        }
        return acc;
      };
      auto elem_off = [&](int nb, int mb, int i) {
        return 4u * (unsigned)((32 * mb + 4 * hh + 8 * (i / 4) + (i % 4)) * D + 32 * nb + l32);
      };

      if (XCD) {
        // Every contributor of this tile runs on this XCD, so its L2 holds the
        // accumulator coherently for all of them. After our turn, drop this
        // CU's write-through L1 copies, start the loads of the running sum,
        // compute the partial while they are in flight, then add and store.
        // (The first contributor adds to 0, which only turns -0 into +0.)
        static_assert(!XCD || NCOL * NROW == 2, "XCD-local hand-off is written for two dQ blocks per wave");
        const int nb0 = col_of(0), mb0 = row_of(0);
        const int nb1 = col_of(NCOL > 1 ? 1 : 0), mb1 = row_of(NCOL > 1 ? 0 : 1);
        const f32x16 acc0 = dq_block(0, mb0);  // overlaps the early poll
        float prev0[16], prev1[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) prev0[i] = prev1[i] = 0.0f;
        if (r > 0) {
          wait_turn();
          asm volatile("buffer_inv sc0" ::: "memory");
#pragma unroll
          for (int i = 0; i < 16; ++i) prev0[i] = *at_bytes(wsrow, elem_off(nb0, mb0, i));
#pragma unroll
          for (int i = 0; i < 16; ++i) prev1[i] = *at_bytes(wsrow, elem_off(nb1, mb1, i));
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the second block's MFMAs
        const f32x16 acc1 = dq_block(NCOL > 1 ? 1 : 0, mb1);
#pragma unroll
        for (int i = 0; i < 16; ++i) *at_bytes(wsrow, elem_off(nb0, mb0, i)) = prev0[i] + acc0[i];
#pragma unroll
        for (int i = 0; i < 16; ++i) *at_bytes(wsrow, elem_off(nb1, mb1, i)) = prev1[i] + acc1[i];
      } else {
        // Device-scope atomic RMWs (the deterministic mode serialises them with
        // the counters, so each element receives the same fp32 additions in
        // the same order on every run; the first contributor swaps its value in).
#pragma unroll
        for (int kc = 0; kc < NCOL; ++kc) {
#pragma unroll 1
          for (int kr = 0; kr < NROW; ++kr) {
            const int nb = col_of(kc), mb = row_of(kr);
            const f32x16 acc = dq_block(kc, mb);
            if (!ATOMIC && r > 0 && kc == 0 && kr == 0) wait_turn();
            if (!ATOMIC && r == 0) {
#pragma unroll
              for (int i = 0; i < 16; ++i)
                __hip_atomic_exchange(at_bytes(wsrow, elem_off(nb, mb, i)), acc[i], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            } else {
#pragma unroll
              for (int i = 0; i < 16; ++i)
                __hip_atomic_fetch_add(at_bytes(wsrow, elem_off(nb, mb, i)), acc[i], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
      if (!ATOMIC && !last) pend = cidx;
      // XCD-local mode prefetches here, keeping the dQ phase free of staging
      // registers; the loads still have the whole next S/dP phase to land
      if (XCD && idx + 2 < total) {
        const Task n2 = sched_task(p.N, CAUSAL, p.sched, wk, (idx + 2) / NSUB);
        stage_load(bh, n2.q * T + ((idx + 2) % NSUB) * BR);
      }
    }
    if (pend >= 0) {  // the unit's last hand-off
      wait_vmem();
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(&p.counters[pend], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (cur_kv >= 0) finalize_kv(bh, cur_kv);
  }
}

// --------------------------------------------------------------------------------------
// post-pass: dq = bf16(scale * dQ accumulator)

template <int D>
__global__ void __launch_bounds__(256) bwd_post_kernel(const float* dq_ws, bf16* dq, long long BH, int S,
                                                       int S_pad, float scale) {
  const long long n4 = BH * S * (D / 4);
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    const long long e = i * 4;
    const long long row = e / D;  // bh * S + s
    const int col = (int)(e % D);
    const long long bh = row / S;
    const int s = (int)(row % S);
    const f32x4 v = *(const f32x4*)(dq_ws + ((bh * S_pad + s) * D + col));
    bf16x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = to_bf16(v[j] * scale);
    *(bf16x4*)(dq + e) = o;
  }
}

// --------------------------------------------------------------------------------------
// launcher

template <int D, int T, int BR, bool CAUSAL, int MODE>
static hipError_t launch_main(const MainParams& mp, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_main_kernel<D, T, BR, CAUSAL, MODE>), dim3((unsigned)grid), dim3(T / 32 * 64), 0, stream,
                     mp);
  return hipGetLastError();
}

template <int D, int T, int BR, bool CAUSAL>
static hipError_t launch_mask(const MainParams& mp, bool atomic, int num_cu, int protocol, hipStream_t stream,
                              int* xcd_out) {
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, bwd_main_kernel<D, T, BR, CAUSAL, MODE_DEVICE>, T / 32 * 64, 0);
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
  // (the XCD-local hand-off is written for two dQ blocks per wave)
  constexpr bool kXcdShape = (BR / 32) * (D / 32) == 2 * (T / 32);
  const bool xcd = kXcdShape && !atomic && protocol != DQ_DEVICE_ATOMIC && (!cyclic || mp.n_workers <= per_xcd);
  *xcd_out = xcd ? 1 : 0;
  if (atomic) return launch_main<D, T, BR, CAUSAL, MODE_ATOMIC>(mp, (int)grid, stream);
  if constexpr (kXcdShape) {
    if (xcd) return launch_main<D, T, BR, CAUSAL, MODE_XCD>(mp, (int)grid, stream);
  }
  return launch_main<D, T, BR, CAUSAL, MODE_DEVICE>(mp, (int)grid, stream);
}

template <int D, int T, int BR>
static hipError_t dispatch_mask(const MainParams& mp, bool causal, bool atomic, int num_cu, int protocol,
                                hipStream_t s, int* xcd) {
  return causal ? launch_mask<D, T, BR, true>(mp, atomic, num_cu, protocol, s, xcd)
                : launch_mask<D, T, BR, false>(mp, atomic, num_cu, protocol, s, xcd);
}

hipError_t launch_bwd(const BwdArgs& a, int num_cu, hipStream_t stream) {
  const long long BH = (long long)a.B * a.H;
  int* header = (int*)(a.ws + a.lay.header);
  int* counters = (int*)(a.ws + a.lay.counters);
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
  pp.counters = counters;
  pp.header = header;
  pp.heads = heads;
  pp.n_heads = (long long)kMaxQueues * BH;
  pp.rows = BH * a.S_pad;
  pp.S = a.S;
  pp.S_pad = a.S_pad;
  pp.n_counters = BH * a.n_qsub;
  pp.dq_ws_elems = a.atomic ? BH * a.S_pad * a.D : 0;
  pp.poison = a.atomic ? 0 : a.poison;
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
  mp.counters = counters;
  mp.header = header;
  mp.heads = heads;
  mp.dq = (bf16*)a.dq;
  mp.BH = (int)BH;
  mp.S = a.S;
  mp.S_pad = a.S_pad;
  mp.N = a.N;
  mp.n_qsub = a.n_qsub;
  mp.sched = a.atomic ? SCHED_NAIVE : a.sched;
  mp.n_workers = sched_workers(a.N, mp.sched);
  mp.n_units = (int)(BH * mp.n_workers);
  mp.scale = a.scale;
  mp.scale_log2 = a.scale * 1.4426950408889634f;
  mp.wait_limit = a.wait_limit;

  int xcd_local = 0;
  hipError_t e = hipErrorInvalidValue;
  const bool causal = a.causal != 0, atomic = a.atomic != 0;
  if (a.ev_before && a.ev_after) {
    e = hipEventRecord(a.ev_before, stream);
    if (e != hipSuccess) return e;
  }
  if (a.D == 128 && a.T == 128) e = dispatch_mask<128, 128, 64>(mp, causal, atomic, num_cu, a.dq_protocol, stream, &xcd_local);
  else if (a.D == 128 && a.T == 64) e = dispatch_mask<128, 64, 64>(mp, causal, atomic, num_cu, a.dq_protocol, stream, &xcd_local);
  else if (a.D == 64 && a.T == 128) e = dispatch_mask<64, 128, 128>(mp, causal, atomic, num_cu, a.dq_protocol, stream, &xcd_local);
  else if (a.D == 64 && a.T == 64) e = dispatch_mask<64, 64, 64>(mp, causal, atomic, num_cu, a.dq_protocol, stream, &xcd_local);
  if (e != hipSuccess) return e;
  if (a.ev_before && a.ev_after) {
    e = hipEventRecord(a.ev_after, stream);
    if (e != hipSuccess) return e;
  }

  {
    const long long want = (BH * a.S * (a.D / 4) + 255) / 256;
    const unsigned g = (unsigned)(want < 8192 ? (want < 1 ? 1 : want) : 8192);
    if (a.D == 64)
      hipLaunchKernelGGL(bwd_post_kernel<64>, dim3(g), dim3(256), 0, stream, dq_ws, (bf16*)a.dq, BH, a.S,
                         a.S_pad, a.scale);
    else
      hipLaunchKernelGGL(bwd_post_kernel<128>, dim3(g), dim3(256), 0, stream, dq_ws, (bf16*)a.dq, BH, a.S,
                         a.S_pad, a.scale);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace attn
