// dQ scheduling formulas for the deterministic attention backward.
//
// One attention head is cut into N query tiles and N key/value (KV) tiles of
// the same edge T. A "worker" is the workgroup that owns one KV tile (two for
// Symmetric Shift) for the whole head and keeps its dK/dV accumulators
// on-chip; it walks a list of tasks (query tile i, KV tile j). Each dQ tile i
// receives the partial products of all its tasks in one fixed order; r(i, j)
// is the position of KV tile j in that order.
//
// Strategies (DASH: Deterministic Attention Scheduling for High-throughput
// Reproducible LLM Training; Dutch and Japanese technical summaries, §2.2):
//   NAIVE           worker j walks the query tiles upward; dQ order = KV ascending.
//   DESCENDING      §2.2 A: worker j walks the query tiles downward, last tile
//                   first; dQ order unchanged (KV ascending).
//   SHIFT           §2.2 B, full mask: worker j starts at query tile j and
//                   continues cyclically, so at every step each worker is on a
//                   different dQ tile; dQ order = the order of those steps,
//                   r(i, j) = (i - j) mod N. Causal mask (the DASH abstract
//                   credits Shift Scheduling for both masks): the same cyclic
//                   walk with the fully masked query tiles 0..j-1 left out, so
//                   worker j walks j, j+1, ..., N-1 and dQ tile i receives
//                   KV tiles i, i-1, ..., 0 in that order: r(i, j) = i - j.
//   SYMMETRIC_SHIFT §2.2 B, causal mask: worker p owns KV tiles p and N-1-p
//                   (N even). Steps 0..N/2-1 cover the dense lower-left
//                   rectangle (query tiles N/2..N-1 x KV tile p) with a cyclic
//                   shift; steps N/2..N cover the two leftover triangles, the
//                   lower-right one folded onto the upper-left one, also with a
//                   cyclic shift, the folded square's diagonal taking two steps.
//                   dQ order = step order. Every worker has N+1 tasks.
//
// The rank formula for SYMMETRIC_SHIFT follows from that geometry (h = N/2):
//   i <  h: contributions arrive on the diagonal first, then from KV tiles
//           i-1, i-2, ..., 0            ->  r = i - j
//   i >= h: the rectangle's h contributions come first, in step order
//           r = (i - h - j) mod h (j < h); then the folded diagonal (j = i),
//           r = h; then folded KV tiles h..i-1 in ascending order, r = j + 1.
//
// These are plain integer formulas evaluated per task in scalar registers on
// the device and by attn_schedule_plan() on the host; no table is stored.
#pragma once

// (Every index below stays within [0, 2m) of the modulus m it is reduced by,
// so a conditional subtraction replaces the remainder: no integer division in
// the per-sub-tile scalar code.)

#ifdef __HIPCC__
#define ATTN_HD __host__ __device__ __forceinline__
#else
#define ATTN_HD inline
#endif

namespace attn {

// x mod m for x in [-m, 2m)
ATTN_HD int wrap(int x, int m) { return x >= m ? x - m : (x < 0 ? x + m : x); }

enum { SCHED_NAIVE = 0, SCHED_DESCENDING = 1, SCHED_SHIFT = 2, SCHED_SYMMETRIC_SHIFT = 3 };

struct Task {
  int q;   // query tile
  int kv;  // KV tile
};

// Workers (units) per head.
ATTN_HD int sched_workers(int N, int sched) { return sched == SCHED_SYMMETRIC_SHIFT ? N / 2 : N; }

// Number of tasks worker w walks.
ATTN_HD int sched_num_tasks(int N, bool causal, int sched, int w) {
  switch (sched) {
    case SCHED_NAIVE:
    case SCHED_DESCENDING:
    case SCHED_SHIFT: return causal ? N - w : N;
    default: return N + 1;
  }
}

// The t-th task of worker w.
ATTN_HD Task sched_task(int N, bool causal, int sched, int w, int t) {
  Task k;
  switch (sched) {
    case SCHED_NAIVE:
      k.kv = w;
      k.q = causal ? w + t : t;
      break;
    case SCHED_DESCENDING:
      k.kv = w;
      k.q = N - 1 - t;
      break;
    case SCHED_SHIFT:
      k.kv = w;
      k.q = causal ? w + t : wrap(w + t, N);
      break;
    default: {
      const int h = N / 2;
      if (t < h) {                 // phase 1: dense rectangle
        k.q = h + wrap(w + t, h);
        k.kv = w;
      } else if (t == h) {         // folded square, diagonal, upper-left task
        k.q = w;
        k.kv = w;
      } else if (t == h + 1) {     // folded square, diagonal, lower-right task
        k.q = N - 1 - w;
        k.kv = N - 1 - w;
      } else {                     // folded square, off-diagonal
        const int rho = wrap(w + (t - h - 1), h);
        if (rho > w) {
          k.q = rho;
          k.kv = w;
        } else {
          k.q = N - 1 - rho;
          k.kv = N - 1 - w;
        }
      }
    }
  }
  return k;
}

// Number of KV tiles that contribute to dQ tile i.
ATTN_HD int sched_contributors(int N, bool causal, int i) { return causal ? i + 1 : N; }

// Position r(i, j) of KV tile j in dQ tile i's accumulation order.
ATTN_HD int sched_rank(int N, bool causal, int sched, int i, int j) {
  switch (sched) {
    case SCHED_NAIVE:
    case SCHED_DESCENDING: return j;
    case SCHED_SHIFT: return causal ? i - j : wrap(i - j, N);
    default: {
      const int h = N / 2;
      if (i < h) return i - j;
      if (j < h) return wrap(i - h - j, h);
      if (j == i) return h;
      return j + 1;
    }
  }
}

}  // namespace attn
