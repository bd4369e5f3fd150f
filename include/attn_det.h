/*
 * attn_det.h - deterministic attention backward for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn_det.so. The operation is the backward pass of softmax
 * attention, dQ/dK/dV from Q, K, V, the forward output O, the upstream
 * gradient dO and the forward log-sum-exp, computed so that every result is
 * bit-identical from run to run. The DASH pages (arXiv 2601.21824; Dutch and
 * Japanese technical summaries §1, English abstract) locate the
 * nondeterminism of fused attention backward in the floating-point
 * accumulation of dQ across KV tiles and fix it by accumulating each dQ tile
 * in a predetermined order; §2.2 of the technical summaries gives the
 * schedules implemented here.
 *
 * Conventions shared by every entry point
 *   - Tensors q, k, v, o, dout, dq, dk, dv are bfloat16, contiguous, laid out
 *     [B][H][S][D] (batch, head, position, feature). lse is float32 [B][H][S].
 *   - Query and key length are both S (self-attention). S >= 1, any value: a
 *     ragged last tile is masked inside the kernels. D is 64 or 128.
 *   - mask: ATTN_MASK_FULL, or ATTN_MASK_CAUSAL (key s' visible to query s
 *     iff s' <= s).
 *   - scale multiplies q.k before the softmax (usually 1/sqrt(D)).
 *   - lse is the natural-log log-sum-exp of the scaled (and masked) scores
 *     of each query row, as written by attn_fwd.
 *   - All pointers are device pointers owned by the caller; the library never
 *     allocates or frees device memory. Every pointer must be 16-byte aligned.
 *   - stream is a hipStream_t (passed as void*; NULL = the default stream).
 *     Work is enqueued asynchronously; results are valid after the stream is
 *     synchronised.
 *   - Every entry point returns an attn_status_t. Argument errors are detected
 *     on the host before any HIP call and leave device memory untouched.
 *   - The library keeps no state between calls apart from a per-device cache
 *     of the compute-unit count and the debug settings below; calls on
 *     different streams that use different workspaces may run concurrently.
 */
#ifndef ATTN_DET_H
#define ATTN_DET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, bad enum value */
  ATTN_ERR_UNSUPPORTED = -2,   /* valid request this build does not implement    */
  ATTN_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required      */
  ATTN_ERR_ALIGNMENT = -4,     /* a pointer is not 16-byte aligned                */
  ATTN_ERR_HIP = -5,           /* a HIP runtime call or kernel launch failed      */
  ATTN_ERR_TIMEOUT = -6,       /* a dQ ordering wait exceeded its bound            */
  ATTN_ERR_SCRATCH_LIMIT = -7  /* problem too large for attn_bwd_deterministic_noalloc */
} attn_status_t;

typedef enum { ATTN_MASK_FULL = 0, ATTN_MASK_CAUSAL = 1 } attn_mask_t;

/* dQ schedules: the order in which each worker walks the query tiles and the
 * order in which each dQ tile is accumulated (see attn_schedule_plan). */
typedef enum {
  ATTN_SCHED_NAIVE = 0,          /* ascending query tiles; dQ in KV-ascending order       */
  ATTN_SCHED_DESCENDING = 1,     /* Descending Q-Tile Iteration (DASH §2.2 A)             */
  ATTN_SCHED_SHIFT = 2,          /* Shift Scheduling (DASH §2.2 B; abstract: both masks)  */
  ATTN_SCHED_SYMMETRIC_SHIFT = 3 /* Symmetric Shift, causal mask, even tile count (§2.2 B)*/
} attn_schedule_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_status_string(int status);

/*
 * attn_fwd - attention forward, used to produce the backward's O and LSE.
 *   o   = softmax(scale * q k^T [masked]) v        bf16 [B][H][S][D]
 *   lse = log(sum_j exp(scale * q_i . k_j))        fp32 [B][H][S]
 * Deterministic (fixed accumulation order). Not a tuned kernel.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int S, int D, float scale, int mask, void* stream);

/*
 * attn_bwd_tile - the KV/query tile edge T the backward will use.
 *   tile_request = 0 lets the library choose (64 when S <= 256, else 128);
 *   64 or 128 forces that edge. Returns T (> 0) or a negative status.
 *   The head is cut into N = ceil(S / T) query tiles and N KV tiles.
 */
int attn_bwd_tile(int S, int D, int tile_request);

/*
 * attn_bwd_workspace_size - bytes of device workspace a backward call needs.
 * The workspace holds the fp32 dQ accumulator (B*H*ceil(S/T)*T*D floats), the
 * per-row softmax terms, the dQ hand-off flags and, for Symmetric Shift,
 * the parking area for a worker's second set of dK/dV accumulators.
 * Returns 0 for invalid arguments (then the call itself reports why).
 */
size_t attn_bwd_workspace_size(int B, int H, int S, int D, int mask, int schedule, int tile_request);

/*
 * attn_bwd_deterministic - bit-reproducible attention backward.
 *   In:  q, k, v, o, dout (bf16 [B][H][S][D]), lse (fp32 [B][H][S]).
 *   Out: dq, dk, dv (bf16 [B][H][S][D]); overwritten, no accumulation.
 *   Each workgroup owns one KV tile (two for Symmetric Shift) and keeps its
 *   dK/dV in registers; dQ tile i is accumulated in fp32 in the order the
 *   schedule fixes, each contributor waiting for its turn on per-sub-tile
 *   hand-off flags: the order of the fp32 additions into every dQ element is
 *   the schedule's, never the hardware's.
 *   schedule: attn_schedule_t. NAIVE, DESCENDING and SHIFT take either
 *   mask (SHIFT on a causal mask: worker j walks query tiles j..N-1, dQ tile i
 *   accumulates KV tiles i, i-1, ..., 0); SYMMETRIC_SHIFT needs
 *   ATTN_MASK_CAUSAL and an even tile count, else ATTN_ERR_UNSUPPORTED.
 *   workspace: device memory of at least attn_bwd_workspace_size(...) bytes,
 *   owned by the caller; contents need not be initialised and are scratch
 *   after the call. Concurrent calls must use distinct workspaces.
 *   The output for a given input and (schedule, tile) is the same bit pattern
 *   on every run. Different schedules may differ in the last bits.
 */
int attn_bwd_deterministic(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, int mask, int schedule,
                           void* dq, void* dk, void* dv, int B, int H, int S, int D,
                           float scale, int tile_request, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * attn_bwd_nondeterministic - the same backward with dQ accumulated by
 * hardware fp32 atomic adds in whatever order the hardware performs them (the
 * non-deterministic counterpart the DASH abstract compares against). Ascending
 * query-tile walk; no ordering waits. Workspace as for the deterministic call
 * with schedule ATTN_SCHED_NAIVE.
 */
int attn_bwd_nondeterministic(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, int mask,
                              void* dq, void* dk, void* dv, int B, int H, int S, int D,
                              float scale, int tile_request, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * attn_bwd_deterministic_noalloc - attn_bwd_deterministic for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. The call takes no workspace and
 * makes no allocation: its workspace is a static device array of this
 * library, ATTN_NOALLOC_SCRATCH_MIB MiB per device, held from the library's
 * first use on a device until the process ends. Arguments, layout, results
 * and bits are those of attn_bwd_deterministic (same kernels, same order).
 * Problems whose workspace (attn_bwd_workspace_size) exceeds the array return
 * ATTN_ERR_SCRATCH_LIMIT before any HIP call; 128 MiB covers, e.g., B=4,
 * H=16, S=2048, D=128 (68 MB). Every call on one device shares that device's
 * array: calls that overlap in time on one device (other streams or host
 * threads) race and must not be issued; consecutive calls on one stream are
 * fine. attn_bwd_check does not apply (there is no caller workspace); an
 * expired wait still shows as NaN outputs.
 */
#define ATTN_NOALLOC_SCRATCH_MIB 128
int attn_bwd_deterministic_noalloc(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, int mask, int schedule,
                                   void* dq, void* dk, void* dv, int B, int H, int S, int D,
                                   float scale, int tile_request, void* stream);

/*
 * attn_bwd_check - wait for `stream`, then report whether a deterministic call
 * that used `workspace` tripped the bound on a dQ ordering wait
 * (ATTN_ERR_TIMEOUT), else ATTN_OK. Host-blocking. A call that tripped the
 * bound also writes NaN into every element of its dq, dk and dv (the passes
 * after the main kernel read the workspace's flag), so the failure shows in
 * the gradients without this check or any other host synchronisation.
 */
int attn_bwd_check(const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped-query attention (query heads sharing K/V heads). Not on the pages:
 * the end-to-end models they time share K/V heads across query heads in some
 * configurations, which needs a second fixed-order reduction (dK, dV over the
 * query heads of a group). H query heads, Hkv K/V heads, H % Hkv == 0, and
 * query head h uses K/V head h / (H / Hkv) (consecutive query heads share
 * one). q, o, dout, dq: bf16 [B][H][S][D]; lse: fp32 [B][H][S]; k, v, dk,
 * dv: bf16 [B][Hkv][S][D]. Hkv == H is the plain call. The backward computes
 * each query head's dK (scaled) and dV in fp32 as the plain call does, then
 * sums them over the group in the fixed order of the query heads and rounds
 * once to bf16, so it is bit-reproducible like the plain call. Everything
 * else (masks, schedules, tiles, workspace ownership, status codes) is as for
 * the plain calls; the workspace is sized by attn_bwd_gqa_workspace_size and
 * holds two more fp32 [B][H][S_pad][D] tensors when Hkv < H. H % Hkv != 0 is
 * ATTN_ERR_INVALID_ARG.
 */
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Hkv, int S, int D, float scale, int mask, void* stream);
size_t attn_bwd_gqa_workspace_size(int B, int H, int Hkv, int S, int D, int mask, int schedule,
                                   int tile_request);
int attn_bwd_deterministic_gqa(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, int mask, int schedule,
                               void* dq, void* dk, void* dv, int B, int H, int Hkv, int S, int D,
                               float scale, int tile_request, void* workspace,
                               size_t workspace_bytes, void* stream);
int attn_bwd_nondeterministic_gqa(const void* q, const void* k, const void* v, const void* o,
                                  const void* dout, const float* lse, int mask,
                                  void* dq, void* dk, void* dv, int B, int H, int Hkv, int S, int D,
                                  float scale, int tile_request, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * attn_schedule_plan - host-only export of one head's schedule (no HIP call).
 *   n_tiles = N; mask, schedule as above.
 *   Writes int32 values to out: [n_workers, n_tasks, then for every task, in
 *   (worker, step) order, the five values worker, step, q_tile, kv_tile, rank].
 *   *needed (if not NULL) receives the number of int32 values required.
 *   out may be NULL to query the size; otherwise out_len must be >= *needed
 *   or ATTN_ERR_INVALID_ARG is returned.
 */
int attn_schedule_plan(int n_tiles, int mask, int schedule, int32_t* out, size_t out_len,
                       size_t* needed);

/*
 * attn_debug_set_wait_limit - bound (in polling iterations, each one a
 * hand-off flag read plus a short sleep) on a single dQ ordering wait; 0
 * restores the default (2^21, a few seconds at most). When a wait reaches the bound the
 * workgroup records ATTN_ERR_TIMEOUT in the workspace, stops waiting and
 * finishes normally; the call's outputs are then NaN and attn_bwd_check
 * reports the status. poison_counter != 0 makes the
 * next deterministic calls wait on one dQ hand-off flag for a value it never
 * takes, so that the bound is certain to trip (used to test the timeout
 * path; that call's dq, dk and dv come out as NaN). Process-wide, not
 * thread-safe; for tests only.
 */
void attn_debug_set_wait_limit(uint32_t iterations, int poison_counter);

/*
 * attn_debug_wait_timeouts - synchronises the current device, then returns how
 * many bounded waits (dQ turns and head claims) ran out since the count was
 * last cleared, over every backward launch of this process on that device
 * (>= 0), or a negative status. Unlike attn_bwd_check this is not tied to one
 * workspace or to the last call. reset != 0 clears the count after reading.
 * Host-blocking; for tests and benchmarks.
 */
int attn_debug_wait_timeouts(int reset);

/*
 * attn_debug_set_dq_protocol - how deterministic calls hand dQ partials over
 * (the order is the schedule's in every case):
 *   0 (default) choose per call: XCD-local when every worker of a head can be
 *     resident on one XCD (always for NAIVE/DESCENDING; for SHIFT and
 *     SYMMETRIC_SHIFT when the workers per head fit the XCD), else 1;
 *   1 device-wide: workers of a head may run on any XCD; the accumulator's
 *     running sums and the hand-off flags are read and written with
 *     system-scope accesses (written through to, and read from, the
 *     device-wide coherence point instead of an XCD's L2);
 *   2 XCD-local: all workers of a head run on one XCD and update the fp32
 *     accumulator with plain loads/stores through that XCD's L2 (falls back
 *     to 1 where the workers of a head would not be co-resident).
 * Returns ATTN_ERR_INVALID_ARG for other values. Process-wide, not
 * thread-safe; for tests and measurements.
 */
int attn_debug_set_dq_protocol(int protocol);

/*
 * attn_set_timing_events - profiling hook. When both arguments are non-NULL
 * hipEvent_t handles (created by the caller), every following backward call
 * records `before` on its stream immediately before launching its main tile
 * kernel and `after` immediately after it, so hipEventElapsedTime(before,
 * after) is that kernel's duration. NULL, NULL turns the hook off.
 * Process-wide, not thread-safe; for benchmarks only.
 */
void attn_set_timing_events(void* before, void* after);

/*
 * attn_probe_mfma - measurement probe (not part of the backward): runs one
 * workgroup per CU that issues `iterations` x 4 independent bf16
 * v_mfma_f32_32x32x16 per wave (one wave per SIMD), after one warm-up launch,
 * on `stream` (a hipStream_t), and waits for it. *tflops receives the dense
 * bf16 MFMA throughput reached; *ghz the rate of the shader clock counter
 * (s_memtime) over the timed launch, i.e. the clock the matrix cores ran at.
 * Uses a small static device array; no allocation. Not thread-safe.
 */
int attn_probe_mfma(int iterations, void* stream, double* tflops, double* ghz);

/*
 * attn_probe_atomic - measurement probe (not part of the backward): the fp32
 * atomic-add throughput that bounds the non-deterministic variant, in that
 * variant's access pattern (each instruction adds into 64 consecutive
 * floats; 4 KB blocks; every wave on its own block). `buffer` is caller-owned
 * device memory of `bytes` bytes (256-byte aligned, at least 4096), whose
 * contents the probe overwrites with sums; eight 4-wave workgroups per CU
 * each run `iterations` rounds of 16 adds per lane, after one warm-up
 * launch, on `stream`, and the call waits for them. *gops receives atomic
 * adds per second / 1e9. Returns ATTN_ERR_INVALID_ARG or ATTN_ERR_ALIGNMENT
 * for bad arguments (checked before any HIP call), ATTN_ERR_HIP on a
 * runtime error. Allocates nothing.
 */
int attn_probe_atomic(void* buffer, size_t bytes, int iterations, void* stream, double* gops);

/*
 * attn_debug_wait_profile - only in the profiling build of the library
 * (libattn_det_profile.so, compiled with ATTN_PROFILE_WAIT=1); the regular
 * build returns ATTN_ERR_UNSUPPORTED. Synchronises the device, then writes,
 * for each workgroup of the last backward launch (at most max_workgroups),
 * ATTN_WAIT_PROFILE_VALUES (nine) uint64 values, cycles of the s_memtime
 * counter of one wave of each kind unless noted: [0] tile-wave cycles at the
 * two per-sub-tile hand-over barriers, [1] tile-wave total cycles, [2] dQ-wave
 * cycles waiting for their dQ turn, [3] dQ-wave cycles at the barriers,
 * [4] dQ-wave total cycles, [5] sub-tiles processed (a count), [6] tile-wave
 * cycles switching KV tiles (segment set-up and tear-down), [7] segments run
 * (a count), [8] tile-wave cycles claiming units. Returns the number of
 * workgroups written (>= 0) or a negative status.
 */
#define ATTN_WAIT_PROFILE_VALUES 9
int attn_debug_wait_profile(uint64_t* out, int max_workgroups);

/*
 * attn_debug_order_violations - only in the profiling build (as above); the
 * regular build returns ATTN_ERR_UNSUPPORTED. In that build every dQ hand-off
 * of the deterministic modes checks the ordered-reduction invariant of the
 * DASH paper's dQ accumulation (section 3, the fixed per-tile order): a
 * contributor of rank r that waits for its turn must never see the tile's
 * counter beyond r, and when it hands over, the counter must still read r
 * (no other contributor advanced it). Synchronises the device and returns how
 * many checks failed since the count was last cleared, over every backward
 * launch of this process (>= 0), or a negative status. reset != 0 clears the
 * count after reading. Host-blocking; for tests.
 */
int attn_debug_order_violations(int reset);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DET_H */
