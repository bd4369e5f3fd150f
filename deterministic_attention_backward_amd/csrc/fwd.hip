// Attention forward for gfx950: produces the O and LSE the backward consumes.
// Online softmax over 64-key tiles in ascending key order, so the result is
// the same bit pattern on every run.
//
// Workgroup = 4 waves = 128 query rows; wave w owns queries 32w..32w+31 of
// its tile and keeps them in registers. Scores are computed transposed,
// S^T = K Q^T, so that each lane holds one query column: the row statistics
// (running max, running sum) are per lane plus one exchange with the lane 32
// apart, and O^T = V^T P^T takes P^T straight from the score accumulators as
// its B operand. K and V tiles arrive by LDS DMA into double buffers of
// swizzled rows (the layout the backward stages Q and dO in): K is read
// row-wise (A operand of S^T), V through the transposing read (A operand of
// O^T, rows in the C-row order of P^T). The DMA of tile t+1 is issued before
// tile t is computed; one barrier per tile. Causal masks: a query tile stops
// at its diagonal, and the grid takes the longest query tiles first.
#include "common.hpp"
#include "launch.hpp"
#include "lds.hpp"

namespace attn {

struct FwdParams {
  const bf16 *q, *k, *v;
  bf16* o;
  float* lse;
  int S;
  int H, group;  // query heads per batch; query heads per K/V head
  int n_qt;      // query tiles per head
  float scale_log2;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) fwd_kernel(FwdParams p) {
  constexpr int KT = 64;           // keys per tile
  constexpr int RB = 2 * D;        // staged row bytes
  constexpr int KC = D / 16;
  constexpr int ND = D / 32;
  constexpr int TB = KT * RB;      // bytes of one staged tile (K or V)
  constexpr int PIECES = 2 * TB / 1024, PPW = PIECES / 4;  // 1 KB DMA pieces (K then V), per wave
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TB];  // [buffer][K, V][KT rows]

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = p.S;
  const long long bh = blockIdx.y;
  // causal: the longest query tiles (the last ones) first
  const int qt = CAUSAL ? p.n_qt - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int q0 = qt * 128;
  const int qrow = q0 + 32 * w + l32;   // this lane's query
  const bf16* qh = p.q + bh * S * D;
  const long long kvh = (bh / p.H) * (p.H / p.group) + (bh % p.H) / p.group;  // this query head's K/V head
  const bf16* kh = p.k + kvh * S * D;
  const bf16* vh = p.v + kvh * S * D;

  // DMA of keys k0..k0+63 (K and V) into buffer buf; keys past the end are
  // read as copies of the last key (the mask gives them P = 0 exactly)
  auto stage = [&](int k0, int buf) {
    constexpr int CPR = D / 8, RPP = 64 / CPR, HALF = PIECES / 2;
    int rl = lane / CPR, lx = (lane % CPR) ^ swz<D>(lane / CPR);
    asm volatile("" : "+v"(rl), "+v"(lx));
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int piece = w * PPW + k;  // wave-uniform
      const bool is_v = piece >= HALF;
      const int pr = is_v ? piece - HALF : piece;
      const unsigned off = (unsigned)(min(k0 + pr * RPP + rl, S - 1) * RB + 16 * (lx ^ swz<D>(pr * RPP)));
      char* dst = smem + (2 * buf + (is_v ? 1 : 0)) * TB + pr * 1024;
      __builtin_amdgcn_global_load_lds(at_bytes(is_v ? vh : kh, off), (__attribute__((address_space(3))) void*)dst, 16,
                                       0, 0);
    }
  };

  int kend = S;
  if (CAUSAL) kend = (q0 + 128 < S) ? q0 + 128 : S;
  const int ntiles = (kend + KT - 1) / KT;
  stage(0, 0);

  bf16x8 Qr[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (qrow < S) {
      Qr[c] = *(const bf16x8*)(qh + (size_t)qrow * D + 16 * c + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) Qr[c][e] = (bf16)0.0f;
    }
  }
  f32x16 oacc[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) oacc[n] = zero16();
  float m = -__builtin_inff(), l = 0.0f;
  const int sw = swz<D>(l32);
  const int a_base = l32 * RB + 16 * ((hh ^ sw) & 1), sw1 = sw >> 1;
  TrLane tl;
  tl.init<D>(lane);

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * KT, buf = t & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t has landed (this wave's share)
    __syncthreads();                                   // ... everyone's; tile t-1's buffer is free
    if (t + 1 < ntiles) stage(k0 + KT, buf ^ 1);
    const char* Kb = smem + (2 * buf) * TB;
    const char* Vb = Kb + TB;

    f32x16 st[2];
    float tmax = -__builtin_inff();
    int ab = a_base, s1 = sw1;
    asm volatile("" : "+v"(ab), "+v"(s1));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const char* Kr = Kb + 32 * kb * RB + ab;
      f32x16 acc = zero16();
#pragma unroll
      for (int c = 0; c < KC; ++c) acc = mfma32(*(const bf16x8*)(Kr + ((c ^ s1) << 5)), Qr[c], acc);
      const bool edge = k0 + KT > S || (CAUSAL && k0 + KT > q0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4);
        const bool vis = !edge || (key < S && (!CAUSAL || key <= qrow));
        const float x = vis ? acc[i] * p.scale_log2 : -__builtin_inff();
        acc[i] = x;
        tmax = fmaxf(tmax, x);
      }
      st[kb] = acc;
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - mnew);
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(st[kb][i] - mnew);
        st[kb][i] = pv;
        psum += pv;
      }
    }
    psum += __shfl_xor(psum, 32);
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int n = 0; n < ND; ++n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[n][i] *= alpha;
    }
    int tb[2] = {tl.base[0], tl.base[1]}, th = tl.hi;
    asm volatile("" : "+v"(tb[0]), "+v"(tb[1]), "+v"(th));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 pb0 = pack8(st[kb], 0), pb1 = pack8(st[kb], 8);
      const char* Vk = Vb + 32 * kb * RB;
#pragma unroll
      for (int n = 0; n < ND; ++n) {
        const int nx = (n ^ th) << 6;
        oacc[n] = mfma32(trB<RB>(Vk, 0, tb, nx), pb0, oacc[n]);
        oacc[n] = mfma32(trB<RB>(Vk, 1, tb, nx), pb1, oacc[n]);
      }
    }
  }

  if (qrow < S) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int n = 0; n < ND; ++n) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 ov;
#pragma unroll
        for (int b = 0; b < 4; ++b) ov[b] = to_bf16(oacc[n][4 * a + b] * inv);
        *(bf16x4*)(p.o + (bh * S + qrow) * (long long)D + 32 * n + 8 * a + 4 * hh) = ov;
      }
    }
    if (hh == 0) p.lse[bh * S + qrow] = (m + __log2f(l)) * 0.6931471805599453f;
  }
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  FwdParams fp;
  fp.q = (const bf16*)a.q;
  fp.k = (const bf16*)a.k;
  fp.v = (const bf16*)a.v;
  fp.o = (bf16*)a.o;
  fp.lse = a.lse;
  fp.S = a.S;
  fp.H = a.H;
  fp.group = a.H / a.Hkv;
  fp.n_qt = (a.S + 127) / 128;
  fp.scale_log2 = a.scale * 1.4426950408889634f;
  const dim3 grid((unsigned)((a.S + 127) / 128), (unsigned)((long long)a.B * a.H));
  if (a.D == 64) {
    if (a.causal) hipLaunchKernelGGL((fwd_kernel<64, true>), grid, dim3(256), 0, stream, fp);
    else hipLaunchKernelGGL((fwd_kernel<64, false>), grid, dim3(256), 0, stream, fp);
  } else {
    if (a.causal) hipLaunchKernelGGL((fwd_kernel<128, true>), grid, dim3(256), 0, stream, fp);
    else hipLaunchKernelGGL((fwd_kernel<128, false>), grid, dim3(256), 0, stream, fp);
  }
  return hipGetLastError();
}

}  // namespace attn
