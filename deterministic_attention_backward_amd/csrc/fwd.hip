// Attention forward for gfx950 (support kernel: produces the O and LSE the
// backward consumes). Online softmax over 64-key tiles in ascending key
// order, so the result is the same bit pattern on every run.
//
// Workgroup = 4 waves = 128 query rows; wave w owns queries 32w..32w+31 of
// its tile. Scores are computed transposed, S^T = K Q^T, so that each lane
// holds one query column: the row statistics (running max, running sum) are
// then per lane plus one exchange with the lane 32 apart, and O^T = V^T P^T
// takes P^T straight from the score accumulators as its B operand.
#include "common.hpp"
#include "launch.hpp"

namespace attn {

struct FwdParams {
  const bf16 *q, *k, *v;
  bf16* o;
  float* lse;
  int S;
  int H, group;  // query heads per batch; query heads per K/V head
  float scale_log2;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) fwd_kernel(FwdParams p) {
  constexpr int KT = 64;           // keys per iteration
  constexpr int DP = D + 8;
  constexpr int VP = KT + 8;
  constexpr int KC = D / 16;
  constexpr int ND = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sK[KT * DP];   // K tile [key][d]
  __shared__ __attribute__((aligned(16))) bf16 sVT[D * VP];   // V tile [d][key]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int S = p.S;
  const long long bh = blockIdx.y;
  const int q0 = blockIdx.x * 128;
  const int qrow = q0 + 32 * w + l32;   // this lane's query
  const bf16* qh = p.q + bh * S * D;
  const long long kvh = (bh / p.H) * (p.H / p.group) + (bh % p.H) / p.group;  // this query head's K/V head
  const bf16* kh = p.k + kvh * S * D;
  const bf16* vh = p.v + kvh * S * D;

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

  int kend = S;
  if (CAUSAL) kend = (q0 + 128 < S) ? q0 + 128 : S;
  for (int k0 = 0; k0 < kend; k0 += KT) {
    __syncthreads();
    // stage K (row-major) and V (transposed) for keys k0..k0+63
    for (int ch = tid; ch < KT * D / 8; ch += 256) {
      const int key = ch / (D / 8), dg = ch % (D / 8);
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (k0 + key < S) val = *(const u32x4*)(kh + (size_t)(k0 + key) * D + dg * 8);
      *(u32x4*)&sK[key * DP + dg * 8] = val;
    }
    for (int pc = tid; pc < (KT / 4) * (D / 8); pc += 256) {
      const int kg = pc / (D / 8), dg = pc % (D / 8);
      bf16x8 rows[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = k0 + kg * 4 + rr;
        u32x4 val = u32x4{0u, 0u, 0u, 0u};
        if (key < S) val = *(const u32x4*)(vh + (size_t)key * D + dg * 8);
        rows[rr] = __builtin_bit_cast(bf16x8, val);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 t;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) t[rr] = rows[rr][e];
        *(bf16x4*)&sVT[(dg * 8 + e) * VP + kg * 4] = t;
      }
    }
    __syncthreads();

    f32x16 st[2];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc = zero16();
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const bf16x8 a = *(const bf16x8*)&sK[(32 * kb + l32) * DP + 16 * c + 8 * hh];
        acc = mfma32(a, Qr[c], acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4);
        const bool vis = key < S && (!CAUSAL || key <= qrow);
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
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 pb0 = pack8(st[kb], 0), pb1 = pack8(st[kb], 8);
#pragma unroll
      for (int n = 0; n < ND; ++n) {
        const bf16* rv = &sVT[(32 * n + l32) * VP + 32 * kb + 4 * hh];
        const bf16x8 va0 = cat44(*(const bf16x4*)rv, *(const bf16x4*)(rv + 8));
        const bf16x8 va1 = cat44(*(const bf16x4*)(rv + 16), *(const bf16x4*)(rv + 24));
        oacc[n] = mfma32(va0, pb0, oacc[n]);
        oacc[n] = mfma32(va1, pb1, oacc[n]);
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
