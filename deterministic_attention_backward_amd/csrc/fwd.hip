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
// at its diagonal. Only the tiles that cross the diagonal or the end of the
// sequence evaluate masks, and the output accumulators are rescaled only when
// some lane's running maximum grew (a factor of exactly 1 otherwise).
//
// Work order: workgroup L of the grid runs on XCD L mod 8, so the j-th
// workgroup of an XCD takes query tile level j / (heads per XCD) (longest
// first on a causal mask, over all heads) of one of that XCD's heads: a
// head's K and V are read by one XCD's L2 only, and the grid drains longest
// tiles first.
#include <type_traits>

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
  int BH;        // batch x query heads
  float scale_log2;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) fwd_kernel(FwdParams p) {
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
  long long bh;
  int level;
  {
    const int L = blockIdx.x;
    if (p.BH % 8 == 0) {  // XCD-aware: XCD x owns heads x, x + 8, ...
      const int hpx = p.BH / 8, x = L % 8, j = L / 8;
      level = j / hpx;
      bh = (long long)(j % hpx) * 8 + x;
    } else {
      level = L / p.BH;
      bh = L % p.BH;
    }
  }
  // causal: the longest query tiles (the last ones) first
  const int qt = CAUSAL ? p.n_qt - 1 - level : level;
  const int q0 = qt * 128;
  const int qrow = q0 + 32 * w + l32;   // this lane's query
  const bf16* qh = p.q + bh * S * D;
  const long long kvh = (bh / p.H) * (p.H / p.group) + (bh % p.H) / p.group;  // this query head's K/V head
  const bf16* kh = p.k + kvh * S * D;
  const bf16* vh = p.v + kvh * S * D;

  // DMA of keys k0..k0+63 (K and V) into buffer buf. Lane L of piece pr
  // fetches row pr RPP + rl, chunk lx ^ swz(pr RPP): a byte offset fixed per
  // piece (piece_off) from the tile's first row, so a full tile needs no
  // per-lane address arithmetic. On the last, partial tile keys past the end
  // are read as copies of the last key (the mask gives them P = 0 exactly).
  constexpr int CPR = D / 8, RPP = 64 / CPR, HALF = PIECES / 2;
  unsigned piece_off[PPW];
  int piece_row[PPW];
  {
    const int rl = lane / CPR, lx = (lane % CPR) ^ swz<D>(lane / CPR);
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int piece = w * PPW + k;
      const int pr = piece >= HALF ? piece - HALF : piece;
      piece_row[k] = pr * RPP + rl;
      piece_off[k] = (unsigned)(piece_row[k] * RB + 16 * (lx ^ swz<D>(pr * RPP)));
    }
  }
  auto stage_pieces = [&](int k0, int buf, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int piece = w * PPW + k;  // wave-uniform
      const bool is_v = piece >= HALF;
      const int pr = is_v ? piece - HALF : piece;
      unsigned off = piece_off[k];
      if constexpr (!FULL) off += (unsigned)((min(k0 + piece_row[k], S - 1) - k0 - piece_row[k]) * RB);
      char* dst = smem + (2 * buf + (is_v ? 1 : 0)) * TB + pr * 1024;
      __builtin_amdgcn_global_load_lds(at_bytes((is_v ? vh : kh) + (size_t)k0 * D, off),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };
  auto stage = [&](int k0, int buf) {
    if (k0 + KT <= S) stage_pieces(k0, buf, std::true_type{});  // workgroup-uniform
    else stage_pieces(k0, buf, std::false_type{});
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
  const bool pos = p.scale_log2 >= 0.0f;
  const float hidden = pos ? -__builtin_inff() : __builtin_inff();  // scaled by the scale: -inf
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

    // raw scores S^T; on tiles crossing the diagonal or the end of the
    // sequence, masked entries become the score whose scaled value is -inf
    f32x16 st[2];
    int ab = a_base, s1 = sw1;
    asm volatile("" : "+v"(ab), "+v"(s1));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const char* Kr = Kb + 32 * kb * RB + ab;
      f32x16 acc = zero16();
#pragma unroll
      for (int c = 0; c < KC; ++c) acc = mfma32(*(const bf16x8*)(Kr + ((c ^ s1) << 5)), Qr[c], acc);
      st[kb] = acc;
    }
    // P = exp2(S scale log2(e) - m) with the running maximum m brought up to
    // this tile, one fused multiply-add per score; the two instantiations keep
    // the mask code off the tiles that need none
    auto softmax = [&](auto edge_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
      if constexpr (EDGE) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4);
            if (!(key < S && (!CAUSAL || key <= qrow))) st[kb][i] = hidden;
          }
        }
      }
      // the row's largest scaled score: the largest raw score for a positive
      // scale, the smallest for a negative one
      float tsel = st[0][0];
      if (pos) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) tsel = fmaxf(tsel, st[kb][i]);
        tsel = fmaxf(tsel, __shfl_xor(tsel, 32));
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) tsel = fminf(tsel, st[kb][i]);
        tsel = fminf(tsel, __shfl_xor(tsel, 32));
      }
      const float mnew = fmaxf(m, tsel * p.scale_log2);
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fast_exp2(__builtin_fmaf(st[kb][i], p.scale_log2, -mnew));
          if constexpr (EDGE) {
            if (st[kb][i] == hidden) pv = 0.0f;  // (a zero scale would make it NaN)
          }
          st[kb][i] = pv;
          psum += pv;
        }
      }
      psum += __shfl_xor(psum, 32);
      // rescale by exp2(m - mnew): exactly 1 for the rows whose maximum did not
      // grow (a branch around it costs as much, in copies of the accumulators)
      const float alpha = fast_exp2(m - mnew);
      l = l * alpha + psum;
#pragma unroll
      for (int n = 0; n < ND; ++n) {
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[n][i] *= alpha;
      }
      m = mnew;
    };
    if (k0 + KT > S || (CAUSAL && k0 + KT > q0)) softmax(std::true_type{});  // workgroup-uniform
    else softmax(std::false_type{});
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
  fp.BH = a.B * a.H;
  fp.scale_log2 = a.scale * 1.4426950408889634f;
  const dim3 grid((unsigned)((long long)fp.n_qt * fp.BH));
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
