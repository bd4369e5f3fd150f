// LDS helpers shared by the forward and backward kernels (gfx950): the
// transposing LDS read, the chunk swizzle of staged bf16 rows, and the
// transposed operand reads of 8 staged rows in MFMA C-row order.
#pragma once

#include "common.hpp"

namespace attn {

// Transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// supplies the address of a 4-element row chunk and receives element i % 4 of
// the chunks supplied by lanes 4e + i / 4, e = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Staged rows (Q and dO in the backward, K and V in the forward) hold D bf16
// without padding, in 16-byte chunks; chunk c of row r sits at position c ^ swz(r). With 64 LDS banks of 4 bytes,
// a 16-byte read serves 16 lanes per pass and an 8-byte read 32 lanes:
//  - row-wise reads (16 consecutive rows, one chunk each) land on 16
//    different positions (D = 128: 256-byte rows, swz bijective on r mod 16;
//    D = 64: 128-byte rows, swz bijective on the even and on the odd rows);
//  - transposed reads (4 consecutive rows, 4 consecutive chunks of an aligned
//    group) land on 16 different positions, because swz gives 4 consecutive
//    rows (D = 64: the two of each parity) different bits above the two lowest.
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dims");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Transposed operand reads of staged rows (see swz), lane constants for any
// wave: the operand of 32-column block n (columns 32 n + lane % 32) over the 8
// rows blk + 16 h2 + {4 hh + 0..3, 8 + 4 hh + 0..3} (hh = lane / 32), the row
// order in which an MFMA result's C matrix hands a lane its 8 k-values.
struct TrLane {
  int base[2], hi;
  template <int D>
  __device__ __forceinline__ void init(int lane) {
    constexpr int RB = 2 * D;
    const int hh = lane >> 5, g = lane >> 4, e = (lane >> 2) & 3, t = lane & 3;
    hi = D == 128 ? e : e >> 1;
#pragma unroll
    for (int part = 0; part < 2; ++part)
      base[part] = (4 * hh + e) * RB + 16 * ((2 * (g & 1) + (t >> 1)) ^ (2 * part + hh)) + 8 * (t & 1);
  }
};
template <int RB>
__device__ __forceinline__ bf16x8 trB(const char* blk, int h2, const int* tb, int nx) {
  return cat44(lds_read_tr((const bf16*)(blk + 16 * h2 * RB + tb[0] + nx)),
               lds_read_tr((const bf16*)(blk + (16 * h2 + 8) * RB + tb[1] + nx)));
}

}  // namespace attn
