// Matrix-core rotation helpers shared by the quantize kernels for gfx950: the blockdiag(H_n)
// fragments of the 16x16x32 MFMA layout, cross-lane reductions, and the exact (fp64) rounding
// decision of the near-tie paths.
//
// Layout (16-row sub-tiles): lane l = 16 g + j holds row j of the sub-tile; the B operand of K step
// K is input channels 32 K + 8 g + e, and MFMA row i of a wave's I-block I is output channel
// c = (R/4) w + 8 (i >> 2) + 4 I + (i & 3) (R = 128; R = 64 uses one I-block), so lane l ends with
// output channels (R/4) w + 8 g + [0, 8) of row j.  Every 16 x 32 block of blockdiag(H_n), n = 2^LG,
// factors bit by bit into beta(w, K), from the bits of c and c' that the wave index and the K step
// set alone (a sign, or zero outside the diagonal blocks), times a fragment F_I over the remaining
// bits, so two fragment registers per wave hold the transform.
#pragma once

#include "kvq_device.h"

namespace kvq {
namespace rot {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int DT> __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
}

template <int DT> __device__ __forceinline__ double widen64(uint32_t h) {
  return (double)(DT == DT_F16 ? f16_to_f32(h) : bf16_to_f32(h));
}

// the rounding decision on the fp64 quotient itself: round half to even
__device__ __forceinline__ uint32_t exact_nibble(double v) {
  return (uint32_t)(int)__builtin_rint(v) & 0xfu;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max over the 16 lanes of each row (lanes 16 g .. 16 g + 15) with DPP row rotations
__device__ __forceinline__ uint32_t row_max16(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));   // row_ror:8
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));   // row_ror:4
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));   // row_ror:2
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));   // row_ror:1
  return v;
}

__device__ __forceinline__ uint32_t row_or16(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false);
  return v;
}

// fp64 sum over the wave, the same value in every lane (each step adds a pair symmetrically):
// within a 16-lane row by DPP moves (quad_perm xor 1, xor 2, row_half_mirror, row_mirror), across
// rows by v_permlane16_swap / v_permlane32_swap; no LDS round trips
template <int CTL> __device__ __forceinline__ double dpp64(double v) {
  const u32x2 p = __builtin_bit_cast(u32x2, v);
  return __builtin_bit_cast(double, u32x2{(uint32_t)__builtin_amdgcn_mov_dpp((int)p.x, CTL, 0xF, 0xF, false),
                                          (uint32_t)__builtin_amdgcn_mov_dpp((int)p.y, CTL, 0xF, 0xF, false)});
}
// v_permlane16_swap (32_swap) of a value with itself: one output holds the even (lower) row's
// value in both rows of a pair, the other the odd (upper) row's, so their sum is the pair's sum
__device__ __forceinline__ double pair_sum16(double v) {
  const u32x2 p = __builtin_bit_cast(u32x2, v);
  const auto lo = __builtin_amdgcn_permlane16_swap(p.x, p.x, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(p.y, p.y, false, false);
  return __builtin_bit_cast(double, u32x2{lo[0], hi[0]}) + __builtin_bit_cast(double, u32x2{lo[1], hi[1]});
}
__device__ __forceinline__ double pair_sum32(double v) {
  const u32x2 p = __builtin_bit_cast(u32x2, v);
  const auto lo = __builtin_amdgcn_permlane32_swap(p.x, p.x, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(p.y, p.y, false, false);
  return __builtin_bit_cast(double, u32x2{lo[0], hi[0]}) + __builtin_bit_cast(double, u32x2{lo[1], hi[1]});
}
__device__ __forceinline__ double wave_sum64(double v) {
  v += dpp64<0xB1>(v);      // quad_perm [1, 0, 3, 2]
  v += dpp64<0x4E>(v);      // quad_perm [2, 3, 0, 1]
  v += dpp64<0x141>(v);     // row_half_mirror
  v += dpp64<0x140>(v);     // row_mirror
  v = pair_sum16(v);
  return pair_sum32(v);
}

// entry (c, c') of blockdiag(H_n), n = 2^LG: zero unless c and c' share their n-block
template <int LG> __host__ __device__ constexpr int hval(int c, int cp) {
  if ((c >> LG) != (cp >> LG)) return 0;
  return (__builtin_popcount(c & cp & ((1 << LG) - 1)) & 1) ? -1 : 1;
}

template <int R> __host__ __device__ constexpr int out_channel(int w, int I, int i) {
  return R == 128 ? 32 * w + 8 * (i >> 2) + 4 * I + (i & 3) : 16 * w + 4 * (i >> 2) + (i & 3);
}
// bits of the channel numbers that are set by the wave index (c) and by the K step (c')
template <int R> constexpr int UMASK = R == 128 ? 0x60 : 0x20;

// F_{w,I}: a lane's 8 A-operand entries (row i = lane & 15, inputs 8 (lane >> 4) + e of K step 0)
// over the bits of c and c' that are not both uniform, for every lane, computed at compile time
// into a read-only table, so a wave loads its fragment instead of building it (R = 128:
// c & ~UMASK leaves no bit of w; R = 64: bit 4 of c is w & 1).
template <int DT, int R, int LG> struct alignas(16) FragTable {
  uint32_t v[R == 128 ? 1 : 2][R / 64][64][4];   // [w class][I][lane][word]
  constexpr FragTable() : v{} {
    const uint32_t one = DT == DT_F16 ? 0x3C00u : 0x3F80u;
    for (int wc = 0; wc < (R == 128 ? 1 : 2); ++wc)
      for (int I = 0; I < R / 64; ++I)
        for (int lane = 0; lane < 64; ++lane) {
          const int c = out_channel<R>(wc, I, lane & 15) & ~UMASK<R>;
          for (int q = 0; q < 4; ++q) {
            uint32_t pair = 0u;
            for (int hh = 0; hh < 2; ++hh) {
              const int hv = hval<LG>(c, (8 * (lane >> 4) + 2 * q + hh) & ~UMASK<R>);
              pair |= (hv == 0 ? 0u : (one | (hv < 0 ? 0x8000u : 0u))) << (16 * hh);
            }
            v[wc][I][lane][q] = pair;
          }
        }
  }
};
template <int DT, int R, int LG> __device__ constexpr FragTable<DT, R, LG> kFragTable{};
// F_{w,I} of this lane from the table (a 16-byte global load)
template <int DT, int R, int LG> __device__ __forceinline__ u32x4 fragment_load(int w, int I, int lane) {
  return *(const u32x4*)kFragTable<DT, R, LG>.v[R == 128 ? 0 : (w & 1)][I][lane];
}

// beta(w, K) at run time for R = 128 (w wave-uniform): the same factor as frag_beta
template <int LG> __device__ __forceinline__ int blk_beta(int w, int K) {
  return hval<LG>((32 * w) & 0x60, (32 * K) & 0x60);
}
// beta(w, K): the factor from the uniform bits
template <int R, int LG> __device__ __forceinline__ constexpr int frag_beta(int w, int K) {
  return hval<LG>(out_channel<R>(w, 0, 0) & UMASK<R>, (32 * K) & UMASK<R>);
}


}  // namespace rot
}  // namespace kvq
