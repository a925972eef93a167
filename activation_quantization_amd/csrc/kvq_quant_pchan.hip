// Per-channel quantize (PCHAN, NSEP_PCHAN) for gfx950 with the rotation on the matrix cores.
//
// Method sources (page title, section): norm-separation post "the fix" (fp16 L2 norm + unit
// direction; absmax / Q, round, clamp) and "next" (per-channel scaling); Rotated Runtime Smooth
// analysis "problem definition" (alpha = max|X| / (2^(N-1)-1)) and "term-by-term"
// (R = (1/sqrt K)[+-1]; runtime scale s_j = max over the tokens of column j); NSNQuant summary
// "Hadamard transform" (random signs, then the Hadamard matrix).
//
// Work split: a tile is (sequence, block of B tokens, head).  Persistent workgroups of four
// waves walk the tiles of their XCD's range; the rows of the next tile stream into a second
// LDS buffer (global_load_lds, 1 KiB per wave instruction) while the current tile is
// computed.  Wave w owns the output channels [w R/4, (w + 1) R/4) of every token of the tile,
// so the per-channel max over the block, the scales and the exact re-decision of near-ties
// are all wave-local.  Two workgroup barriers per tile: one publishes the token norms, one
// hands the assembled code rows over, which the next iteration stores whole.
//
// Rotation: Y^T = blockdiag(H_n) diag(sigma) X^T in 16-token sub-tiles with
// v_mfma_f32_16x16x32 (fp16 or bf16 operands, fp32 accumulation; the +-1 products are exact).
// In a sub-tile, lane l = 16 g + j holds token j; the B operand of K step K is channels
// 32 K + 8 g + e, and MFMA row i of the wave's local I-block I is channel
// c = (R/4) w + 8 (i >> 2) + 4 I + (i & 3) (R = 128; R = 64 uses one I-block), so lane l
// receives channels (R/4) w + 8 g + [0, 8) of token j.  Every 16 x 32 block of the n x n matrix
// factors bit by bit into beta(w, K), from the bits of c and c' that are set by w and K alone
// (a sign, or zero outside the diagonal blocks), times a fragment F_{w,I} over the remaining
// bits, so two fragment registers per wave hold the transform.  The random signs and beta flip
// the sign bits of the B operand.  The transform is left unnormalized: 1/sqrt(n) cancels
// in every quotient and only enters the stored scale.
//
// Scales: u = y / ||y|| (||y|| = ||x||, from the input with exact fp16/bf16 squares).  Codes:
// one fma per value, b = bits(u * (Q / m) + 136.5): byte 2 of b is code + 8 (round half up on a
// 2^-16 grid) and b & 0xffff == 0 marks a near-tie, |v - (k + 1/2)| <= 2^-17.  Near-ties are
// re-decided exactly: the channel's max is recomputed in fp64 from the tokens whose fp32
// value is within 2^-12 of it, the flagged values in fp64 too, and the code is rne(fp32(v)).
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

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

__device__ __forceinline__ uint32_t exact_nibble(double v) {
  return (uint32_t)(int)__builtin_rintf((float)v) & 0xfu;
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

__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// entry (c, c') of blockdiag(H_n), n = 2^LG: zero unless c and c' share their n-block
template <int LG> __device__ __forceinline__ constexpr int hval(int c, int cp) {
  if ((c >> LG) != (cp >> LG)) return 0;
  return (__builtin_popcount(c & cp & ((1 << LG) - 1)) & 1) ? -1 : 1;
}

template <int R> __device__ __forceinline__ constexpr int out_channel(int w, int I, int i) {
  return R == 128 ? 32 * w + 8 * (i >> 2) + 4 * I + (i & 3) : 16 * w + 4 * (i >> 2) + (i & 3);
}
// bits of the channel numbers that are set by the wave index (c) and by the K step (c')
template <int R> constexpr int UMASK = R == 128 ? 0x60 : 0x20;

// F_{w,I}: this lane's 8 A-operand entries (row i = lane & 15, inputs 8 (lane >> 4) + e of K
// step 0) over the bits of c and c' that are not both uniform
template <int DT, int R, int LG> __device__ __forceinline__ u32x4 hadamard_fragment(int w, int I, int lane) {
  const int c = out_channel<R>(w, I, lane & 15) & ~UMASK<R>;
  const uint32_t one = DT == DT_F16 ? 0x3C00u : 0x3F80u;
  uint32_t q4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t pair = 0u;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int cp = (8 * (lane >> 4) + 2 * q + hh) & ~UMASK<R>;
      const int v = hval<LG>(c, cp);
      pair |= (v == 0 ? 0u : (one | (v < 0 ? 0x8000u : 0u))) << (16 * hh);
    }
    q4[q] = pair;
  }
  return u32x4{q4[0], q4[1], q4[2], q4[3]};
}
// beta(w, K): the factor from the uniform bits
template <int R, int LG> __device__ __forceinline__ constexpr int frag_beta(int w, int K) {
  return hval<LG>(out_channel<R>(w, 0, 0) & UMASK<R>, (32 * K) & UMASK<R>);
}

template <int DT, int R, int LG, int B>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
quant_pchan_tile(QuantArgs a, int64_t ntiles) {
  constexpr int NK = R / 32;            // K steps of the contraction
  constexpr int NIW = R / 64;           // output I-blocks per wave
  constexpr int LCH = 4 * NIW;          // channels per lane and token
  constexpr int ST = B / 16;            // sub-tiles per tile
  constexpr int OWN = B / 64;           // sub-tiles whose norms this wave computes
  constexpr int ROWB = 2 * R;           // input row bytes
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  constexpr int TSTAGE = B * ROWB;      // bytes of the staged tile
  constexpr int WSTAGE = TSTAGE / 4;    // bytes each wave loads (B / 4 rows)
  constexpr int NLD = WSTAGE / 1024;    // load instructions per wave
  constexpr int RB = R / 2;             // code row bytes
  static_assert(ST % 4 == 0 && NLD >= 1, "tile shape");
  // the tile's input rows; once every wave is done with them, the packed code rows
  // [token][R/2 bytes] (wave w fills bytes [(R/8) w, (R/8)(w + 1)) of every row), which are
  // then stored as one contiguous block (head-major codes)
  __shared__ __attribute__((aligned(16))) unsigned char stage[TSTAGE];
  __shared__ __attribute__((aligned(16))) int8_t sg[R];                 // the head's random signs
  __shared__ __attribute__((aligned(16))) float ninv[16 * ST];         // [j][s]: 1 / norm of token 16 s + j

  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in a scalar register
  // tile ids fit 32 bits (a tile holds >= 8 KiB of input); 32-bit divisions are much cheaper
  // Tiles are numbered along the head-major output streams (block fastest), so the tiles in
  // flight on one XCD write neighbouring blocks of one stream.
  const uint32_t tile = (uint32_t)xcd_tile(blockIdx.x, ntiles);
  const uint32_t nb = (uint32_t)(a.tokens / B);
  const uint32_t hs32 = tile / nb, blk = tile - hs32 * nb;              // hs = seq * heads + h
  const uint32_t seq = hs32 / (uint32_t)a.heads, h = hs32 - seq * (uint32_t)a.heads;
  const int64_t row0 = (int64_t)seq * a.in_seq_tokens + (int64_t)blk * B;   // x row of the tile's first token
  const int64_t hs = hs32;                                            // (sequence, head) output stream
  const int64_t tok0 = hs * a.out_tokens + a.out_tok0 + (int64_t)blk * B;   // head-major index of that token
  const int64_t sblk = hs * (a.out_tokens / B) + a.out_tok0 / B + blk;     // its scale row

  // 1. this wave's B / 4 rows into LDS (instruction k moves 1 KiB; the chunk that lane p fetches
  //    is XOR-swizzled with its row, so slot cc of row r holds chunk cc ^ (r % CPR) and the
  //    MFMA-layout reads below are free of bank conflicts); wave 0 also fetches the signs
  {
    const unsigned char* xw = (const unsigned char*)a.x + ((row0 + (B / 4) * w) * a.heads + h) * ROWB;
    const uint32_t tok_bytes = (uint32_t)(a.heads * ROWB);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int p = 64 * k + lane, row = p / CPR, cc = p % CPR;
      const uint32_t off = (uint32_t)row * tok_bytes + 16u * (uint32_t)(cc ^ ((row + (B / 4) * w) % CPR));
      __builtin_amdgcn_global_load_lds((const void*)(xw + off),
                                       (__attribute__((address_space(3))) void*)(stage + w * WSTAGE + k * 1024), 16, 0, 0);
    }
    if constexpr (LG != 0) {
      if (w == 0 && lane < R / 16)
        __builtin_amdgcn_global_load_lds((const void*)(a.signs + h * R + 16 * lane),
                                         (__attribute__((address_space(3))) void*)sg, 16, 0, 0);
    }
  }
  // this wave's base fragments F_I (the random signs and the block signs beta(w, K) are folded
  // in once the signs have landed), built while the rows are in flight
  u32x4 fb0[NIW];
  if constexpr (LG != 0) {
#pragma unroll
    for (int I = 0; I < NIW; ++I) fb0[I] = hadamard_fragment<DT, R, LG>(w, I, lane);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this wave's rows (and the signs) have landed
  asm volatile("" ::: "memory");
  lds_barrier();

  // the NK operand chunks of tile row 16 s + j: channels 32 K + 8 g + [0, 8) (the swizzle
  // (16 s + j) % CPR = j % CPR does not depend on s)
  auto read_x = [&](int s, int K) {
    return *(const u32x4*)(stage + 16 * s * ROWB + (j * ROWB + 16 * ((4 * K + g) ^ (j % CPR))));
  };
  // squared norm of token 16 s + j from the Gram matrix X X^T of the sub-tile (A = B = the same
  // registers; exact products, fp32 sums).  Token t's diagonal entry sits in lane 16 (t / 4) + t,
  // register t % 4: every lane selects register j % 4 and reads lane j + 16 (j / 4).
  auto gram_ssq = [&](const u32x4 (&x)[NK]) {
    f32x4 gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = 0; K < NK; ++K) gm = mfma16<DT>(x[K], x[K], gm);
    const float d01 = (j & 1) ? gm.y : gm.x, d23 = (j & 1) ? gm.w : gm.z;
    const float dg = (j & 2) ? d23 : d01;
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((j + 16 * (j >> 2)) << 2, __builtin_bit_cast(int, dg)));
  };

  // 2. norms of this wave's own sub-tiles -> LDS (and the stored fp16 norms)
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    const int s = OWN * w + o;
    u32x4 x[NK];
#pragma unroll
    for (int K = 0; K < NK; ++K) x[K] = read_x(s, K);
    const float ssq = gram_ssq(x);
    const float rq = __builtin_amdgcn_rsqf(ssq);            // +inf for a zero vector
    const float rinv = ssq > 0.f ? rq : 0.f;
    if (g == 0) {
      ninv[j * ST + s] = a.nsep ? rinv : 1.f;
      if (a.nsep) a.norms[tok0 + 16 * s + j] = (uint16_t)f32_to_f16(ssq * rinv);   // sqrt(ssq)
    }
  }

  // 3. the rotation of this wave's channels, sub-tile by sub-tile (unnormalized)
  f32x4 u[ST][NIW];
  auto rotate = [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    // fragments of the nonzero blocks of this wave, signed for the head
    u32x4 fk[NK][NIW];
    if constexpr (LG != 0) {
#pragma unroll
      for (int K = 0; K < NK; ++K) {
        const int bt = frag_beta<R, LG>(W, K);
        if (bt == 0) continue;
        const u32x2 s8 = *(const u32x2*)(sg + 32 * K + 8 * g);
        uint32_t m[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          m[q] = (__builtin_amdgcn_perm(0u, q < 2 ? s8.x : s8.y, (q & 1) ? 0x030C020Cu : 0x010C000Cu) & 0x80008000u) ^
                 (bt < 0 ? 0x80008000u : 0u);
#pragma unroll
        for (int I = 0; I < NIW; ++I) fk[K][I] = fb0[I] ^ u32x4{m[0], m[1], m[2], m[3]};
      }
    }
    auto one = [&](int s, f32x4 (&us)[NIW]) {
      u32x4 x[NK];
#pragma unroll
      for (int K = 0; K < NK; ++K) x[K] = read_x(s, K);
      if constexpr (LG == 0) {
        const int c0 = (R / 4) * W + LCH * g;               // no rotation: the lane's own channels
        const uint32_t e0 = (uint32_t)((c0 & 7) >> 1);
        const u32x4 xr = R == 128 ? x[W] : *(const u32x4*)(stage + 16 * s * ROWB + (j * ROWB + 16 * ((c0 >> 3) ^ (j % CPR))));
        const uint32_t xw[4] = {xr.x, xr.y, xr.z, xr.w};
#pragma unroll
        for (int I = 0; I < NIW; ++I) {
          const uint32_t w0 = xw[(e0 + 2 * I) & 3], w1 = xw[(e0 + 2 * I + 1) & 3];
          us[I] = f32x4{lo_f32<DT>(w0), hi_f32<DT>(w0), lo_f32<DT>(w1), hi_f32<DT>(w1)};
        }
      } else {
#pragma unroll
        for (int I = 0; I < NIW; ++I) us[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < NK; ++K) {
          if (frag_beta<R, LG>(W, K) == 0) continue;
#pragma unroll
          for (int I = 0; I < NIW; ++I) us[I] = mfma16<DT>(fk[K][I], x[K], us[I]);
        }
      }
    };
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      one(s, u[s]);
      // keeps the scheduler from hoisting every sub-tile's operand reads (register pressure)
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  switch (w) {
    case 0: rotate(std::integral_constant<int, 0>{}); break;
    case 1: rotate(std::integral_constant<int, 1>{}); break;
    case 2: rotate(std::integral_constant<int, 2>{}); break;
    default: rotate(std::integral_constant<int, 3>{}); break;
  }

  // 4. every wave's norms are published: u = y / norm, the per-channel maxima over the tile
  lds_barrier();
  float rn[ST];
#pragma unroll
  for (int s4 = 0; s4 < ST / 4; ++s4) {
    const f32x4 v = *(const f32x4*)(ninv + j * ST + 4 * s4);
    rn[4 * s4] = v.x; rn[4 * s4 + 1] = v.y; rn[4 * s4 + 2] = v.z; rn[4 * s4 + 3] = v.w;
  }
  float mxf[LCH];
#pragma unroll
  for (int q = 0; q < LCH; ++q) mxf[q] = 0.f;
#pragma unroll
  for (int s = 0; s < ST; ++s)
#pragma unroll
    for (int I = 0; I < NIW; ++I) {
      u[s][I] *= rn[s];
#pragma unroll
      for (int r = 0; r < 4; ++r) mxf[4 * I + r] = fmaxf(mxf[4 * I + r], fabsf(u[s][I][r]));
    }
  uint32_t mx[LCH];
#pragma unroll
  for (int q = 0; q < LCH; ++q) mx[q] = row_max16(__builtin_bit_cast(uint32_t, mxf[q]));   // values >= 0

  // 5. scales (lane j < LCH stores channel (R/4) w + LCH g + j) and inverse scales
  float iv[LCH];
  uint32_t s16 = 0u;
#pragma unroll
  for (int q = 0; q < LCH; ++q) {
    const float m = __builtin_bit_cast(float, mx[q]);
    iv[q] = m > 0.f ? a.q * __builtin_amdgcn_rcpf(m) : 0.f;
    if (q == j) s16 = f32_to_f16(m * a.scale_mul);
  }
  if (j < LCH) a.scales[sblk * R + (R / 4) * w + LCH * g + j] = (uint16_t)s16;

  // 6. codes and near-tie flags
  uint32_t pk[ST];
  uint32_t fl = 0xffffffffu;
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    uint32_t b[8];
#pragma unroll
    for (int q = 0; q < LCH; ++q) b[q] = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[s][q >> 2][q & 3], iv[q], CODE_MAGIC));
    if constexpr (LCH == 8) {
      fl = min3_u16(fl, b[0], b[1]);
      fl = min3_u16(fl, b[2], b[3]);
      fl = min3_u16(fl, b[4], b[5]);
      fl = min3_u16(fl, b[6], b[7]);
    } else {
      fl = min3_u16(fl, b[0], b[1]);
      fl = min3_u16(fl, b[2], b[3]);
      b[4] = b[5] = b[6] = b[7] = 0x00080000u;              // code 0 padding (dropped on store)
    }
    pk[s] = pack8(b);
  }

  // 7. rare path, wave-local: exact re-decision of this wave's near-ties (u is still live)
  if (__ballot((fl & 0xffffu) == 0u) != 0ull) {
    uint32_t cm = 0u;                                       // bit q: channel (R/4) w + LCH g + q
#pragma unroll
    for (int q = 0; q < LCH; ++q) {
      uint32_t mn = 0xffffffffu;
#pragma unroll
      for (int s = 0; s < ST; s += 2)
        mn = min3_u16(mn, __builtin_bit_cast(uint32_t, __builtin_fmaf(u[s][q >> 2][q & 3], iv[q], CODE_MAGIC)),
                      __builtin_bit_cast(uint32_t, __builtin_fmaf(u[s + 1][q >> 2][q & 3], iv[q], CODE_MAGIC)));
      cm |= ((mn & 0xffffu) == 0u ? 1u : 0u) << q;
    }
    // OR over the 16 lanes of each row, then the four rows side by side
    cm = row_or16(cm);
    uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)cm, 0) |
                    ((uint32_t)__builtin_amdgcn_readlane((int)cm, 16) << LCH) |
                    ((uint32_t)__builtin_amdgcn_readlane((int)cm, 32) << (2 * LCH)) |
                    ((uint32_t)__builtin_amdgcn_readlane((int)cm, 48) << (3 * LCH));
    const double qd = (double)a.q;
    // exact u of tile row r for channel c: lane l takes inputs l, l + 64, ...
    auto exact_u = [&](int r, int c) {
      double y = 0.0, ss = 0.0;
#pragma unroll
      for (int e = 0; e < R / 64; ++e) {
        const int p = lane + 64 * e;
        const uint32_t hw = *(const uint16_t*)(stage + r * ROWB + 16 * ((p >> 3) ^ (r % CPR)) + 2 * (p & 7));
        const double x = widen64<DT>(hw);
        ss = __builtin_fma(x, x, ss);
        const int hv = LG == 0 ? (p == c ? 1 : 0) : hval<LG>(c, p);
        if (hv != 0) y += ((hv < 0) != (LG != 0 && sg[p] < 0)) ? -x : x;
      }
      y = wave_sum64(y);
      ss = wave_sum64(ss);
      const double nu = sqrt(ss);
      return a.nsep ? (nu > 0.0 ? y / nu : 0.0) : y;
    };
    // one flagged channel; its lane slot Q is a compile-time constant, so u and iv are plain
    // registers (pass 0: exact max over the tokens near the fp32 max; pass 1: exact codes of
    // the flagged values)
    auto fix_channel = [&](auto qc, int gc, int c) {
      constexpr int Q = decltype(qc)::value;
      double mm = 0.0;
#pragma unroll 1
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int s = 0; s < ST; ++s) {
          const float uq = u[s][Q >> 2][Q & 3];
          const bool hit = pass == 0
                               ? fabsf(uq) * iv[Q] >= a.q * (1.f - 0x1p-12f)
                               : (__builtin_bit_cast(uint32_t, __builtin_fmaf(uq, iv[Q], CODE_MAGIC)) & 0xffffu) == 0u;
          uint64_t tok = (__ballot(g == gc && hit) >> (16 * gc)) & 0xffffull;
          while (tok) {
            const int jt = __builtin_ctzll(tok);
            tok &= tok - 1ull;
            const double uex = exact_u(16 * s + jt, c);
            if (pass == 0) {
              mm = fmax(mm, fabs(uex));
            } else if (lane == 16 * gc + jt) {
              const uint32_t nib = mm > 0.0 ? exact_nibble(qd * uex / mm) : 0u;
              pk[s] = (pk[s] & ~(0xFu << (4 * Q))) | (nib << (4 * Q));
            }
          }
        }
      }
    };
    while (bits) {
      const int cl = __builtin_ctz(bits);                   // channel (R/4) w + cl
      bits &= bits - 1u;
      const int gc = cl / LCH, c = (R / 4) * w + cl;
      switch (cl % LCH) {
        case 0: fix_channel(std::integral_constant<int, 0>{}, gc, c); break;
        case 1: fix_channel(std::integral_constant<int, 1>{}, gc, c); break;
        case 2: fix_channel(std::integral_constant<int, 2>{}, gc, c); break;
        case 3: fix_channel(std::integral_constant<int, 3>{}, gc, c); break;
        default:
          if constexpr (LCH == 8) {
            switch (cl % LCH) {
              case 4: fix_channel(std::integral_constant<int, 4 % LCH>{}, gc, c); break;
              case 5: fix_channel(std::integral_constant<int, 5 % LCH>{}, gc, c); break;
              case 6: fix_channel(std::integral_constant<int, 6 % LCH>{}, gc, c); break;
              default: fix_channel(std::integral_constant<int, 7 % LCH>{}, gc, c); break;
            }
          }
          break;
      }
    }
  }

  // 8. codes -> LDS rows (every wave is done with the staged input), then the tile's code
  //    block out in contiguous 16-byte pieces
  lds_barrier();
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    unsigned char* cp = stage + (16 * s + j) * RB + (R / 8) * w + (LCH / 2) * g;
    if constexpr (R == 128)
      *(uint32_t*)cp = pk[s];
    else
      *(uint16_t*)cp = (uint16_t)pk[s];
  }
  lds_barrier();
  // the tile's codes are one contiguous block of B R/2 bytes; wave w stores its quarter
  constexpr int WPIECES = B * RB / 64;                      // 16-byte pieces per wave
  unsigned char* cb = a.codes + tok0 * RB + w * (B * RB / 4);
#pragma unroll
  for (int k = 0; k < (WPIECES + 63) / 64; ++k) {
    const int pc = 64 * k + lane;
    if (WPIECES % 64 == 0 || pc < WPIECES)
      *(u32x4*)(cb + 16 * pc) = *(const u32x4*)(stage + w * (B * RB / 4) + 16 * pc);
  }
}

template <int DT, int R, int LG>
void launch_r(const QuantArgs& a, hipStream_t st) {
  const int64_t ntiles = a.seqs * (a.tokens / a.block) * a.heads;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles); };
  if (a.block == 64) go(quant_pchan_tile<DT, R, LG, 64>);
  else if (a.block == 128) go(quant_pchan_tile<DT, R, LG, 128>);
  else if constexpr (R == 64) go(quant_pchan_tile<DT, R, LG, 256>);
}

template <int DT, int R>
void launch_lg(const QuantArgs& a, hipStream_t st) {
  switch (a.lg_had) {
    case 0: launch_r<DT, R, 0>(a, st); break;
    case 4: launch_r<DT, R, 4>(a, st); break;
    case 5: launch_r<DT, R, 5>(a, st); break;
    case 6: launch_r<DT, R, 6>(a, st); break;
    default: if constexpr (R == 128) launch_r<DT, R, 7>(a, st); break;
  }
}

template <int DT>
void launch_dt(const QuantArgs& a, hipStream_t st) {
  if (a.dim == 128) launch_lg<DT, 128>(a, st);
  else launch_lg<DT, 64>(a, st);
}

}  // namespace

hipError_t launch_quantize_pchan(const QuantArgs& a, hipStream_t st) {
  if (a.dtype == DT_F16) launch_dt<DT_F16>(a, st);
  else launch_dt<DT_BF16>(a, st);
  return hipGetLastError();
}

}  // namespace kvq
