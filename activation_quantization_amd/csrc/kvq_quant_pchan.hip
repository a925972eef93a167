// Per-channel quantize (PCHAN, NSEP_PCHAN) for gfx950 with the rotation on the matrix cores.
//
// Method sources (page title, section): norm-separation post "the fix" (fp16 L2 norm + unit
// direction; absmax / Q, round, clamp) and "next" (per-channel scaling); Rotated Runtime Smooth
// analysis "problem definition" (alpha = max|X| / (2^(N-1)-1)) and "term-by-term"
// (R = (1/sqrt K)[+-1]; runtime scale s_j = max over the tokens of column j); NSNQuant summary
// "Hadamard transform" (random signs, then the Hadamard matrix).
//
// Work split: a tile is (sequence, block of B tokens, head), one tile per workgroup of four
// waves (tile ids remapped so each XCD walks a contiguous range).  The tile's rows stream into
// one LDS buffer (global_load_lds, 1 KiB per wave instruction).  Wave w owns the output
// channels [w R/4, (w + 1) R/4) of every token of the tile, so the per-channel max over the
// block, the scales and the exact re-decision of near-ties are all wave-local.  Workgroup
// barriers: the rows have landed; every wave's token norms are published; every wave is done
// with the staged rows (the buffer then takes the packed code rows); the code rows are
// complete, and the tile's code block is stored whole.  With B = 128 a workgroup takes 34 KB
// of LDS and its waves at most 128 registers, so four workgroups share a CU (four waves per
// SIMD); the rotated tile is therefore not kept past the codes, and the near-tie path
// recomputes the part it needs.
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
// value is within 2^-12 of it, the flagged values in fp64 too, and the code is rne(v) of that
// fp64 quotient.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_rotate.h"

namespace kvq {
namespace {

using namespace rot;

// n / d for every 32-bit n as (umulhi(n, m) + n) >> l, with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1 (Granlund and Montgomery's round-up method, the sum taken in
// 64 bits); the tile decomposition divides wave-uniform values, so this stays in scalar registers
struct FastDiv {
  uint32_t m, l;
};
FastDiv fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  return FastDiv{(uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1), l};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.l);
}

template <int DT, int R, int LG, int B>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(B > 128 ? 3 : 4)))
quant_pchan_tile(QuantArgs a, int64_t ntiles, FastDiv nb_div, FastDiv heads_div) {
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
  // the head's random signs as fp16/bf16 sign-bit masks: word p holds channel 2p in bit 15 and
  // channel 2p + 1 in bit 31
  __shared__ __attribute__((aligned(16))) uint32_t sgm[R / 2];
  __shared__ __attribute__((aligned(16))) float ninv[16 * ST];         // [j][s]: 1 / norm of token 16 s + j

  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, in a scalar register
  // tile ids fit 32 bits (the launcher keeps them below 2^31)
  // Tiles are numbered along the head-major output streams (block fastest), so the tiles in
  // flight on one XCD write neighbouring blocks of one stream.
  uint32_t tile;
  {
    const uint32_t x = blockIdx.x & 7u, k = blockIdx.x >> 3, per = (uint32_t)ntiles >> 3, rem = (uint32_t)ntiles & 7u;
    tile = x * per + (x < rem ? x : rem) + k;                 // each XCD walks a contiguous range
  }
  const uint32_t nb = (uint32_t)(a.tokens / B);
  const uint32_t hs32 = fdiv(tile, nb_div), blk = tile - hs32 * nb;     // hs = seq * heads + h
  const uint32_t seq = fdiv(hs32, heads_div), h = hs32 - seq * (uint32_t)a.heads;
  const int64_t row0 = (int64_t)seq * a.in_seq_tokens + (int64_t)blk * B;   // x row of the tile's first token
  const int64_t hs = hs32;                                            // (sequence, head) output stream
  const int64_t tok0 = hs * a.out_tokens + a.out_tok0 + (int64_t)blk * B;   // head-major index of that token
  const int64_t sblk = hs * (a.out_tokens / B) + a.out_tok0 / B + blk;     // its scale row

  // 1. this wave's B / 4 rows into LDS (instruction k moves 1 KiB; the chunk that lane p fetches
  //    is XOR-swizzled with its row, so slot cc of row r holds chunk cc ^ (r % CPR) and the
  //    MFMA-layout reads below are free of bank conflicts); wave 0 also fetches the signs
  uint32_t sg2 = 0u;                                        // wave 0: the signs of channels 2 lane, 2 lane + 1
  {
    const unsigned char* xw = (const unsigned char*)a.x + ((row0 + (B / 4) * w) * a.heads + h) * ROWB;
    const int64_t tok_bytes = a.heads * ROWB;               // x bytes from one token to the next
    // instruction k reads rows RPI k + lane / CPR: a wave-uniform 64-bit base plus a 32-bit lane
    // offset (below 8 rows of at most 2^20 heads x 256 bytes: the descriptor check caps heads at 2^20)
    constexpr int RPI = 64 / CPR;                             // rows per load instruction
    const uint32_t lrow = (uint32_t)(lane / CPR);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int row = RPI * k + (int)lrow, cc = lane % CPR;
      const unsigned char* base = xw + (int64_t)(RPI * k) * tok_bytes;
      const uint32_t off = lrow * (uint32_t)tok_bytes + 16u * (uint32_t)(cc ^ ((row + (B / 4) * w) % CPR));
      __builtin_amdgcn_global_load_lds((const void*)(base + off),
                                       (__attribute__((address_space(3))) void*)(stage + w * WSTAGE + k * 1024), 16, 0, KVQ_LOAD_NT);
    }
    if constexpr (LG != 0) {
      if (w == 0 && lane < R / 2) sg2 = *(const uint16_t*)(a.signs + h * R + 2 * lane);
    }
  }
  // this wave's base fragments F_I (the random signs and the block signs beta(w, K) are folded
  // in once the signs have landed), loaded while the rows are in flight
  u32x4 fb0[NIW];
  if constexpr (LG != 0) {
#pragma unroll
    for (int I = 0; I < NIW; ++I) fb0[I] = fragment_load<DT, R, LG>(w, I, lane);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this wave's rows (and the signs) have landed
  asm volatile("" ::: "memory");
  if constexpr (LG != 0) {
    // sign byte bit 7 -> bit 15 / bit 31
    if (w == 0 && lane < R / 2) sgm[lane] = __builtin_amdgcn_perm(0u, sg2, 0x010C000Cu) & 0x80008000u;
  }
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
        const uint32_t bm = bt < 0 ? 0x80008000u : 0u;
        const u32x4 m = *(const u32x4*)(sgm + 16 * K + 4 * g) ^ u32x4{bm, bm, bm, bm};   // channels 32 K + 8 g + [0, 8)
#pragma unroll
        for (int I = 0; I < NIW; ++I) fk[K][I] = fb0[I] ^ m;
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
  // 5. scales and inverse scales
  float iv[LCH];
  if constexpr (LCH == 8) {
    // the max over the 16 lanes of a row as a reduce-scatter (values >= 0, compared as bits):
    // each exchange halves the slots a lane keeps (partner j ^ 8, then the mirror within 8
    // lanes, then j ^ 2) and the last one (j ^ 1) completes the max, so lane j ends with slot
    // j >> 1.  That lane computes the slot's inverse scale and stores its scale (even j); the
    // inverse scales are then broadcast back from lanes 2 q.
    auto dpp = [](uint32_t v, auto ctl) {
      return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, decltype(ctl)::value, 0xF, 0xF, false);
    };
    using ROR8 = std::integral_constant<int, 0x128>;      // row_ror:8 (= lane j ^ 8)
    using HMIR = std::integral_constant<int, 0x141>;      // row_half_mirror
    using QX2 = std::integral_constant<int, 0x4E>;        // quad_perm [2, 3, 0, 1]
    using QX1 = std::integral_constant<int, 0xB1>;        // quad_perm [1, 0, 3, 2]
    const bool h8 = (j & 8) != 0, h4 = (j & 4) != 0, h2 = (j & 2) != 0;
    uint32_t m4[4], m2[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = __builtin_bit_cast(uint32_t, mxf[k]), hi = __builtin_bit_cast(uint32_t, mxf[k + 4]);
      m4[k] = umax(h8 ? hi : lo, dpp(h8 ? lo : hi, ROR8{}));
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) m2[k] = umax(h4 ? m4[k + 2] : m4[k], dpp(h4 ? m4[k] : m4[k + 2], HMIR{}));
    uint32_t m1 = umax(h2 ? m2[1] : m2[0], dpp(h2 ? m2[0] : m2[1], QX2{}));
    m1 = umax(m1, dpp(m1, QX1{}));
    const float m = __builtin_bit_cast(float, m1);
    const float ivl = m > 0.f ? a.q * __builtin_amdgcn_rcpf(m) : 0.f;
    if ((j & 1) == 0) a.scales[sblk * R + (R / 4) * w + LCH * g + (j >> 1)] = (uint16_t)f32_to_f16(m * a.scale_mul);
    auto bcast = [&](auto qc) {   // row_newbcast: lane 2 q of each row to the whole row
      return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, ivl), 0x150 + 2 * decltype(qc)::value, 0xF, 0xF, true));
    };
    iv[0] = bcast(std::integral_constant<int, 0>{});
    iv[1] = bcast(std::integral_constant<int, 1>{});
    iv[2] = bcast(std::integral_constant<int, 2>{});
    iv[3] = bcast(std::integral_constant<int, 3>{});
    iv[4] = bcast(std::integral_constant<int, 4>{});
    iv[5] = bcast(std::integral_constant<int, 5>{});
    iv[6] = bcast(std::integral_constant<int, 6>{});
    iv[7] = bcast(std::integral_constant<int, 7>{});
  } else {
    // (lane j < LCH stores channel (R/4) w + LCH g + j)
    uint32_t s16 = 0u;
#pragma unroll
    for (int q = 0; q < LCH; ++q) {
      const float m = __builtin_bit_cast(float, row_max16(__builtin_bit_cast(uint32_t, mxf[q])));
      iv[q] = m > 0.f ? a.q * __builtin_amdgcn_rcpf(m) : 0.f;
      if (q == j) s16 = f32_to_f16(m * a.scale_mul);
    }
    if (j < LCH) a.scales[sblk * R + (R / 4) * w + LCH * g + j] = (uint16_t)s16;
  }

  // 6. codes and near-tie flags
  uint32_t pk[ST];
  uint32_t fl = 0xffffffffu, fl1 = 0xffffffffu;            // flags of I-block 0 and of I-block 1
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    uint32_t b[8];
#pragma unroll
    for (int q = 0; q < LCH; ++q) b[q] = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[s][q >> 2][q & 3], iv[q], CODE_MAGIC));
    if constexpr (LCH == 8) {
      fl = min3_u16(fl, b[0], b[1]);
      fl = min3_u16(fl, b[2], b[3]);
      fl1 = min3_u16(fl1, b[4], b[5]);
      fl1 = min3_u16(fl1, b[6], b[7]);
    } else {
      fl = min3_u16(fl, b[0], b[1]);
      fl = min3_u16(fl, b[2], b[3]);
      b[4] = b[5] = b[6] = b[7] = 0x00080000u;              // code 0 padding (dropped on store)
    }
    pk[s] = pack8(b);
  }

  // 7. rare path, wave-local: exact re-decision of this wave's near-ties.  The rotated values are
  //    not kept past step 6 (that would hold 64 more registers through the common path): the path
  //    recomputes one I-block at a time with the same matrix-core sequence (same operands, same
  //    K order, same accumulator start), so every value, flag and code it sees is bit for bit the
  //    one step 6 saw.  One code path serves every flagged channel: the channel's lane slot is a
  //    wave-uniform runtime value and the tokens to evaluate exactly are bit masks walked by a
  //    single loop, so the path stays small in the instruction cache.
  const uint64_t flagged0 = __ballot((fl & 0xffffu) == 0u), flagged1 = NIW == 2 ? __ballot((fl1 & 0xffffu) == 0u) : 0ull;
  if ((flagged0 | flagged1) != 0ull) {
    const double qd = (double)a.q;
    // exact unnormalized y (a sum of fp16/bf16 values, exact in fp64) and norm of tile rows ra
    // and rb for channel c, side by side so their wave reductions overlap: lane l takes inputs
    // l, l + 64, ... (each row's sums are accumulated and reduced in the same order either way)
    auto exact2 = [&](int ra, int rb, int c, double& ya, double& nua, double& yb, double& nub) {
      double sa = 0.0, sb = 0.0;
      ya = yb = 0.0;
#pragma unroll
      for (int e = 0; e < R / 64; ++e) {
        const int p = lane + 64 * e;
        const int off = 16 * (p >> 3), lo = 2 * (p & 7);
        const double xa = widen64<DT>(*(const uint16_t*)(stage + ra * ROWB + (off ^ (16 * (ra % CPR))) + lo));
        const double xb = widen64<DT>(*(const uint16_t*)(stage + rb * ROWB + (off ^ (16 * (rb % CPR))) + lo));
        sa = __builtin_fma(xa, xa, sa);
        sb = __builtin_fma(xb, xb, sb);
        const int hv = LG == 0 ? (p == c ? 1 : 0) : hval<LG>(c, p);
        const bool neg = (hv < 0) != (LG != 0 && ((sgm[p >> 1] >> (15 + 16 * (p & 1))) & 1u) != 0u);
        if (hv != 0) {
          ya += neg ? -xa : xa;
          yb += neg ? -xb : xb;
        }
      }
      sa = wave_sum64(sa);
      sb = wave_sum64(sb);
      ya = wave_sum64(ya);
      yb = wave_sum64(yb);
      nua = sqrt(sa);
      nub = sqrt(sb);
    };
    // step 3's rotation of sub-tile s, I-block I, times step 4's 1 / norm (w and I at run time)
    // (op is an opaque zero added to the operand addresses, so the reads stay inside the I loop
    // instead of being hoisted out of it with every sub-tile's operands live)
    auto rotated = [&](int s, int I, const u32x4& fbI, int op) {
      auto rx = [&](int K) {
        return *(const u32x4*)(stage + op + 16 * s * ROWB + (j * ROWB + 16 * ((4 * K + g) ^ (j % CPR))));
      };
      f32x4 us = {0.f, 0.f, 0.f, 0.f};
      if constexpr (LG == 0) {
        const int c0 = (R / 4) * w + LCH * g;
        const uint32_t e0 = (uint32_t)((c0 & 7) >> 1);
        const u32x4 xr = R == 128 ? rx(w) : *(const u32x4*)(stage + op + 16 * s * ROWB + (j * ROWB + 16 * ((c0 >> 3) ^ (j % CPR))));
        const uint32_t i0 = (e0 + 2 * I) & 3, i1 = (e0 + 2 * I + 1) & 3;
        const uint32_t w0 = i0 == 0 ? xr.x : i0 == 1 ? xr.y : i0 == 2 ? xr.z : xr.w;
        const uint32_t w1 = i1 == 0 ? xr.x : i1 == 1 ? xr.y : i1 == 2 ? xr.z : xr.w;
        us = f32x4{lo_f32<DT>(w0), hi_f32<DT>(w0), lo_f32<DT>(w1), hi_f32<DT>(w1)};
      } else {
#pragma unroll
        for (int K = 0; K < NK; ++K) {
          const int bt = frag_beta<R, LG>(w, K);
          if (bt == 0) continue;
          const uint32_t bm = bt < 0 ? 0x80008000u : 0u;
          const u32x4 m = *(const u32x4*)(sgm + 16 * K + 4 * g) ^ u32x4{bm, bm, bm, bm};
          us = mfma16<DT>(fbI ^ m, rx(K), us);
        }
      }
      return us * ninv[j * ST + s];
    };
#pragma unroll 1
    for (int I = 0; I < NIW; ++I) {
      if ((I == 0 ? flagged0 : flagged1) == 0ull) continue;  // no near-tie in this I-block
      // an opaque zero: the fragments and operand reads below are recomputed here rather than
      // matched to the common path's and kept live through it
      int op = 0;
      asm volatile("" : "+v"(op));
      const u32x4 fbI = LG != 0 ? fragment_load<DT, R, LG>(w, I, lane + op) : u32x4{0u, 0u, 0u, 0u};
      f32x4 us[ST];
#pragma unroll
      for (int s = 0; s < ST; ++s) us[s] = rotated(s, I, fbI, op);
      float ivI[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ivI[r] = NIW == 1 || I == 0 ? iv[r] : iv[(4 + r) % LCH];
      uint32_t cm = 0u;                                     // bit r: channel (R/4) w + LCH g + 4 I + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t mn = 0xffffffffu;
#pragma unroll
        for (int s = 0; s < ST; s += 2)
          mn = min3_u16(mn, __builtin_bit_cast(uint32_t, __builtin_fmaf(us[s][r], ivI[r], CODE_MAGIC)),
                        __builtin_bit_cast(uint32_t, __builtin_fmaf(us[s + 1][r], ivI[r], CODE_MAGIC)));
        cm |= ((mn & 0xffffu) == 0u ? 1u : 0u) << r;
      }
      // OR over the 16 lanes of each row, then the four rows side by side
      cm = row_or16(cm);
      uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)cm, 0) | ((uint32_t)__builtin_amdgcn_readlane((int)cm, 16) << 4) |
                      ((uint32_t)__builtin_amdgcn_readlane((int)cm, 32) << 8) |
                      ((uint32_t)__builtin_amdgcn_readlane((int)cm, 48) << 12);
      while (bits) {
        const int cl = __builtin_ctz(bits);                 // wave-uniform
        bits &= bits - 1u;
        const int gc = cl >> 2, r = cl & 3, qc = 4 * I + r; // lane row, slot in the lane
        const int c = (R / 4) * w + LCH * gc + qc;
        float uq[ST];
#pragma unroll
        for (int s = 0; s < ST; ++s) uq[s] = r == 0 ? us[s][0] : r == 1 ? us[s][1] : r == 2 ? us[s][2] : us[s][3];
        const float ivq = r == 0 ? ivI[0] : r == 1 ? ivI[1] : r == 2 ? ivI[2] : ivI[3];
        // per lane of row gc, bit s: token 16 s + j is near the fp32 max (within 2^-12 of it) / is
        // flagged
        uint32_t hn = 0u, hf = 0u;
#pragma unroll
        for (int s = 0; s < ST; ++s) {
          hn |= (fabsf(uq[s]) * ivq >= a.q * (1.f - 0x1p-12f) ? 1u : 0u) << s;
          hf |= ((__builtin_bit_cast(uint32_t, __builtin_fmaf(uq[s], ivq, CODE_MAGIC)) & 0xffffu) == 0u ? 1u : 0u) << s;
        }
        if (g != gc) hn = hf = 0u;
        // the next token of a kind, lane by lane (wave-uniform result; -1 once the kind is spent)
        auto pop = [&](uint32_t& hm) {
          const uint64_t lanes = __ballot(hm != 0u);
          if (lanes == 0ull) return -1;
          const int lj = (int)__builtin_ctzll(lanes);
          const int sb = __builtin_ctz((uint32_t)__builtin_amdgcn_readlane((int)hm, lj));
          if (lane == lj) hm &= hm - 1u;
          return 16 * sb + (lj & 15);                       // tile row
        };
        // every near token before any flagged one: the one holding the channel's exact max keeps
        // its |y| and norm; every flagged value is then re-decided from v = Q (y / |y_max|)
        // (nu_max / nu) (the second factor only with NSEP): Q y / |y_max| is one correctly rounded
        // division of exact values, so an exact tie between tokens of equal norm stays an exact
        // tie and rounds half to even.  Two tokens per pass (a near one then a flagged one in the
        // common case of one each); a flagged token is decided only after every near one is done.
        double um = 0.0, ym = 0.0, num = 0.0;
        auto take = [&](int t, bool flagged, double yex, double nu) {
          if (!flagged) {
            const double ua = a.nsep ? (nu > 0.0 ? fabs(yex) / nu : 0.0) : fabs(yex);
            if (ua > um) { um = ua; ym = fabs(yex); num = nu; }
          } else if (lane == 16 * gc + (t & 15)) {
            double v = 0.0;
            if (ym > 0.0 && yex != 0.0) v = a.nsep ? (qd * yex / ym) * (num / nu) : qd * yex / ym;
            const uint32_t nib = exact_nibble(v) << (4 * qc), keep = ~(0xFu << (4 * qc));
#pragma unroll
            for (int s = 0; s < ST; ++s)
              if (s == (t >> 4)) pk[s] = (pk[s] & keep) | nib;
          }
        };
#pragma unroll 1
        while (true) {
          int ta = pop(hn);
          bool fa = false;
          if (ta < 0) { ta = pop(hf); fa = true; }
          if (ta < 0) break;
          int tb = fa ? -1 : pop(hn);
          bool fb = false;
          if (tb < 0) { tb = pop(hf); fb = true; }
          double ya, nua, yb, nub;
          exact2(ta, tb < 0 ? ta : tb, c, ya, nua, yb, nub);
          take(ta, fa, ya, nua);
          if (tb >= 0) take(tb, fb, yb, nub);
        }
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
      __builtin_nontemporal_store(*(const u32x4*)(stage + w * (B * RB / 4) + 16 * pc), (u32x4*)(cb + 16 * pc));
  }
}

template <int DT, int R, int LG>
void launch_r(const QuantArgs& a, hipStream_t st) {
  const int64_t ntiles = a.seqs * (a.tokens / a.block) * a.heads;
  const FastDiv nbd = fast_div((uint32_t)(a.tokens / a.block)), hd = fast_div((uint32_t)a.heads);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles, nbd, hd); };
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
