// Quantize kernels for gfx950: randomized Hadamard -> norm separation -> absmax scale ->
// round-half-even -> nibble packing, one pass over HBM.
//
// Method sources (page title, section): norm-separation post "the fix" (fp16 L2 norm + unit
// direction, absmax / 7, round and clamp to +-7) and "root cause" (per-row absmax);
// Rotated Runtime Smooth analysis "problem definition" (alpha = max|X| / (2^(N-1)-1)) and
// "term-by-term" (R = (1/sqrt K)[+-1]; runtime scale s_j = max over tokens of column j);
// NSNQuant summary "Hadamard transform" (randomized Hadamard before quantization).
//
// Layout: one thread owns one row of R = min(head_dim, 128) channels of one (token, head) and
// keeps it in VGPRs from load to store, so the transform needs no cross-lane traffic.  Tiles
// come in with coalesced 16-byte loads through an XOR-swizzled LDS tile and leave the same way.
//
// Arithmetic (all equal to the plain definition up to rounding):
//   * signs + first butterfly stage + fp16/bf16 -> fp32 widening in one v_dot2 per output:
//     (s0 x0 + s1 x1, s0 x0 - s1 x1) with the sign pair as a packed +-1 operand.
//   * the transform is left unnormalized (Y = H diag(s) x); 1/sqrt(n) cancels in every
//     quotient and only enters the stored scale.  ||y|| = ||x|| (orthonormal rotation), so the
//     norm is taken from the input with v_dot2 (exact squares).  For per-token scales the norm
//     cancels too: v = Q Y_c / max_c |Y_c|.
//   * one fma per code: b = bits(u * (Q/m) + 192.5) rounds v = u Q / m onto a 2^-16 grid; bits
//     16..19 of b are the code's nibble (round half up) and b & 0xffff == 0 flags a near-tie
//     (|v - (k + 1/2)| <= 2^-17).  The clamp to [-Q, Q] is implied: |u| <= m.
//   * near-ties (a few per 10^5 codes) are re-decided exactly: the affected channel (per-
//     channel scales) or vector (per-token scales) is recomputed in fp64 from the input and
//     the code is rne(v) of the fp64 quotient.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_launch.h"

namespace kvq {

constexpr float MAGIC = 192.5f;   // [128, 256): ulp 2^-16; + 0.5 turns truncation into rounding

// packed +-1 pair (s0, s1) for v_dot2; s* given as the sign bits (bit 15 and 31 positions)
template <int DT> __device__ __forceinline__ uint32_t one_pair() {
  return DT == DT_F16 ? 0x3C003C00u : 0x3F803F80u;
}
// x.lo * c.lo + x.hi * c.hi in fp32 (NEG_HI: x.lo * c.lo - x.hi * c.hi).  VOP3 form with a
// literal zero accumulator: the builtin selects the accumulate-in-place encoding, which needs
// an extra register clear per use.
template <int DT, bool NEG_HI = false> __device__ __forceinline__ float dot2(uint32_t x, uint32_t c) {
  float r;
  if constexpr (DT == DT_F16) {
    if constexpr (NEG_HI) asm("v_dot2_f32_f16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(c));
    else asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(x), "v"(c));
  } else {
    if constexpr (NEG_HI) asm("v_dot2_f32_bf16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(c));
    else asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(x), "v"(c));
  }
  return r;
}
template <int DT> __device__ __forceinline__ float dot2acc(uint32_t x, float acc) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, x), acc, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, x), acc, false);
}

// Row of packed 16-bit inputs -> fp32 after signs and the first butterfly stage (or plain
// widening without rotation).  sg: this row's R sign bytes (16-byte aligned).
template <int DT, int R>
__device__ __forceinline__ void widen_stage1(float (&y)[R], const uint32_t (&w)[R / 2], const int8_t* __restrict__ sg,
                                             bool rotate) {
  if (rotate) {
#pragma unroll
    for (int c = 0; c < R / 16; ++c) {
      // wave-uniform: read through the constant address space so it becomes a scalar load
      // (lgkmcnt), which does not wait behind the tile prefetch in flight on vmcnt
      const u32x4 sv = *(const __attribute__((address_space(4))) u32x4*)(sg + 16 * c);
      const uint32_t s4[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {           // pair k of this 16-channel group
        const uint32_t sw = s4[k >> 1];
        const uint32_t sb = (k & 1) ? (((sw >> 8) & 0x8000u) | (sw & 0x80000000u))
                                    : (((sw << 8) & 0x8000u) | ((sw << 16) & 0x80000000u));
        const uint32_t cp = one_pair<DT>() | sb;
        const int i = 8 * c + k;
        y[2 * i] = dot2<DT>(w[i], cp);
        y[2 * i + 1] = dot2<DT, true>(w[i], cp);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < R / 2; ++i) {
      y[2 * i] = lo_f32<DT>(w[i]);
      y[2 * i + 1] = hi_f32<DT>(w[i]);
    }
  }
}

// Per-lane signs (per-token kernel): flip the sign bits of the packed inputs right after
// they are loaded (v_perm moves sign byte k's bit 7 to bit 15 / 31 of its pair).
template <int R>
__device__ __forceinline__ void apply_signs_packed(uint32_t (&w)[R / 2], const int8_t* __restrict__ sg) {
#pragma unroll
  for (int c = 0; c < R / 16; ++c) {
    const u32x4 sv = *(const u32x4*)(sg + 16 * c);
    const uint32_t s4[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t sw = s4[k >> 1];
      const uint32_t m = __builtin_amdgcn_perm(0u, sw, (k & 1) ? 0x030C020Cu : 0x010C000Cu) & 0x80008000u;
      w[8 * c + k] ^= m;
    }
  }
}

template <int DT, int R>
__device__ __forceinline__ void stage1_unsigned(float (&y)[R], const uint32_t (&w)[R / 2]) {
#pragma unroll
  for (int i = 0; i < R / 2; ++i) {
    y[2 * i] = dot2<DT>(w[i], one_pair<DT>());
    y[2 * i + 1] = dot2<DT, true>(w[i], one_pair<DT>());
  }
}

// in-register butterfly stages 1 .. LG-1 on blocks of 2^LG (stage 0 is done by widen_stage1)
template <int R, int LG>
__device__ __forceinline__ void fwht_rest(float (&v)[R]) {
#pragma unroll
  for (int s = 1; s < LG; ++s) {
    const int st = 1 << s;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if ((i & st) == 0) {
        const float a = v[i], b = v[i + st];
        v[i] = a + b;
        v[i + st] = a - b;
      }
    }
  }
}

template <int DT, int R>
__device__ __forceinline__ float sum_squares_in(const uint32_t (&w)[R / 2]) {
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < R / 2; ++i) p[i & 3] = dot2acc<DT>(w[i], p[i & 3]);
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// Codes of R values with per-element inverse scale.  cw[i] holds codes 8i..8i+7 (channel
// 8i + e in nibble e).  Near-ties are reported two ways: the return value is true in lanes
// holding one, and chm (wave-uniform, R/32 words) gets bit c when any lane of the wave holds
// a near-tie in channel c (the ballot of the compare itself, reduced on the scalar unit).
template <int R, bool CHANNEL_FLAGS, typename InvF>
__device__ __forceinline__ bool quantize_row(const float (&u)[R], InvF inv, uint32_t (&cw)[R / 8], uint32_t (&chm)[R / 32]) {
  bool f = false;
#pragma unroll
  for (int g = 0; g < R / 32; ++g) chm[g] = 0u;
#pragma unroll
  for (int i = 0; i < R / 8; ++i) {
    uint32_t p[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 8 * i + 2 * k;
      const uint32_t be = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[c], inv(c), MAGIC));
      const uint32_t bo = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[c + 1], inv(c + 1), MAGIC));
      const bool fe = (be & 0xffffu) == 0u, fo = (bo & 0xffffu) == 0u;
      if constexpr (CHANNEL_FLAGS) {
        if (__ballot(fe)) chm[c >> 5] |= 1u << (c & 31);
        if (__ballot(fo)) chm[c >> 5] |= 2u << (c & 31);
      } else {
        f = f | fe | fo;
      }
      p[k] = (be & 0x000F0000u) | ((bo << 4) & ~0x000F0000u);   // byte 2 = code pair (v_bfi)
    }
    const uint32_t lo = __builtin_amdgcn_perm(p[1], p[0], 0x0C0C0602u);
    const uint32_t hi = __builtin_amdgcn_perm(p[3], p[2], 0x06020C0Cu);
    cw[i] = lo | hi;
  }
  return f;
}

// ---------------------------------------------------------------------------------- exact
// the exact rounding decision: rne of the fp64 quotient
__device__ __forceinline__ uint32_t exact_code(double v) {
  return (uint32_t)(int)__builtin_rint(v) & 0xfu;
}

// replace the nibble of channel c in row `row` of a staged code tile
__device__ __forceinline__ void patch_nibble(unsigned char* stage, int row, int crb, int c, uint32_t nib) {
  const int byte = c >> 1;
  unsigned char* p = stage + row * crb + swz_chunk(row, byte >> 4, crb) * 16 + (byte & 15);
  const uint32_t sh = (c & 1) * 4;
  *p = (unsigned char)((*p & ~(0xFu << sh)) | (nib << sh));
}

// ---------------------------------------------------------------------------------------
// Asynchronous tile load straight into LDS (global_load_lds_dwordx4: no VGPRs, completes in
// the background).  One wave instruction fills 1 KiB of LDS, lane i at +16 i; lane i fetches
// the global chunk that the XOR swizzle places there.  `rows` rows of ROWB bytes, row r at
// src + r * stride; the calling wave handles instructions w, w + nw, ...
template <int ROWB>
__device__ __forceinline__ void load_tile_lds(unsigned char* lds, const unsigned char* src, int64_t stride, int rows,
                                              int w, int nw, int lane) {
  constexpr int CPR = ROWB / 16;
  const int ninst = rows * CPR / 64;
  for (int k = w; k < ninst; k += nw) {
    const int p = k * 64 + lane;
    const int row = p / CPR, ccp = p % CPR;
    const int cc = swz_chunk(row, ccp, ROWB);   // the XOR swizzle is an involution
    __builtin_amdgcn_global_load_lds((const void*)(src + row * stride + cc * 16),
                                     (__attribute__((address_space(3))) void*)(lds + k * 1024), 16, 0, 0);
  }
}

// Exact fp64 value of channel c of the unnormalized rotation of row `r` of a staged tile
// (R signed inputs per row, XOR-swizzled), computed by the whole wave: lane l takes channels
// 2l and 2l + 1, and the sum over c's 2^LG-block is reduced across the lanes.  Exact for fp16
// inputs (a sum of 128 fp16 values fits in 53 bits); every lane returns the same value.
template <int DT, int R, int LG>
__device__ __forceinline__ double wave_exact_y(const unsigned char* tile, int r, int c) {
  constexpr int ROWB = 2 * R;
  const int lane = threadIdx.x;
  double t = 0.0;
  if (lane < R / 2) {
    const int j = 2 * lane;
    const bool in0 = ((j ^ c) >> LG) == 0, in1 = (((j + 1) ^ c) >> LG) == 0;
    if (in0 || in1) {
      const uint32_t w = *(const uint32_t*)(tile + r * ROWB + swz_chunk(r, lane >> 2, ROWB) * 16 + (lane & 3) * 4);
      double x0 = (double)lo_f32<DT>(w), x1 = (double)hi_f32<DT>(w);
      if constexpr (LG != 0) {
        constexpr int NM = (1 << LG) - 1;
        if (__builtin_popcount(c & j & NM) & 1) x0 = -x0;
        if (__builtin_popcount(c & (j + 1) & NM) & 1) x1 = -x1;
      }
      t = (in0 ? x0 : 0.0) + (in1 ? x1 : 0.0);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
  return t;
}

// Per-token rare path.  A code whose fp32 quotient lies within 2^-17 of a half-integer is
// re-decided from the exact quotient Q Y_c / max |Y| (the norm cancels in both per-token
// modes); that needs the exact Y_c and the exact max of its vector.  The fp32 transform is
// accurate to far better than a relative 2^-12 of the max, so the max is attained among the
// channels whose fp32 magnitude lies within that distance of the fp32 max ("candidates", taken
// only in vectors holding a near-tie).  Per channel, one ballot each gives the lanes with a
// near-tie and with a candidate; channels with either are queued in LDS, and each (lane,
// channel) item is then computed exactly by the whole wave: first the candidates (exact max
// per lane, reduced over the vector's L lanes), then the near-ties, patched into the staged
// codes.  tile: the staged input tile, signs applied; queue: 5 R words of LDS.  sdiv (RRS
// activations, else null): lane l's segment is divided by sdiv[l mod L] (the tile starts a vector).
template <int DT, int R, int LG>
__device__ __forceinline__ void ptok_fix(const float (&y)[R], float m, float inv_scale, float q, int L, uint64_t ball,
                                         const unsigned char* tile, unsigned char* stage_codes, uint32_t* queue,
                                         const float* sdiv) {
  constexpr int CRB = R / 2;
  const int lane = threadIdx.x;
  const uint64_t gm = (L == 64 ? ~0ull : ((1ull << L) - 1ull)) << (lane & ~(L - 1));
  const uint64_t fv = __ballot((ball & gm) != 0ull);      // lanes of vectors holding a near-tie
  const float thr = m - m * 0x1p-12f;
  int nq = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_fmaf(y[i], inv_scale, MAGIC));
    const uint64_t fb = __ballot((b & 0xffffu) == 0u) & ball;
    const uint64_t cb = __ballot(fabsf(y[i]) >= thr) & fv;
    if (fb | cb) {
      if (lane == 0) {
        queue[5 * nq] = (uint32_t)i;
        queue[5 * nq + 1] = (uint32_t)fb;
        queue[5 * nq + 2] = (uint32_t)(fb >> 32);
        queue[5 * nq + 3] = (uint32_t)cb;
        queue[5 * nq + 4] = (uint32_t)(cb >> 32);
      }
      ++nq;
    }
  }
  wave_lds_sync();
  auto entry = [&](int k, int w) -> uint64_t {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)queue[5 * k + w]);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)queue[5 * k + w + 1]);
    return ((uint64_t)hi << 32) | lo;
  };
  // the exact value of lane l's channel c (divided by the segment's divisor for RRS activations)
  auto exact = [&](int l, int c) {
    double v = wave_exact_y<DT, R, LG>(tile, l, c);
    if (sdiv) {
      const float d = sdiv[l & (L - 1)];
      v = d > 0.f ? v / (double)d : 0.0;
    }
    return v;
  };
  double mxl = 0.0;
  for (int k = 0; k < nq; ++k) {
    const int c = __builtin_amdgcn_readfirstlane((int)queue[5 * k]);
    for (uint64_t cb = entry(k, 3); cb; cb &= cb - 1ull) {
      const int l = __builtin_ctzll(cb);
      const double v = fabs(exact(l, c));
      if (lane == l) mxl = fmax(mxl, v);
    }
  }
  for (int o = 1; o < L; o <<= 1) mxl = fmax(mxl, __shfl_xor(mxl, o));
  for (int k = 0; k < nq; ++k) {
    const int c = __builtin_amdgcn_readfirstlane((int)queue[5 * k]);
    for (uint64_t fb = entry(k, 1); fb; fb &= fb - 1ull) {
      const int l = __builtin_ctzll(fb);
      const double v = exact(l, c);
      const double mx = __shfl(mxl, l);
      if (lane == l) patch_nibble(stage_codes, l, CRB, c, mx > 0.0 ? exact_code((double)q * v / mx) : 0u);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per-token modes (NAIVE, NSEP): persistent single-wave workgroups; a tile is 64 consecutive
// row segments of R channels (16 KiB for R = 128), prefetched into LDS one tile ahead.  A
// (token, head) vector of D = L * R channels spans L = 2^lgL neighbouring lanes.
template <int DT, int R, int LG>
__global__ void __launch_bounds__(64) quant_ptok_kernel(QuantArgs a, int64_t nseg, int64_t ntiles, int lgL) {
  constexpr int ROWB = R * 2, CPR = ROWB / 16, CRB = R / 2, CCR = CRB / 16;
  __shared__ __attribute__((aligned(16))) unsigned char stage_in[2][64 * ROWB];   // current / prefetched tile
  __shared__ __attribute__((aligned(16))) unsigned char stage_codes[64 * CRB];
  __shared__ uint32_t queue[5 * R];                             // near-tie work list
  const int lane = threadIdx.x;
  const int L = 1 << lgL;
  const int64_t G = gridDim.x;
  const int64_t full_tiles = nseg / 64;                         // tiles without a ragged tail
  // codes are head-major: segment `seg` (x order) goes to segment head_major(vector) L + part
  auto store_codes = [&](int64_t seg0, int nvalid) {
#pragma unroll
    for (int k = 0; k < CCR; ++k) {
      const int q = lane + k * 64;
      const int row = q / CCR, cc = q % CCR;
      if (row < nvalid) {
        const u32x4 t = *(const u32x4*)(stage_codes + row * CRB + swz_chunk(row, cc, CRB) * 16);
        const int64_t sg = seg0 + row;
        const int64_t dst = a.heads == 1 ? sg : (head_major(a.heads, a.tokens, sg >> lgL) << lgL) + (sg & (L - 1));
        __builtin_nontemporal_store(t, (u32x4*)(a.codes + dst * CRB + cc * 16));
      }
    }
  };

  // only full tiles are prefetched; the tile order is remapped per XCD, so test the tile
  // index itself (the ragged last tile is loaded with guarded loads when its turn comes)
  int64_t v = blockIdx.x;
  int64_t pseg0 = -1;
  int pvalid = 0;
  if (v < ntiles && xcd_tile(v, ntiles) < full_tiles)
    load_tile_lds<ROWB>(stage_in[0], (const unsigned char*)a.x + xcd_tile(v, ntiles) * 64 * ROWB, ROWB, 64, 0, 1, lane);
  for (int buf = 0; v < ntiles; v += G, buf ^= 1) {
    unsigned char* const tile = stage_in[buf];
    const int64_t seg0 = xcd_tile(v, ntiles) * 64;
    const int nvalid = (int)(nseg - seg0 < 64 ? nseg - seg0 : 64);
    const unsigned char* xb = (const unsigned char*)a.x + seg0 * ROWB;
    if (nvalid < 64) {
      // ragged last tile: plain guarded loads (no prefetch was issued for it)
#pragma unroll
      for (int k = 0; k < CPR; ++k) {
        const int q = lane + k * 64;
        const int row = q / CPR, cc = q % CPR;
        u32x4 t = {0u, 0u, 0u, 0u};
        if (row < nvalid) t = __builtin_nontemporal_load((const u32x4*)(xb + row * ROWB + cc * 16));
        *(u32x4*)(tile + row * ROWB + swz_chunk(row, cc, ROWB) * 16) = t;
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): the prefetch landed
    wave_lds_sync();
    uint32_t wv[R / 2];
#pragma unroll
    for (int cc = 0; cc < CPR; ++cc) {
      const u32x4 t = *(const u32x4*)(tile + lane * ROWB + swz_chunk(lane, cc, ROWB) * 16);
      wv[4 * cc] = t.x; wv[4 * cc + 1] = t.y; wv[4 * cc + 2] = t.z; wv[4 * cc + 3] = t.w;
    }
    wave_lds_sync();
    const int64_t seg = seg0 + lane;
    const int64_t vec = seg >> lgL;
    const int part = (int)(seg & (L - 1));
    const int64_t h = vec % a.heads;
    const int8_t* sg = a.signs ? a.signs + h * a.dim + part * R : nullptr;
    // per-lane signs are vector loads: apply them before the next prefetch is in flight, so
    // their wait does not include it; then store the previous tile's codes and prefetch.  The
    // signed row goes back into the tile, where the exact near-tie path reads it.
    if constexpr (LG != 0) {
      apply_signs_packed<R>(wv, sg);
#pragma unroll
      for (int cc = 0; cc < CPR; ++cc)
        *(u32x4*)(tile + lane * ROWB + swz_chunk(lane, cc, ROWB) * 16) = u32x4{wv[4 * cc], wv[4 * cc + 1], wv[4 * cc + 2], wv[4 * cc + 3]};
    }
    if (pseg0 >= 0) store_codes(pseg0, pvalid);
    if (v + G < ntiles && xcd_tile(v + G, ntiles) < full_tiles)
      load_tile_lds<ROWB>(stage_in[buf ^ 1], (const unsigned char*)a.x + xcd_tile(v + G, ntiles) * 64 * ROWB, ROWB, 64, 0, 1, lane);

    float ss = 0.f;
    if (a.nsep) {
      ss = sum_squares_in<DT, R>(wv);
      for (int o = 1; o < L; o <<= 1) ss += shfl_xor_f(ss, o);
    }
    float y[R];
    if constexpr (LG != 0) {
      stage1_unsigned<DT, R>(y, wv);
    } else {
      widen_stage1<DT, R>(y, wv, nullptr, false);
    }
    fwht_rest<R, LG>(y);
    if (a.seg_div) {                                    // RRS: the segment's smoothing divisor
      const float d = a.seg_div[part];
      const float di = d > 0.f ? 1.f / d : 0.f;
#pragma unroll
      for (int i = 0; i < R; ++i) y[i] *= di;
    }
    float m = 0.f;
    {
      float mm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < R; ++i) mm[i & 3] = fmaxf(mm[i & 3], fabsf(y[i]));
      m = fmaxf(fmaxf(mm[0], mm[1]), fmaxf(mm[2], mm[3]));
    }
    for (int o = 1; o < L; o <<= 1) m = fmaxf(m, shfl_xor_f(m, o));
    const float inv_scale = m > 0.f ? a.q / m : 0.f;

    uint32_t cw[R / 8], chm_unused[R / 32];
    const bool flagged = quantize_row<R, false>(y, [&](int) { return inv_scale; }, cw, chm_unused);
    wave_lds_sync();   // the previous tile's codes have been read out of stage_codes
#pragma unroll
    for (int cc = 0; cc < CCR; ++cc) {
      const u32x4 t = {cw[4 * cc], cw[4 * cc + 1], cw[4 * cc + 2], cw[4 * cc + 3]};
      *(u32x4*)(stage_codes + lane * CRB + swz_chunk(lane, cc, CRB) * 16) = t;
    }

    // rare path: re-decide the near-ties exactly
    const uint64_t ball = __ballot(lane < nvalid && flagged);
    if (ball) ptok_fix<DT, R, LG>(y, m, inv_scale, a.q, L, ball, tile, stage_codes, queue, a.seg_div);
    if (part == 0 && lane < nvalid) {
      const float nu = sqrtf(ss);
      const int64_t vh = head_major(a.heads, a.tokens, vec);
      if (a.nsep) a.norms[vh] = (uint16_t)f32_to_f16(nu);
      const float scale = a.nsep ? (nu > 0.f ? m * a.scale_mul / nu : 0.f) : m * a.scale_mul;
      a.scales[vh] = (uint16_t)f32_to_f16(scale);
    }
    wave_lds_sync();
    pseg0 = seg0;
    pvalid = nvalid;
  }
  if (pseg0 >= 0) store_codes(pseg0, pvalid);
}

// ---------------------------------------------------------------------------------------
// RRS runtime smoothing scales (Rotated Runtime Smooth analysis, "master equation" and
// "term-by-term": s_j = the largest |(X R)_tj| over the tokens; Figure 4: one scale per group of
// 128 channels, the group's largest).  Rows of x are [n, K] with K = L 128: a tile is 64
// consecutive 128-channel segments (lane l: segment seg0 + l, part l mod L), rotated like the
// per-token kernel does; the largest |y| of each part is reduced over the tile's lanes and
// merged into the fp32 bits of smax[part] with an integer atomic max (every value is >= 0).
template <int DT, int LG>
__global__ void __launch_bounds__(64) rrs_colmax_kernel(QuantArgs a, uint32_t* smax, int64_t nseg, int64_t ntiles,
                                                        int lgL) {
  constexpr int R = 128, ROWB = 2 * R, CPR = ROWB / 16;
  __shared__ __attribute__((aligned(16))) unsigned char tile[64 * ROWB];
  const int lane = threadIdx.x, L = 1 << lgL;
  float mpart = 0.f;                                    // this lane's part, over all its tiles
  for (int64_t v = blockIdx.x; v < ntiles; v += gridDim.x) {
    const int64_t seg0 = v * 64;
    const int nvalid = (int)(nseg - seg0 < 64 ? nseg - seg0 : 64);
    const unsigned char* xb = (const unsigned char*)a.x + seg0 * ROWB;
#pragma unroll
    for (int k = 0; k < CPR; ++k) {
      const int q = lane + k * 64;
      const int row = q / CPR, cc = q % CPR;
      u32x4 t = {0u, 0u, 0u, 0u};
      if (row < nvalid) t = __builtin_nontemporal_load((const u32x4*)(xb + row * ROWB + cc * 16));
      *(u32x4*)(tile + row * ROWB + swz_chunk(row, cc, ROWB) * 16) = t;
    }
    wave_lds_sync();
    uint32_t wv[R / 2];
#pragma unroll
    for (int cc = 0; cc < CPR; ++cc) {
      const u32x4 t = *(const u32x4*)(tile + lane * ROWB + swz_chunk(lane, cc, ROWB) * 16);
      wv[4 * cc] = t.x; wv[4 * cc + 1] = t.y; wv[4 * cc + 2] = t.z; wv[4 * cc + 3] = t.w;
    }
    wave_lds_sync();
    const int part = lane & (L - 1);
    float y[R];
    if constexpr (LG != 0) {
      apply_signs_packed<R>(wv, a.signs + part * R);
      stage1_unsigned<DT, R>(y, wv);
    } else {
      widen_stage1<DT, R>(y, wv, nullptr, false);
    }
    fwht_rest<R, LG>(y);
    float mm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < R; ++i) mm[i & 3] = fmaxf(mm[i & 3], fabsf(y[i]));
    if (lane < nvalid) mpart = fmaxf(mpart, fmaxf(fmaxf(mm[0], mm[1]), fmaxf(mm[2], mm[3])));
  }
  // lanes l and l' hold the same part when l = l' mod L
  for (int o = L; o < 64; o <<= 1) mpart = fmaxf(mpart, shfl_xor_f(mpart, o));
  if (lane < L) atomicMax(smax + lane, __builtin_bit_cast(uint32_t, mpart * a.inv_sqrt_n));
}

__global__ void __launch_bounds__(64) rrs_fill_zero(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

template <int DT, int LG> struct ColmaxK {
  static void run(const QuantArgs& a, uint32_t* smax, hipStream_t st, int64_t nseg, int lgL) {
    const int64_t ntiles = (nseg + 63) / 64;
    const int64_t grid = persistent_grid(rrs_colmax_kernel<DT, LG>, 64, ntiles);
    hipLaunchKernelGGL((rrs_colmax_kernel<DT, LG>), dim3((unsigned)grid), dim3(64), 0, st, a, smax, nseg, ntiles, lgL);
  }
};

template <int DT>
static void colmax_dt(const QuantArgs& a, uint32_t* smax, hipStream_t st, int64_t nseg, int lgL) {
  switch (a.lg_had) {
    case 0: ColmaxK<DT, 0>::run(a, smax, st, nseg, lgL); break;
    case 4: ColmaxK<DT, 4>::run(a, smax, st, nseg, lgL); break;
    case 5: ColmaxK<DT, 5>::run(a, smax, st, nseg, lgL); break;
    case 6: ColmaxK<DT, 6>::run(a, smax, st, nseg, lgL); break;
    default: ColmaxK<DT, 7>::run(a, smax, st, nseg, lgL); break;
  }
}

// the RRS smoothing scales on the matrix cores (kvq_quant_ptok.hip; smax zero-filled beforehand)
hipError_t launch_rrs_colmax_mfma(const QuantArgs& a, uint32_t* smax, hipStream_t st);

hipError_t launch_rrs_colmax(const QuantArgs& a, float* s, hipStream_t st) {
  int lgL = 0;
  while ((128 << lgL) < a.dim) ++lgL;
  const int64_t nseg = a.seqs * a.tokens * (a.dim / 128);
  uint32_t* smax = reinterpret_cast<uint32_t*>(s);
  hipLaunchKernelGGL(rrs_fill_zero, dim3(1), dim3(64), 0, st, smax, (int)(a.dim / 128));
  if (nseg > 0) {
    if (!rotation_butterfly()) return launch_rrs_colmax_mfma(a, smax, st);   // the matrix-core kernel
    if (a.dtype == DT_F16) colmax_dt<DT_F16>(a, smax, st, nseg, lgL); else colmax_dt<DT_BF16>(a, smax, st, nseg, lgL);
  }
  return hipGetLastError();
}

template <int DT, int R, int LG>
static void launch_ptok_k(const QuantArgs& a, hipStream_t st, int64_t nseg, int lgL) {
  const int64_t ntiles = (nseg + 63) / 64;
  const int64_t grid = persistent_grid(quant_ptok_kernel<DT, R, LG>, 64, ntiles);
  hipLaunchKernelGGL((quant_ptok_kernel<DT, R, LG>), dim3((unsigned)grid), dim3(64), 0, st, a, nseg, ntiles, lgL);
}

// compile-time Hadamard size: LG = log2(n) in {0 (none), 4, 5, 6, 7}
template <int DT, int R, template <int, int, int> class K, typename... Args>
static void by_lg(int lg, Args&&... args) {
  switch (lg) {
    case 0: K<DT, R, 0>::run(args...); break;
    case 4: K<DT, R, 4>::run(args...); break;
    case 5: K<DT, R, 5>::run(args...); break;
    case 6: K<DT, R, 6>::run(args...); break;
    default: if constexpr (R >= 128) K<DT, R, 7>::run(args...); break;
  }
}
template <int DT, int R, int LG> struct PtokK {
  static void run(const QuantArgs& a, hipStream_t st, int64_t nseg, int lgL) { launch_ptok_k<DT, R, LG>(a, st, nseg, lgL); }
};

template <int DT>
static void ptok_dt(const QuantArgs& a, hipStream_t st) {
  const int R = a.dim >= 128 ? 128 : 64;
  int lgL = 0;
  while ((R << lgL) < a.dim) ++lgL;
  const int64_t nseg = a.seqs * a.tokens * a.heads * (a.dim / R);
  if (R == 128) by_lg<DT, 128, PtokK>(a.lg_had, a, st, nseg, lgL);
  else by_lg<DT, 64, PtokK>(a.lg_had, a, st, nseg, lgL);
}

hipError_t launch_quantize_ptok(const QuantArgs& a, hipStream_t st) {
  if (a.dim >= 128 && !rotation_butterfly()) return launch_quantize_ptok_mfma(a, st);
  if (a.dtype == DT_F16) ptok_dt<DT_F16>(a, st); else ptok_dt<DT_BF16>(a, st);
  return hipGetLastError();
}

}  // namespace kvq
