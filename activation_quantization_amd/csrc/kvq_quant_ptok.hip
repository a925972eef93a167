// Per-token quantize (NAIVE, NSEP, and the RRS activation and weight quantizers) for gfx950, with
// the rotation on the matrix cores.
//
// Method sources (page title, section): norm-separation post "the fix" (fp16 L2 norm + unit
// direction; absmax / Q, round, clamp) and "root cause" (per-row absmax); Rotated Runtime Smooth
// analysis "problem definition" (alpha = max|X| / (2^(N-1)-1)), "master equation" (the smoothed
// activations X R diag(s)^-1 are quantized) and "term-by-term" (R = (1/sqrt K)[+-1]); NSNQuant
// summary "Hadamard transform" (random signs, then the Hadamard matrix).
//
// Work split: x is [rows, heads, D] with D = L * 128, so the (token, head) vectors are runs of L
// consecutive 128-channel rows and the rows of all vectors follow each other in memory.  A tile is
// 128 consecutive rows (128 / L whole vectors, 32 KiB contiguous), one tile per workgroup of four
// waves.  The rows stream into LDS (global_load_lds, 1 KiB per wave instruction, XOR-swizzled
// chunks); each wave flips the sign bits of the rows it loaded in place with the random signs of
// their channels (signs vary from row to row, so they cannot be folded into the Hadamard operand);
// then wave w computes output channels [32 w, 32 w + 32) of every row on the matrix cores with the
// layout of kvq_rotate.h (lane 16 g + j of sub-tile s holds channels 32 w + 8 g + [0, 8) of row
// 16 s + j).  The transform is left unnormalized: 1/sqrt(n) cancels in the quotient (and, per
// token, so does the norm: the code is rne(Q Y_c / max |Y|)) and only enters the stored scale.
//
// Per-token max: each lane's max over its 8 channels of a row, then over the vector's rows (its
// sub-tiles in the lane, its lanes by DPP and lane permutes), then over the four waves through
// LDS.  Codes by one fma per value against a magic constant (byte 2 of the result is the code + 8,
// its low 16 bits flag values within 2^-17 of a tie), packed into the tile's code rows in LDS and
// stored in 16-byte pieces.  Vectors that hold a flagged value take the exact path: the waves find
// the channels whose fp32 magnitude is within 2^-12 of the vector's fp32 max (the only ones that
// can hold the exact max), compute them exactly in fp64 from the staged rows and merge the exact max
// with an LDS integer max on its bits; the flagged values are then re-decided as rne(Q Y / max|Y|)
// of the fp64 values (one correctly rounded division of exact sums, so an exact tie stays a tie).
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_launch.h"
#include "kvq_rotate.h"

namespace kvq {
namespace {

using namespace rot;

constexpr int PT_ROWS = 64;    // rows per tile (16 per wave; a vector of at most 64 rows fits)
constexpr float PT_MAGIC = 136.5f;

template <int CTL> __device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTL, 0xF, 0xF, false);
}

// max of non-negative floats (compared as their bits) over aligned groups of 2^lg lanes of each
// 16-lane row; lg <= 4 is wave-uniform
__device__ __forceinline__ uint32_t group_max(uint32_t v, int lg) {
  if (lg >= 1) v = umax(v, dpp<0xB1>(v));    // quad_perm [1, 0, 3, 2]
  if (lg >= 2) v = umax(v, dpp<0x4E>(v));    // quad_perm [2, 3, 0, 1]
  if (lg >= 3) v = umax(v, dpp<0x141>(v));   // row_half_mirror
  if (lg >= 4) v = umax(v, dpp<0x140>(v));   // row_mirror
  return v;
}
__device__ __forceinline__ float group_sum(float v, int lg) {
  auto d = [](float x, auto ctl) {
    return __builtin_bit_cast(float, dpp<decltype(ctl)::value>(__builtin_bit_cast(uint32_t, x)));
  };
  if (lg >= 1) v += d(v, std::integral_constant<int, 0xB1>{});
  if (lg >= 2) v += d(v, std::integral_constant<int, 0x4E>{});
  if (lg >= 3) v += d(v, std::integral_constant<int, 0x141>{});
  if (lg >= 4) v += d(v, std::integral_constant<int, 0x140>{});
  return v;
}

// LGLT: log2 of the 128-channel rows per vector when fixed at compile time (0: head_dim 128, 5: head_dim
// 4096), so the row -> vector arithmetic and the reductions' shapes fold; -1 takes lgL_arg at run time
template <int DT, int LG, bool RRS, int LGLT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
quant_ptok_tile(QuantArgs a, int64_t nrows, int64_t ntiles, int lgL_arg) {
  const int lgL = LGLT >= 0 ? LGLT : lgL_arg;
  constexpr int R = 128, NK = 4, NIW = 2, LCH = 8, ST = PT_ROWS / 16, ROWB = 2 * R, CPR = ROWB / 16, RB = R / 2;
  constexpr int WSTAGE = PT_ROWS / 4 * ROWB;                 // bytes of the rows each wave loads
  constexpr int NLD = WSTAGE / 1024;                          // load instructions per wave
  __shared__ __attribute__((aligned(16))) unsigned char stage[PT_ROWS * ROWB];   // the tile's rows (signed)
  __shared__ __attribute__((aligned(16))) unsigned char cstage[PT_ROWS * RB];    // the tile's code rows
  __shared__ __attribute__((aligned(16))) uint32_t pmax[PT_ROWS][4];            // per (vector, wave) max bits
  __shared__ __attribute__((aligned(16))) float psum[PT_ROWS][4];              // per vector partial sums of squares
  __shared__ uint32_t vflag[PT_ROWS / 32];                                      // vectors holding a near-tie
  __shared__ uint64_t xmax[PT_ROWS];                                            // their exact max (fp64 bits)
  __shared__ float dinv_s[64];                                                  // RRS: 1 / smoothing scale per segment

  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t row0 = tile * PT_ROWS;
  const int nvalid = (int)(nrows - row0 < PT_ROWS ? nrows - row0 : PT_ROWS);
  const int L = 1 << lgL;
  const int lgJ = lgL < 4 ? lgL : 4;            // log2 rows of one vector inside a sub-tile
  const int lgS = lgL > 4 ? lgL - 4 : 0;        // log2 sub-tiles one vector spans
  if (tid < PT_ROWS / 32) vflag[tid] = 0u;
  if (tid < PT_ROWS) {
    xmax[tid] = 0ull;
    *(f32x4*)psum[tid] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // 1. this wave's 32 rows into LDS: instruction k moves rows 32 w + 4 k + g, lane slot j holding
  //    global chunk j ^ (row % 16); the sign bytes of those chunks come along into registers
  const unsigned char* xw = (const unsigned char*)a.x + (row0 + (PT_ROWS / 4) * w) * ROWB;
  // head of the tile's first vector (vectors are (token, head) pairs, head fastest)
  const uint32_t h0 = a.heads > 1 ? (uint32_t)((row0 >> lgL) % a.heads) : 0u;
  u32x2 sgn[NLD];
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const int r = (PT_ROWS / 4) * w + 4 * k + g;            // tile row
    const int gc = j ^ (r % CPR);
    if (r < nvalid) {
      __builtin_amdgcn_global_load_lds((const void*)(xw + (4 * k + g) * ROWB + 16 * gc),
                                       (__attribute__((address_space(3))) void*)(stage + w * WSTAGE + k * 1024), 16, 0,
                                       KVQ_LOAD_NT);
      if constexpr (LG != 0) {
        const uint32_t h = a.heads > 1 ? (h0 + ((uint32_t)r >> lgL)) % (uint32_t)a.heads : 0u;
        sgn[k] = *(const u32x2*)(a.signs + (int64_t)h * a.dim + (r & (L - 1)) * R + 8 * gc);
      }
    }
  }
  // RRS: the inverse smoothing divisor of every segment (row 16 s + j is segment (16 s + j) mod L)
  if constexpr (RRS) {
    if (tid < L) {
      const float d = a.seg_div[tid];
      dinv_s[tid] = d > 0.f ? 1.f / d : 0.f;
    }
  }
  u32x4 fb[NIW];
  if constexpr (LG != 0) {
#pragma unroll
    for (int I = 0; I < NIW; ++I) fb[I] = fragment_load<DT, R, LG>(w, I, lane);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this wave's rows and sign bytes have landed
  asm volatile("" ::: "memory");

  // 2. sign bits of this wave's own rows, in place (sign byte k of a pair goes to bit 15 / 31); rows
  //    past the end of x are zero
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const int r = (PT_ROWS / 4) * w + 4 * k + g;
    u32x4* p = (u32x4*)(stage + w * WSTAGE + k * 1024 + 16 * lane);
    if (r < nvalid) {
      if constexpr (LG != 0) {
        u32x4 d = *p;
        d.x ^= __builtin_amdgcn_perm(0u, sgn[k].x, 0x010C000Cu) & 0x80008000u;
        d.y ^= __builtin_amdgcn_perm(0u, sgn[k].x, 0x030C020Cu) & 0x80008000u;
        d.z ^= __builtin_amdgcn_perm(0u, sgn[k].y, 0x010C000Cu) & 0x80008000u;
        d.w ^= __builtin_amdgcn_perm(0u, sgn[k].y, 0x030C020Cu) & 0x80008000u;
        *p = d;
      }
    } else {
      *p = u32x4{0u, 0u, 0u, 0u};
    }
  }
  lds_barrier();

  // operand chunks of row 16 s + j for K step K: channels 32 K + 8 g + [0, 8)
  auto read_x = [&](int s, int K) {
    return *(const u32x4*)(stage + 16 * s * ROWB + (j * ROWB + 16 * ((4 * K + g) ^ (j % CPR))));
  };

  // 3. NSEP: sums of squares of this wave's own rows (its SW sub-tiles) from the diagonal of the Gram
  //    matrix, summed over each vector's rows.  A vector of at most 16 rows lies in one sub-tile; a
  //    longer one covers whole waves' rows (or a whole wave covers it), and each of its waves adds
  //    one partial (slot w mod partials).
  if (a.nsep) {
    constexpr int SW = ST / 4;                                // sub-tiles per wave
    float tot = 0.f;
#pragma unroll
    for (int o = 0; o < SW; ++o) {
      const int s = SW * w + o;
      u32x4 x[NK];
#pragma unroll
      for (int K = 0; K < NK; ++K) x[K] = read_x(s, K);
      f32x4 gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < NK; ++K) gm = mfma16<DT>(x[K], x[K], gm);
      const float d01 = (j & 1) ? gm.y : gm.x, d23 = (j & 1) ? gm.w : gm.z;
      const float dg = (j & 2) ? d23 : d01;
      float ssq = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((j + 16 * (j >> 2)) << 2,
                                                                         __builtin_bit_cast(int, dg)));
      ssq = group_sum(ssq, lgJ);
      if (lgS == 0) {
        if (lane < 16 && (j & (L - 1)) == 0) psum[(16 * s + j) >> lgL][0] = ssq;
      } else {
        tot += ssq;
      }
    }
    if (lgS >= 1 && lane == 0) {
      const int np = (L >> 4) / SW > 1 ? (L >> 4) / SW : 1;   // partials per vector
      psum[(16 * SW * w) >> lgL][w & (np - 1)] = tot;
    }
  }

  // 4. the rotation of this wave's channels, sub-tile by sub-tile.  The block sign beta(w, K) is a
  //    wave-uniform mask (0 outside the diagonal blocks: that K step is skipped), so one code path
  //    serves every wave.
  f32x4 u[ST][NIW];
  {
    u32x4 fk[NK][NIW];
    if constexpr (LG != 0) {
#pragma unroll
      for (int K = 0; K < NK; ++K) {
        const uint32_t neg = blk_beta<LG>(w, K) < 0 ? 0x80008000u : 0u;
#pragma unroll
        for (int I = 0; I < NIW; ++I) fk[K][I] = fb[I] ^ neg;
      }
    }
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      if constexpr (LG == 0) {
        const u32x4 xr = read_x(s, w);                       // the lane's own 8 channels
        const uint32_t xw4[4] = {xr.x, xr.y, xr.z, xr.w};
#pragma unroll
        for (int I = 0; I < NIW; ++I)
          u[s][I] = f32x4{lo_f32<DT>(xw4[2 * I]), hi_f32<DT>(xw4[2 * I]), lo_f32<DT>(xw4[2 * I + 1]),
                          hi_f32<DT>(xw4[2 * I + 1])};
      } else {
        u32x4 x[NK];
#pragma unroll
        for (int K = 0; K < NK; ++K) x[K] = read_x(s, K);
#pragma unroll
        for (int I = 0; I < NIW; ++I) u[s][I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < NK; ++K) {
          if (blk_beta<LG>(w, K) == 0) continue;             // wave-uniform
#pragma unroll
          for (int I = 0; I < NIW; ++I) u[s][I] = mfma16<DT>(fk[K][I], x[K], u[s][I]);
        }
      }
      if constexpr (RRS) {
        const float di = dinv_s[(16 * s + j) & (L - 1)];
#pragma unroll
        for (int I = 0; I < NIW; ++I) u[s][I] *= di;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // 5. per-token max: in the lane, over the vector's sub-tiles, its lanes, then the four waves
  uint32_t ms[ST];
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    const float m0 = __builtin_fmaxf(fmaxf(fabsf(u[s][0].x), fabsf(u[s][0].y)), fabsf(u[s][0].z));
    const float m1 = __builtin_fmaxf(fmaxf(fabsf(u[s][0].w), fabsf(u[s][1].x)), fabsf(u[s][1].y));
    const float m2 = __builtin_fmaxf(fmaxf(fabsf(u[s][1].z), fabsf(u[s][1].w)), m0);
    ms[s] = __builtin_bit_cast(uint32_t, fmaxf(m1, m2));
  }
  // a vector spanning 2^lgS sub-tiles: merge them (branch-free selects on a wave-uniform condition)
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    const uint32_t p = umax(ms[s], ms[s ^ 1]);
    ms[s] = lgS >= 1 ? p : ms[s];
  }
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    const uint32_t p = umax(ms[s], ms[s ^ 2]);
    ms[s] = lgS >= 2 ? p : ms[s];
  }
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    uint32_t m = ms[s];
    m = umax(m, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, (int)m));
    m = umax(m, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)m));
    m = group_max(m, lgJ);
    if (lane < 16 && (j & ((1 << lgJ) - 1)) == 0 && (s & ((1 << lgS) - 1)) == 0) pmax[(16 * s + j) >> lgL][w] = m;
  }
  lds_barrier();

  // 6. each row's vector max and inverse scale
  float iv[ST];
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    const u32x4 p = *(const u32x4*)pmax[(16 * s + j) >> lgL];
    const float m = __builtin_bit_cast(float, umax(umax(p.x, p.y), umax(p.z, p.w)));
    iv[s] = m > 0.f ? a.q * __builtin_amdgcn_rcpf(m) : 0.f;
  }
  // the stored scale (and norm) of vector tid
  if (tid < (PT_ROWS >> lgL) && (tid << lgL) < nvalid) {
    const u32x4 p = *(const u32x4*)pmax[tid];
    const float m = __builtin_bit_cast(float, umax(umax(p.x, p.y), umax(p.z, p.w)));
    const int64_t vh = head_major(a.heads, a.tokens, (row0 >> lgL) + tid);
    float scale = m * a.scale_mul;
    if (a.nsep) {
      const f32x4 ps = *(const f32x4*)psum[tid];
      const float nu = sqrtf((ps.x + ps.y) + (ps.z + ps.w));
      a.norms[vh] = (uint16_t)f32_to_f16(nu);
      scale = nu > 0.f ? scale / nu : 0.f;
    }
    a.scales[vh] = (uint16_t)f32_to_f16(scale);
  }

  // 7. codes and near-tie flags -> the code rows (row 16 s + j, bytes 16 w + 4 g ..)
  uint32_t pk[ST], flagged = 0u;
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    uint32_t b[8];
#pragma unroll
    for (int q = 0; q < LCH; ++q) b[q] = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[s][q >> 2][q & 3], iv[s], PT_MAGIC));
    uint32_t fl = min3_u16(0xffffu, b[0], b[1]);
    fl = min3_u16(fl, b[2], b[3]);
    fl = min3_u16(fl, b[4], b[5]);
    fl = min3_u16(fl, b[6], b[7]);
    flagged |= ((fl & 0xffffu) == 0u && 16 * s + j < nvalid ? 1u : 0u) << s;
    pk[s] = pack8(b);
    *(uint32_t*)(cstage + (16 * s + j) * RB + 16 * w + 4 * g) = pk[s];
  }
  // vectors holding a flagged value -> vflag (rare)
  if (__ballot(flagged != 0u) != 0ull) {
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      if ((flagged >> s) & 1u) {
        const int v = (16 * s + j) >> lgL;
        atomicOr(&vflag[v >> 5], 1u << (v & 31));
      }
    }
  }
  lds_barrier();

  constexpr int NVW = PT_ROWS / 32;                          // flag words (one bit per vector)
  uint32_t vfw[NVW], vany = 0u;
#pragma unroll
  for (int k = 0; k < NVW; ++k) {
    vfw[k] = vflag[k];
    vany |= vfw[k];
  }
  if (vany != 0u) {
    // the rare path recomputes its row -> vector indices from an opaque copy of the shift, so the
    // main path does not keep them live for it
    int lgLr;
    asm volatile("s_mov_b32 %0, %1" : "=s"(lgLr) : "s"(lgL));
    // 8. rare path.  Exact fp64 value of channel c of tile row r (signed rows in LDS; lane l takes
    //    inputs l and l + 64), divided by the row's smoothing scale for RRS
    auto exact_y = [&](int r, int c) {
      double y = 0.0;
#pragma unroll
      for (int e = 0; e < R / 64; ++e) {
        const int p = lane + 64 * e;
        const uint32_t hw = *(const uint16_t*)(stage + r * ROWB + 16 * ((p >> 3) ^ (r % CPR)) + 2 * (p & 7));
        const double xv = widen64<DT>(hw);
        const int hv = LG == 0 ? (p == c ? 1 : 0) : hval<LG>(c, p);
        if (hv != 0) y += hv < 0 ? -xv : xv;
      }
      y = wave_sum64(y);
      if constexpr (RRS) {
        const float d = a.seg_div[r & ((1 << lgLr) - 1)];
        y = d > 0.f ? y / (double)d : 0.0;
      }
      return y;
    };
    auto vflagged = [&](int v) {
      uint32_t wd = vfw[0];
#pragma unroll
      for (int k = 1; k < NVW; ++k) wd = (v >> 5) == k ? vfw[k] : wd;
      return ((wd >> (v & 31)) & 1u) != 0u;
    };
    // Sub-tile by sub-tile, the rotated values are computed again (so the main path need not keep
    // them), and slot 8 s + q of a lane (its channel 32 w + 8 g + q of row 16 s + j) goes into fmask
    // when it is flagged; the slots of flagged vectors within 2^-12 of the vector's fp32 max (the
    // candidates for its exact max) are computed exactly and merged into xmax.
    int wr;
    asm volatile("s_mov_b32 %0, %1" : "=s"(wr) : "s"(w));
    u32x4 fkr[NK][NIW];
    if constexpr (LG != 0) {
      int op = 0;                                           // opaque zero: a fresh load, not the common path's
      asm volatile("" : "+v"(op));
#pragma unroll
      for (int I = 0; I < NIW; ++I) {
        const u32x4 f = fragment_load<DT, R, LG>(wr, I, lane + op);
#pragma unroll
        for (int K = 0; K < NK; ++K) fkr[K][I] = f ^ (blk_beta<LG>(wr, K) < 0 ? 0x80008000u : 0u);
      }
    }
    uint64_t fmask = 0ull;
#pragma unroll 1
    for (int s = 0; s < ST; ++s) {
      f32x4 us[NIW];
      if constexpr (LG == 0) {
        const u32x4 xr = read_x(s, wr);
        us[0] = f32x4{lo_f32<DT>(xr.x), hi_f32<DT>(xr.x), lo_f32<DT>(xr.y), hi_f32<DT>(xr.y)};
        us[1] = f32x4{lo_f32<DT>(xr.z), hi_f32<DT>(xr.z), lo_f32<DT>(xr.w), hi_f32<DT>(xr.w)};
      } else {
        u32x4 x[NK];
#pragma unroll
        for (int K = 0; K < NK; ++K) x[K] = read_x(s, K);
        us[0] = us[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < NK; ++K) {
          if (blk_beta<LG>(wr, K) == 0) continue;
#pragma unroll
          for (int I = 0; I < NIW; ++I) us[I] = mfma16<DT>(fkr[K][I], x[K], us[I]);
        }
      }
      if constexpr (RRS) {
        const float di = dinv_s[(16 * s + j) & ((1 << lgLr) - 1)];
        us[0] *= di;
        us[1] *= di;
      }
      const int v = (16 * s + j) >> lgLr;
      const u32x4 p = *(const u32x4*)pmax[v];
      const float m = __builtin_bit_cast(float, umax(umax(p.x, p.y), umax(p.z, p.w)));
      const float ivs = m > 0.f ? a.q * __builtin_amdgcn_rcpf(m) : 0.f;
      const float thr = m * (1.f - 0x1p-12f);
      const bool rowf = vflagged(v) && 16 * s + j < nvalid;
      const bool rowflag = ((flagged >> s) & 1u) != 0u;
      uint32_t cm = 0u;
#pragma unroll
      for (int q = 0; q < LCH; ++q) {
        const float uq = us[q >> 2][q & 3];
        const bool f = rowflag && (__builtin_bit_cast(uint32_t, __builtin_fmaf(uq, ivs, PT_MAGIC)) & 0xffffu) == 0u;
        fmask |= (uint64_t)(f ? 1u : 0u) << (8 * s + q);
        cm |= (rowf && fabsf(uq) >= thr ? 1u : 0u) << q;
      }
      if (__ballot(cm != 0u) == 0ull) continue;
#pragma unroll 1
      for (int q = 0; q < LCH; ++q) {
        for (uint64_t cb = __ballot((cm >> q) & 1u); cb; cb &= cb - 1ull) {
          const int l = __builtin_ctzll(cb);
          const int r = 16 * s + (l & 15);
          const double y = fabs(exact_y(r, 32 * wr + 8 * (l >> 4) + q));
          if (lane == l) atomicMax((unsigned long long*)&xmax[r >> lgLr], (unsigned long long)__builtin_bit_cast(uint64_t, y));
        }
      }
    }
    lds_barrier();
    // (b) the flagged values, decided from the exact quotient
    const double qd = (double)a.q;
#pragma unroll 1
    for (int sl = 0; sl < 8 * ST; ++sl) {
      for (uint64_t fb2 = __ballot((fmask >> sl) & 1ull); fb2; fb2 &= fb2 - 1ull) {
        const int l = __builtin_ctzll(fb2);
        const int r = 16 * (sl >> 3) + (l & 15);
        const double y = exact_y(r, 32 * wr + 8 * (l >> 4) + (sl & 7));
        if (lane == l) {
          const double xm = __builtin_bit_cast(double, xmax[r >> lgLr]);
          const uint32_t nib = xm > 0.0 ? exact_nibble(qd * y / xm) : 0u;
          const int q = sl & 7;
          unsigned char* cp = cstage + r * RB + 16 * wr + 4 * g + (q >> 1);
          const uint32_t sh = 4 * (q & 1);
          *cp = (unsigned char)((*cp & ~(0xFu << sh)) | (nib << sh));
        }
      }
    }
    lds_barrier();
  }

  // 9. the code rows out in 16-byte pieces: with one head they are one contiguous block
  if (a.heads == 1) {
    unsigned char* cb = a.codes + (row0 + (PT_ROWS / 4) * w) * RB;
#pragma unroll
    for (int k = 0; k < PT_ROWS / 64; ++k) {
      const int pc = 64 * k + lane;                          // piece of this wave's rows
      if ((PT_ROWS / 4) * w + pc / 4 < nvalid)
        __builtin_nontemporal_store(*(const u32x4*)(cstage + (PT_ROWS / 4) * w * RB + 16 * pc), (u32x4*)(cb + 16 * pc));
    }
  } else {
    const int r = (PT_ROWS / 4) * w + (lane >> 1);          // two lanes per row
    if ((lane >> 1) < PT_ROWS / 4 && r < nvalid) {
      const int64_t rabs = row0 + r;
      const int64_t dst = (head_major(a.heads, a.tokens, rabs >> lgL) << lgL) + (rabs & (L - 1));
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int piece = 2 * (lane & 1) + k;
        __builtin_nontemporal_store(*(const u32x4*)(cstage + r * RB + 16 * piece), (u32x4*)(a.codes + dst * RB + 16 * piece));
      }
    }
  }
}

// this wave's rows of tile t into the stage st (the per-token kernel's swizzled layout), the sign
// bytes of their chunks into sg
template <int LG>
__device__ __forceinline__ void colmax_issue(const QuantArgs& a, unsigned char* st, int64_t t, int64_t nrows, int L, int w,
                                             int lane, u32x2 (&sg)[PT_ROWS * 256 / 4 / 1024]) {
  constexpr int R = 128, ROWB = 2 * R, CPR = ROWB / 16, WSTAGE = PT_ROWS / 4 * ROWB, NLD = WSTAGE / 1024;
  const int j = lane & 15, g = lane >> 4;
  const int64_t row0 = t * PT_ROWS;
  const int nvalid = (int)(nrows - row0 < PT_ROWS ? nrows - row0 : PT_ROWS);
  const unsigned char* xw = (const unsigned char*)a.x + (row0 + (PT_ROWS / 4) * w) * ROWB;
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const int r = (PT_ROWS / 4) * w + 4 * k + g;
    const int gc = j ^ (r % CPR);
    if (r < nvalid) {
      __builtin_amdgcn_global_load_lds((const void*)(xw + (4 * k + g) * ROWB + 16 * gc),
                                       (__attribute__((address_space(3))) void*)(st + w * WSTAGE + k * 1024), 16, 0,
                                       KVQ_LOAD_NT);
      if constexpr (LG != 0) sg[k] = *(const u32x2*)(a.signs + (r & (L - 1)) * R + 8 * gc);
    }
  }
}

// RRS smoothing scales on the matrix cores: s[g] = (1/sqrt n) max |H sigma x| over every row of
// segment g (rows are the 128-channel segments of the [n, k] input, row r in segment r mod L).
// Resident workgroups of four waves walk the 64-row tiles b, b + G, ...; each tile is copied into
// one of two LDS stages while the previous one is rotated (the per-token kernel's layout: signs
// flipped in place by the wave that loaded the rows, wave w rotating output channels
// [32 w, 32 w + 32) of every row), and each lane keeps the max of its 8 channels per tile row
// position.  At the end the positions are merged over the lane groups, the waves and the rows of
// each segment (tiles start at multiples of 64 and L divides 64, so position r is segment r mod L),
// and each segment's max enters s with an integer max on its float bits (non-negative values), skipped
// when the value already there is not smaller.
template <int DT, int LG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
rrs_colmax_tile(QuantArgs a, uint32_t* smax, int64_t nrows, int64_t ntiles, int lgL) {
  constexpr int R = 128, NK = 4, NIW = 2, ST = PT_ROWS / 16, ROWB = 2 * R, CPR = ROWB / 16;
  constexpr int WSTAGE = PT_ROWS / 4 * ROWB;                 // bytes of the rows each wave loads
  constexpr int NLD = WSTAGE / 1024;                          // load instructions per wave
  __shared__ __attribute__((aligned(16))) unsigned char stage[2][PT_ROWS * ROWB];
  __shared__ __attribute__((aligned(16))) uint32_t rmax[PT_ROWS][4];   // per (row position, wave) max bits
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = 1 << lgL;
  const int64_t G = gridDim.x;

  u32x4 fk[NK][NIW];
  if constexpr (LG != 0) {
#pragma unroll
    for (int I = 0; I < NIW; ++I) {
      const u32x4 f = fragment_load<DT, R, LG>(w, I, lane);
#pragma unroll
      for (int K = 0; K < NK; ++K) fk[K][I] = f ^ (blk_beta<LG>(w, K) < 0 ? 0x80008000u : 0u);
    }
  }
  uint32_t acc[ST];
#pragma unroll
  for (int s = 0; s < ST; ++s) acc[s] = 0u;

  u32x2 sgn[NLD], sgn_next[NLD];
  int b = 0;
  int64_t t = blockIdx.x;
  if (t < ntiles) colmax_issue<LG>(a, stage[0], t, nrows, L, w, lane, sgn);
  for (; t < ntiles; t += G) {
    const int nvalid = (int)(nrows - t * PT_ROWS < PT_ROWS ? nrows - t * PT_ROWS : PT_ROWS);
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this tile's rows and sign bytes (no stores in flight)
    asm volatile("" ::: "memory");
    // sign bits of this wave's own rows, in place; rows past the end are zero
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int r = (PT_ROWS / 4) * w + 4 * k + g;
      u32x4* p = (u32x4*)(stage[b] + w * WSTAGE + k * 1024 + 16 * lane);
      if (r < nvalid) {
        if constexpr (LG != 0) {
          u32x4 d = *p;
          d.x ^= __builtin_amdgcn_perm(0u, sgn[k].x, 0x010C000Cu) & 0x80008000u;
          d.y ^= __builtin_amdgcn_perm(0u, sgn[k].x, 0x030C020Cu) & 0x80008000u;
          d.z ^= __builtin_amdgcn_perm(0u, sgn[k].y, 0x010C000Cu) & 0x80008000u;
          d.w ^= __builtin_amdgcn_perm(0u, sgn[k].y, 0x030C020Cu) & 0x80008000u;
          *p = d;
        }
      } else {
        *p = u32x4{0u, 0u, 0u, 0u};
      }
    }
    lds_barrier();   // every wave's rows are in stage b, and every wave is done with stage b ^ 1
    if (t + G < ntiles) colmax_issue<LG>(a, stage[b ^ 1], t + G, nrows, L, w, lane, sgn_next);
    const unsigned char* sb = stage[b];
    auto read_x = [&](int s, int K) {
      return *(const u32x4*)(sb + 16 * s * ROWB + (j * ROWB + 16 * ((4 * K + g) ^ (j % CPR))));
    };
#pragma unroll
    for (int s = 0; s < ST; ++s) {
      f32x4 u[NIW];
      if constexpr (LG == 0) {
        const u32x4 xr = read_x(s, w);                       // the lane's own 8 channels
        u[0] = f32x4{lo_f32<DT>(xr.x), hi_f32<DT>(xr.x), lo_f32<DT>(xr.y), hi_f32<DT>(xr.y)};
        u[1] = f32x4{lo_f32<DT>(xr.z), hi_f32<DT>(xr.z), lo_f32<DT>(xr.w), hi_f32<DT>(xr.w)};
      } else {
        u32x4 x[NK];
#pragma unroll
        for (int K = 0; K < NK; ++K) x[K] = read_x(s, K);
        u[0] = u[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < NK; ++K) {
          if (blk_beta<LG>(w, K) == 0) continue;             // wave-uniform
#pragma unroll
          for (int I = 0; I < NIW; ++I) u[I] = mfma16<DT>(fk[K][I], x[K], u[I]);
        }
      }
      const float m0 = __builtin_fmaxf(fmaxf(fabsf(u[0].x), fabsf(u[0].y)), fabsf(u[0].z));
      const float m1 = __builtin_fmaxf(fmaxf(fabsf(u[0].w), fabsf(u[1].x)), fabsf(u[1].y));
      const float m2 = __builtin_fmaxf(fmaxf(fabsf(u[1].z), fabsf(u[1].w)), m0);
      acc[s] = umax(acc[s], __builtin_bit_cast(uint32_t, fmaxf(m1, m2)));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k = 0; k < NLD; ++k) sgn[k] = sgn_next[k];
    b ^= 1;
  }
  // position 16 s + j: over the lane groups, then the waves, then the positions of each segment
#pragma unroll
  for (int s = 0; s < ST; ++s) {
    uint32_t m = acc[s];
    m = umax(m, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, (int)m));
    m = umax(m, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)m));
    if (lane < 16) rmax[16 * s + j][w] = m;
  }
  lds_barrier();
  if (w == 0) {
    const u32x4 p = *(const u32x4*)rmax[lane];
    float m = __builtin_bit_cast(float, umax(umax(p.x, p.y), umax(p.z, p.w)));
    for (int o = L; o < 64; o <<= 1) m = fmaxf(m, shfl_xor_f(m, o));
    // the maxima only grow, so a value not above the one already there (read without ordering: a
    // stale read is at most the current value, and then the atomic is merely not skipped) needs no
    // atomic; the workgroups' atomics on this one line would otherwise serialize
    const uint32_t mb = __builtin_bit_cast(uint32_t, m * a.inv_sqrt_n);
    if (lane < L && mb > ld_global(smax + lane)) atomicMax(smax + lane, mb);
  }
}

template <int DT, int LG>
void launch_colmax(const QuantArgs& a, uint32_t* smax, hipStream_t st, int64_t nrows, int lgL) {
  const int64_t ntiles = (nrows + PT_ROWS - 1) / PT_ROWS;
  const int64_t grid = persistent_grid(rrs_colmax_tile<DT, LG>, 256, ntiles);
  hipLaunchKernelGGL((rrs_colmax_tile<DT, LG>), dim3((unsigned)grid), dim3(256), 0, st, a, smax, nrows, ntiles, lgL);
}

template <int DT, int LG, bool RRS>
void launch_t(const QuantArgs& a, hipStream_t st, int64_t nrows, int lgL) {
  const int64_t ntiles = (nrows + PT_ROWS - 1) / PT_ROWS;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3((unsigned)ntiles), dim3(256), 0, st, a, nrows, ntiles, lgL); };
  if (lgL == 5) go(quant_ptok_tile<DT, LG, RRS, 5>);
  else if (lgL == 0) go(quant_ptok_tile<DT, LG, RRS, 0>);
  else go(quant_ptok_tile<DT, LG, RRS, -1>);
}

template <int DT, bool RRS>
void launch_lg(const QuantArgs& a, hipStream_t st, int64_t nrows, int lgL) {
  switch (a.lg_had) {
    case 0: launch_t<DT, 0, RRS>(a, st, nrows, lgL); break;
    case 4: launch_t<DT, 4, RRS>(a, st, nrows, lgL); break;
    case 5: launch_t<DT, 5, RRS>(a, st, nrows, lgL); break;
    case 6: launch_t<DT, 6, RRS>(a, st, nrows, lgL); break;
    default: launch_t<DT, 7, RRS>(a, st, nrows, lgL); break;
  }
}

}  // namespace

// the RRS smoothing scales (s zero-filled by the caller): rows of 128 channels, k a power of two in
// [128, 8192]
hipError_t launch_rrs_colmax_mfma(const QuantArgs& a, uint32_t* smax, hipStream_t st) {
  int lgL = 0;
  while ((int64_t(128) << lgL) < a.dim) ++lgL;
  if ((1 << lgL) > PT_ROWS) return hipErrorInvalidValue;   // segments must divide the tile
  const int64_t nrows = a.seqs * a.tokens * a.heads * (a.dim / 128);
  if (nrows == 0) return hipGetLastError();
  auto by_lg = [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    switch (a.lg_had) {
      case 0: launch_colmax<DT, 0>(a, smax, st, nrows, lgL); break;
      case 4: launch_colmax<DT, 4>(a, smax, st, nrows, lgL); break;
      case 5: launch_colmax<DT, 5>(a, smax, st, nrows, lgL); break;
      case 6: launch_colmax<DT, 6>(a, smax, st, nrows, lgL); break;
      default: launch_colmax<DT, 7>(a, smax, st, nrows, lgL); break;
    }
  };
  if (a.dtype == DT_F16) by_lg(std::integral_constant<int, DT_F16>{});
  else by_lg(std::integral_constant<int, DT_BF16>{});
  return hipGetLastError();
}

// head_dim a power of two in [128, 8192]
hipError_t launch_quantize_ptok_mfma(const QuantArgs& a, hipStream_t st) {
  int lgL = 0;
  while ((int64_t(128) << lgL) < a.dim) ++lgL;
  if ((1 << lgL) > PT_ROWS) return hipErrorInvalidValue;   // a vector must fit in one tile
  const int64_t nrows = a.seqs * a.tokens * a.heads * (a.dim / 128);
  if (nrows > 0) {
    const bool rrs = a.seg_div != nullptr;
    if (a.dtype == DT_F16) {
      if (rrs) launch_lg<DT_F16, true>(a, st, nrows, lgL); else launch_lg<DT_F16, false>(a, st, nrows, lgL);
    } else {
      if (rrs) launch_lg<DT_BF16, true>(a, st, nrows, lgL); else launch_lg<DT_BF16, false>(a, st, nrows, lgL);
    }
  }
  return hipGetLastError();
}

}  // namespace kvq
