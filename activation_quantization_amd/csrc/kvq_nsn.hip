// NSN variant for gfx950: normalize -> shift -> normalize, then the per-channel quantizer.
//
// Method source (page title, section): NSNQuant summary, "Normalize-Shift-Normalize (NSN)" (token
// norms to sqrt(d), subtract the channel means, token norms to sqrt(d) again; s1, o, s2 kept to
// reconstruct) and "Hadamard transform" (combined with a randomized Hadamard rotation).  The
// per-channel absmax scale over a block of B tokens and the rounded codes are the norm-separation
// post's quantizer ("the fix") with the Rotated Runtime Smooth analysis' per-channel reading.
//
//   y = R x,  s1 = ||y|| / sqrt(D),  u1 = y / s1,  o = mean of u1 over the block's tokens,
//   u2 = u1 - o,  s2 = ||u2|| / sqrt(D),  u3 = u2 / s2,  scale = max over the block |u3| / Q,
//   c = rne(fp32(u3 / scale));  stored: codes, s1, s2, R^T o (the offset, original domain), scale.
//
// Everything after the fp16/bf16 load is fp64, so every code is the rounding decision of the fp64
// definition (what differs is summation order at the 2^-53 level) and no near-tie path over the
// statistics is needed.  fp64 adds and fmas issue at the fp32 rate on this chip, so the cost is
// the instruction count per element, which the layout keeps low:
//
//   row phase    thread 2 t + h holds channels [h D/2, h D/2 + D/2) of token t: the butterflies
//                over the low channel bits are in registers, the top one (when the rotation spans
//                the row) is a DPP exchange with the neighbouring lane; the token norm is a
//                register sum plus that exchange.
//   transpose    two v_permlane32_swap / v_permlane16_swap steps turn the wave's 32 tokens x D
//                channels into lanes holding D/8 consecutive channels of 4 tokens (tokens
//                differing in bits 3 and 4), with no arithmetic.
//   block phase  the column sums and maxima over the block are 4-token register reductions,
//                then one LDS partial per (lane group, wave), reduced by all threads; the second
//                token norm is a register sum plus three lane exchanges.
//
// Input rows are staged in LDS by global_load_lds (1 KiB per wave instruction, XOR-swizzled
// 16-byte chunks, so the half-row reads are free of bank conflicts); the partials reuse that
// buffer.  Codes leave as D/16-byte pieces, eight lanes completing each token's row.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

template <int N>
__device__ __forceinline__ void fwht64(double (&v)[N], int stages) {
#pragma unroll
  for (int s = 0; s < 7; ++s) {
    if (s < stages) {
      const int st = 1 << s;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if ((i & st) == 0 && i + st < N) {
          const double a = v[i], b = v[i + st];
          v[i] = a + b;
          v[i + st] = a - b;
        }
      }
    }
  }
}

// the value of lane ^ 1 (DPP quad_perm [1, 0, 3, 2] on both halves)
__device__ __forceinline__ double xor1(double x) {
  const u32x2 b = __builtin_bit_cast(u32x2, x);
  u32x2 r;
  r.x = (uint32_t)__builtin_amdgcn_mov_dpp((int)b.x, 0xB1, 0xF, 0xF, false);
  r.y = (uint32_t)__builtin_amdgcn_mov_dpp((int)b.y, 0xB1, 0xF, 0xF, false);
  return __builtin_bit_cast(double, r);
}

// v_permlane32_swap on a pair of doubles: lanes 32..63 of p trade places with lanes 0..31 of q
__device__ __forceinline__ void swap32(double& p, double& q) {
  const u32x2 a = __builtin_bit_cast(u32x2, p), b = __builtin_bit_cast(u32x2, q);
  const auto lo = __builtin_amdgcn_permlane32_swap(a.x, b.x, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(a.y, b.y, false, false);
  p = __builtin_bit_cast(double, u32x2{lo[0], hi[0]});
  q = __builtin_bit_cast(double, u32x2{lo[1], hi[1]});
}
// v_permlane16_swap on a pair of doubles: the odd 16-lane rows of p trade places with the even
// rows of q
__device__ __forceinline__ void swap16(double& p, double& q) {
  const u32x2 a = __builtin_bit_cast(u32x2, p), b = __builtin_bit_cast(u32x2, q);
  const auto lo = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
  p = __builtin_bit_cast(double, u32x2{lo[0], hi[0]});
  q = __builtin_bit_cast(double, u32x2{lo[1], hi[1]});
}
// x + (x of lane ^ 16), x + (x of lane ^ 32): a swap of x with a copy of itself puts both terms in
// every lane
__device__ __forceinline__ double add_xor16(double x) {
  double y = x;
  swap16(x, y);
  return x + y;
}
__device__ __forceinline__ double add_xor32(double x) {
  double y = x;
  swap32(x, y);
  return x + y;
}

// 1 / sqrt(x) for x > 0 to fp64 accuracy: the hardware estimate and two Newton steps (each squares
// the relative error; the estimate is good to about 2^-23)
__device__ __forceinline__ double rsqrt64(double x) {
  double r = __builtin_amdgcn_rsq(x);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double h = -0.5 * x * r;                     // r' = r (3 - x r^2) / 2 = r + r (1/2 - x r^2 / 2)
    r = __builtin_fma(r, __builtin_fma(h, r, 0.5), r);
  }
  return r;
}

// fp64 -> fp16 bits through fp32 (the opaque step keeps the compiler from replacing the two hardware
// conversions by a bitwise fp64 -> fp16 routine)
__device__ __forceinline__ uint16_t f64_to_f16(double x) {
  float f = (float)x;
  asm volatile("" : "+v"(f));
  return (uint16_t)f32_to_f16(f);
}

// byte offset of the double (p, c) in the partials: rows of D doubles in 16-byte chunks, chunk k of
// row p stored at k ^ x with x = (p mod 8) + 8 (bit 4 of p xor the chunk's half-row bit), so that
// the 16 lanes of a partial write (8 rows, both row halves) and those of a reducer read (8
// chunks of rows p and p + 16) hit 16 different 16-byte bank groups
template <int D> __device__ __forceinline__ int part_off(int p, int c) {
  constexpr int HB = D == 128 ? 5 : 4;                 // chunk bit of the half row
  const int k = c >> 1;
  const int x = (p & 7) | ((((p >> 4) ^ (k >> HB)) & 1) << 3);
  return p * (8 * D) + 16 * (k ^ x) + 8 * (c & 1);
}
// index of channel c in the padded per-channel arrays (4 doubles of padding per D/8 channels: the
// eight lanes reading D/8 consecutive channels each at different bases hit different banks)
template <int D> __device__ __forceinline__ int cpad(int c) { return c + 4 * (c / (D / 8)); }

template <int DT, int D, int LG, int B>
__global__ void __launch_bounds__(2 * B) __attribute__((amdgpu_waves_per_eu(2))) quant_nsn_tile(NsnArgs a, int64_t ntiles) {
  constexpr int RH = D / 2;                            // row phase: channels per thread
  constexpr int CQ = D / 8;                            // block phase: channels per lane (x 4 tokens)
  constexpr int NW = 2 * B / 64;                       // waves (32 tokens each)
  constexpr int ROWB = 2 * D, CPR = ROWB / 16;         // input row bytes, 16-byte chunks per row
  constexpr int WSTAGE = B * ROWB / NW, NLD = WSTAGE / 1024;
  constexpr int LGD = D == 128 ? 7 : 6;
  constexpr bool CROSS = LG == LGD;                    // the rotation's top stage crosses the halves
  constexpr int P = 8 * NW;                            // partial rows: (wave, lane group)
  constexpr int TPC = 2 * B / D, RPT = P / TPC;        // reducers per channel, rows each
  static_assert(B * ROWB == P * 8 * D && NLD >= 1, "tile shape");
  // two tile buffers: the staged input rows of the tile in work (which then hold its column
  // partials) and those of the next tile, in flight
  __shared__ __attribute__((aligned(16))) unsigned char stage0[B * ROWB];
  __shared__ __attribute__((aligned(16))) unsigned char stage1[B * ROWB];
  __shared__ __attribute__((aligned(16))) double omean[D + 32];   // the block's column mean o (cpad)
  __shared__ __attribute__((aligned(16))) double oinv[D + 32];    // Q / the column's max |u3| (cpad)
  __shared__ __attribute__((aligned(16))) uint32_t smask[D / 2];   // sign bits of the channel pairs

  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int64_t nb = a.tokens / B;
  const double rd = sqrt((double)D), qd = (double)a.q;
  // this workgroup's tiles [t_first, t_end): an equal contiguous share
  const int64_t t_first = (int64_t)blockIdx.x * ntiles / gridDim.x;
  const int64_t t_end = ((int64_t)blockIdx.x + 1) * ntiles / gridDim.x;

  // issue the loads of tile tl's rows into buf (this wave's B / NW rows; slot cc of row r holds
  // chunk cc ^ (r % CPR)); returns the head's sign bytes of channels 2 tid, 2 tid + 1 (a load in
  // flight, first used after the next full wait)
  // a tile's coordinates: stream hs = seq heads + h and block blk; consecutive tiles advance blk
  // first, then the head, then the sequence (no divisions past the first tile)
  struct TileC { int64_t hs, blk, seq, h; };
  auto next_tile = [&](TileC c) {
    if (++c.blk == nb) {
      c.blk = 0;
      ++c.hs;
      if (++c.h == a.heads) { c.h = 0; ++c.seq; }
    }
    return c;
  };

  auto prefetch = [&](const TileC& tc, unsigned char* buf) -> uint32_t {
    int tid = threadIdx.x;                             // opaque: the addresses are not hoisted
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int64_t blk = tc.blk, seq = tc.seq, h = tc.h;
    const unsigned char* xw =
        (const unsigned char*)a.x + (((seq * a.tokens + blk * B) + (B / NW) * w) * a.heads + h) * ROWB;
    const uint32_t tok_bytes = (uint32_t)(a.heads * ROWB);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int p = 64 * k + lane, r = p / CPR, cc = p % CPR;
      const uint32_t off = (uint32_t)r * tok_bytes + 16u * (uint32_t)(cc ^ ((r + (B / NW) * w) % CPR));
      __builtin_amdgcn_global_load_lds((const void*)(xw + off),
                                       (__attribute__((address_space(3))) void*)(buf + w * WSTAGE + k * 1024), 16, 0, KVQ_LOAD_NT);
    }
    uint32_t sg = 0u;
    if constexpr (LG != 0)
      if (tid < D / 2) sg = *(const uint16_t*)(a.signs + h * D + 2 * tid);
    return sg;
  };

  // one tile from `cur` (whose loads were issued one tile earlier, with the sign bytes `sgc`);
  // issues the next tile's loads into `nxt` and returns its sign bytes
  auto step = [&](int64_t tl, const TileC& tc, unsigned char* cur, unsigned char* nxt, uint32_t sgc) -> uint32_t {
    // the lane index, opaque per tile: the many lane-dependent LDS addresses below are then
    // recomputed in each tile instead of being hoisted out of the tile loop and held in registers
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, half = lane & 1, tau = lane >> 1, t = 32 * w + tau;
    const int64_t hs = tc.hs, blk = tc.blk;
    const int64_t tok0 = hs * a.tokens + blk * B;      // head-major index of the tile's first token
    const int64_t sblk = hs * nb + blk;                // the block's scale and offset row

    __builtin_amdgcn_s_waitcnt(0x0070);                // vmcnt(0): this tile's rows and signs
    asm volatile("" ::: "memory");
    if constexpr (LG != 0)
      if (tid < D / 2) smask[tid] = ((sgc & 0x80u) << 8) | ((sgc & 0x8000u) << 16);
    lds_barrier();
    uint32_t sgn = 0u;
    if (tl + 1 < t_end) sgn = prefetch(next_tile(tc), nxt);

    // 1. row phase: y = H diag(sigma) x on this thread's half row in fp64 (left unnormalized)
    double v[RH];
#pragma unroll
    for (int k = 0; k < CPR / 2; ++k) {
      const int cc = half * (CPR / 2) + k;
      u32x4 xv = *(const u32x4*)(cur + t * ROWB + 16 * (cc ^ (t % CPR)));
      if constexpr (LG != 0) xv ^= *(const u32x4*)(smask + half * (RH / 2) + 4 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * k + 2 * e] = (double)lo_f32<DT>(xv[e]);
        v[8 * k + 2 * e + 1] = (double)hi_f32<DT>(xv[e]);
      }
    }
    fwht64<RH>(v, CROSS ? LG - 1 : LG);
    if constexpr (CROSS) {
      const double sgn1 = half ? -1.0 : 1.0;           // (a, b) -> (a + b, a - b) across the pair
#pragma unroll
      for (int i = 0; i < RH; ++i) v[i] = __builtin_fma(v[i], sgn1, xor1(v[i]));
    }
    double k1;                                         // sqrt(D) / ||y||: u1 = k1 y
    {
      double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int i = 0; i < RH; ++i) s4[i & 3] = __builtin_fma(v[i], v[i], s4[i & 3]);
      double ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      ss += xor1(ss);
      const double ri = ss > 0.0 ? rsqrt64(ss) : 0.0;  // 1 / ||y||
      k1 = rd * ri;
      // s1 = ||y|| / (sqrt(n) sqrt(D)) = ss ri / (sqrt(n) sqrt(D))
      if (half == 0) a.s1[tok0 + t] = f64_to_f16(ss * ri * (1.0 / (sqrt((double)(1 << LG)) * rd)));
    }
    lds_barrier();                                     // every row has been read: cur -> partials

    // 2. transpose: register q CQ + i (q = 2 s + r) becomes channel cb + i of token tq(q) =
    //    (tau & 7) + 8 r + 16 s; the token scale k1 follows the same swaps
#pragma unroll
    for (int i = 0; i < RH / 2; ++i) swap32(v[i], v[i + RH / 2]);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < RH / 4; ++i) swap16(v[s * (RH / 2) + i], v[s * (RH / 2) + i + RH / 4]);
    double kk[4] = {k1, k1, k1, k1};
    swap32(kk[0], kk[2]);
    swap32(kk[1], kk[3]);
    swap16(kk[0], kk[1]);
    swap16(kk[2], kk[3]);
    const int cb = half * RH + ((lane >> 5) & 1) * (RH / 2) + ((lane >> 4) & 1) * (RH / 4);
    const int prow = 8 * w + (tau & 7);
    auto tq = [&](int q) { return (tau & 7) + 8 * (q & 1) + 16 * (q >> 1); };

    // block-wide column reduction of this lane's CQ values val(i) (computed a pair at a time, just
    // before its LDS write, so that no array of them is live) through the partials: the reducers
    // (TPC threads per channel, RPT rows each) leave the result of `fin` in dst[c]
    auto column_reduce = [&](auto val, auto op, auto fin, double* dst) {
#pragma unroll
      for (int m = 0; m < CQ / 2; ++m) {
        typedef double d2 __attribute__((ext_vector_type(2)));
        *(d2*)(cur + part_off<D>(prow, cb + 2 * m)) = d2{val(2 * m), val(2 * m + 1)};
      }
      lds_barrier();
      const int c = tid / TPC, j = tid % TPC;
      double r = *(const double*)(cur + part_off<D>(j * RPT, c));
#pragma unroll
      for (int k = 1; k < RPT; ++k) r = op(r, *(const double*)(cur + part_off<D>(j * RPT + k, c)));
#pragma unroll
      for (int m = 1; m < TPC; m <<= 1) r = op(r, __shfl_xor(r, m));
      if (j == 0) dst[cpad<D>(c)] = fin(r, c);
      lds_barrier();
    };

    // 3. o: column sums of u1 = k y over the block
    column_reduce(
        [&](int i) {
          return __builtin_fma(v[i], kk[0],
                               __builtin_fma(v[CQ + i], kk[1], __builtin_fma(v[2 * CQ + i], kk[2], v[3 * CQ + i] * kk[3])));
        },
        [](double x, double y) { return x + y; }, [](double r, int) { return r * (1.0 / (double)B); }, omean);

    // 4. the stored offset R^T o = diag(sigma) H o / sqrt(n), by the last wave (D / 64 channels a lane)
    if (w == NW - 1) {
      constexpr int PL = D / 64;
      double of[PL];
#pragma unroll
      for (int e = 0; e < PL; ++e) of[e] = omean[cpad<D>(lane + 64 * e)];
      if constexpr (PL == 2 && LG == 7) {
        const double x0 = of[0], x1 = of[1];
        of[0] = x0 + x1;
        of[1] = x0 - x1;
      }
#pragma unroll
      for (int s = 0; s < 6; ++s) {
        if (s < LG) {
          const int m = 1 << s;
#pragma unroll
          for (int e = 0; e < PL; ++e) {
            const double pv = __shfl_xor(of[e], m);
            of[e] = (lane & m) ? pv - of[e] : of[e] + pv;
          }
        }
      }
      const double rn = 1.0 / sqrt((double)(1 << LG));
#pragma unroll
      for (int e = 0; e < PL; ++e) {
        const int c = lane + 64 * e;
        double x = of[e] * rn;
        if constexpr (LG != 0)
          if ((smask[c >> 1] >> (c & 1 ? 31 : 15)) & 1u) x = -x;
        a.offsets[sblk * D + c] = f64_to_f16(x);
      }
    }

    // 5. u2 = k y - o, s2 = ||u2|| / sqrt(D) (0 under 2^-16 sqrt(D)), u3 = u2 / s2; column maxima
    {
      double ss[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int i = 0; i < CQ; ++i) {
        const double o = omean[cpad<D>(cb) + i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q * CQ + i] = __builtin_fma(v[q * CQ + i], kk[q], -o);
          ss[q] = __builtin_fma(v[q * CQ + i], v[q * CQ + i], ss[q]);
        }
      }
      double a2[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double x = ss[q] + xor1(ss[q]);                // the lanes holding token tq(q): lane bits 0, 4, 5
        x = add_xor16(x);
        x = add_xor32(x);
        const bool zero = x < 0x1p-32 * (double)D;    // ||u2|| < 2^-16 sqrt(D)
        const double ri = zero ? 0.0 : rsqrt64(x);     // 1 / ||u2||
        a2[q] = rd * ri;
        if ((lane & 0x31) == 0) a.s2[tok0 + 32 * w + tq(q)] = zero ? (uint16_t)0 : f64_to_f16(x * ri * (1.0 / rd));
      }
      column_reduce(
          [&](int i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q * CQ + i] *= a2[q];
            return fmax(fmax(fabs(v[i]), fabs(v[CQ + i])), fmax(fabs(v[2 * CQ + i]), fabs(v[3 * CQ + i])));
          },
          [](double x, double y) { return fmax(x, y); },
          [&](double r, int c) {
            a.scales[sblk * D + c] = f64_to_f16(r / qd);
            return r > 0.0 ? qd / r : 0.0;
          },
          oinv);
    }

    // 6. codes c = rne(u3 / scale): g = fp32(u3 (Q / max) + 136.5) from one fp64 fma; g lies on
    //    the 2^-16 grid of [128, 256), so byte 2 of its bits is floor(u3 / scale + 8.5) unless the
    //    rounding landed g on an integer, which happens exactly for the values within 2^-17 of a
    //    tie (and every value whose fp32 rounding could decide the tie); a lane holding such a value
    //    (rare) rounds its values again as rint(u3 / scale) in fp64
    constexpr int NG = CQ / 8;                         // packed words per token
    uint32_t pk[4][NG];
    uint32_t fl = 0xffffffffu;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      double iv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) iv[e] = oinv[cpad<D>(cb) + 8 * g + e];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          b[e] = __builtin_bit_cast(uint32_t, (float)__builtin_fma(v[q * CQ + 8 * g + e], iv[e], (double)CODE_MAGIC));
        fl = min3_u16(fl, b[0], b[1]);
        fl = min3_u16(fl, b[2], b[3]);
        fl = min3_u16(fl, b[4], b[5]);
        fl = min3_u16(fl, b[6], b[7]);
        pk[q][g] = pack8(b);
      }
    }
    if ((fl & 0xffffu) == 0u) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          uint32_t word = 0u;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int c = (int)__builtin_rint(v[q * CQ + 8 * g + e] * oinv[cpad<D>(cb) + 8 * g + e]);
            word |= ((uint32_t)c & 0xFu) << (4 * e);
          }
          pk[q][g] = word;
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned char* cp = a.codes + (tok0 + 32 * w + tq(q)) * (D / 2) + cb / 2;
      if constexpr (NG == 2)
        __builtin_nontemporal_store(u32x2{pk[q][0], pk[q][1]}, (u32x2*)cp);
      else
        __builtin_nontemporal_store(pk[q][0], (uint32_t*)cp);
    }
    return sgn;
  };

  if (t_first >= t_end) return;
  TileC tc;
  tc.hs = t_first / nb;
  tc.blk = t_first - tc.hs * nb;
  tc.seq = tc.hs / a.heads;
  tc.h = tc.hs - tc.seq * a.heads;
  uint32_t sg = prefetch(tc, stage0);
  for (int64_t tl = t_first; tl < t_end; ++tl) {
    const bool odd = ((tl - t_first) & 1) != 0;
    sg = step(tl, tc, odd ? stage1 : stage0, odd ? stage0 : stage1, sg);
    tc = next_tile(tc);
  }
}

template <int DT, int D, int LG, int B>
void launch_nsn_k(const NsnArgs& a, hipStream_t st) {
  const int64_t ntiles = a.seqs * (a.tokens / B) * a.heads;
  const int64_t grid = persistent_grid(quant_nsn_tile<DT, D, LG, B>, 2 * B, ntiles);
  hipLaunchKernelGGL((quant_nsn_tile<DT, D, LG, B>), dim3((unsigned)grid), dim3(2 * B), 0, st, a, ntiles);
}

template <int DT, int D, int LG>
void nsn_by_b(const NsnArgs& a, hipStream_t st) {
  if (a.block == 64) launch_nsn_k<DT, D, LG, 64>(a, st);
  else if (a.block == 128) launch_nsn_k<DT, D, LG, 128>(a, st);
  else if constexpr (D == 64) launch_nsn_k<DT, D, LG, 256>(a, st);
}

template <int DT, int D>
void nsn_by_lg(const NsnArgs& a, hipStream_t st) {
  switch (a.lg_had) {
    case 0: nsn_by_b<DT, D, 0>(a, st); break;
    case 4: nsn_by_b<DT, D, 4>(a, st); break;
    case 5: nsn_by_b<DT, D, 5>(a, st); break;
    case 6: nsn_by_b<DT, D, 6>(a, st); break;
    default: if constexpr (D == 128) nsn_by_b<DT, D, 7>(a, st); break;
  }
}

}  // namespace

hipError_t launch_quantize_nsn(const NsnArgs& a, hipStream_t st) {
  if (a.dtype == DT_F16) {
    if (a.dim == 128) nsn_by_lg<DT_F16, 128>(a, st); else nsn_by_lg<DT_F16, 64>(a, st);
  } else {
    if (a.dim == 128) nsn_by_lg<DT_BF16, 128>(a, st); else nsn_by_lg<DT_BF16, 64>(a, st);
  }
  return hipGetLastError();
}

}  // namespace kvq
