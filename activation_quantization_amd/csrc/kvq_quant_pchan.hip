// Per-channel quantize (PCHAN, NSEP_PCHAN) for gfx950 with the rotation on the matrix cores.
//
// Method sources (page title, section): norm-separation post "the fix" (fp16 L2 norm + unit
// direction; absmax / Q, round, clamp) and "next" (per-channel scaling); Rotated Runtime Smooth
// analysis "problem definition" (alpha = max|X| / (2^(N-1)-1)) and "term-by-term"
// (R = (1/sqrt K)[+-1]; runtime scale s_j = max over the tokens of column j); NSNQuant summary
// "Hadamard transform" (random signs, then the Hadamard matrix).
//
// Work split: one workgroup per tile = (sequence, block of B tokens, head), B / 32 waves; wave
// w takes tokens [32 w, 32 w + 32) of the block as two sub-tiles of 16 tokens.  In a sub-tile,
// lane l = 16 g + j holds token j and the R/4 channels [g R/4, (g + 1) R/4): it loads them as
// its part of the MFMA B operand and gets back the rotated values of the same channels from
// the MFMA D layout, so norms, codes and their packing never leave the lane.
//
// Rotation: Y^T = blockdiag(H_n) diag(sigma) X^T per sub-tile with v_mfma_f32_16x16x32 (f16 or
// bf16 operands, fp32 accumulation; the +-1 products are exact).  Output rows are channels
// c = (R/4)(i >> 2) + 4 I + (i & 3) of I-block I, the contraction index of K step K is
// c' = (R/4) g + 8 K + e.  With this numbering every 16 x 32 block of the n x n matrix is
// beta(I, K) * F_{I mod 2}: two fixed +-1/0 fragments and a sign or zero that depends only on
// (I, K) and is known at compile time, so four fragment registers hold the whole transform.
// The random signs flip the sign bits of the B operand.  The transform is left unnormalized:
// 1/sqrt(n) cancels in every quotient and only enters the stored scale.
//
// Scales: u = y / ||y|| (||y|| = ||x||, taken from the input with exact fp16/bf16 squares);
// the per-channel max over the block goes through LDS once per tile.  Codes: one fma per value,
// b = bits(u * (Q / m) + 136.5): byte 2 of b is code + 8 (round half up on a 2^-16 grid) and
// b & 0xffff == 0 marks a near-tie, |v - (k + 1/2)| <= 2^-17.  Near-ties are re-decided
// exactly: the channel's max is recomputed in fp64 from the tokens whose fp32 value is within
// 2^-12 of it, the flagged values in fp64 too, and the code is rne(fp32(v)).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float CODE_MAGIC = 136.5f;   // 128 + 8 + 1/2: [128, 256) has ulp 2^-16

template <int DT> __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
}

// Sign / zero of block (I, K) relative to F_{I mod 2}: bits 3.. of the output channel come
// from I >> 1 and bits 3.. of the input channel from K.
template <int LG> __device__ __forceinline__ constexpr int frag_beta(int I, int K) {
  const int n = 1 << LG, a = (I >> 1) << 3, k = K << 3;
  if ((a & ~(n - 1)) != (k & ~(n - 1))) return 0;
  return (__builtin_popcount(a & k & (n - 1)) & 1) ? -1 : 1;
}

// This lane's part of F_p (A operand: row i = lane & 15, inputs 8 (lane >> 4) + e): entry
// (c, c') of blockdiag(H_n) for I = p, K = 0.
template <int DT, int R, int LG> __device__ __forceinline__ u32x4 hadamard_fragment(int p, int lane) {
  const int i = lane & 15, gk = lane >> 4;
  const int c = (R / 4) * (i >> 2) + 4 * p + (i & 3);
  const uint32_t one = DT == DT_F16 ? 0x3C00u : 0x3F80u;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t pair = 0u;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int cp = (R / 4) * gk + 2 * q + hh;
      uint32_t v = 0u;
      if ((c >> LG) == (cp >> LG)) v = one | ((uint32_t)(__builtin_popcount(c & cp & ((1 << LG) - 1)) & 1) << 15);
      pair |= v << (16 * hh);
    }
    w[q] = pair;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Sign-bit masks of the 8 random signs of K step K in this lane (0x8000 per negated half).
template <int R> __device__ __forceinline__ u32x4 sign_masks(const int8_t* __restrict__ sg, int g, int K) {
  const u32x2 s8 = *(const u32x2*)(sg + (R / 4) * g + 8 * K);
  uint32_t m[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t sw = q < 2 ? s8.x : s8.y;
    m[q] = __builtin_amdgcn_perm(0u, sw, (q & 1) ? 0x030C020Cu : 0x010C000Cu) & 0x80008000u;
  }
  return u32x4{m[0], m[1], m[2], m[3]};
}

template <int DT> __device__ __forceinline__ float sumsq2(uint32_t x, float acc) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, x), acc, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, x), acc, false);
}

__device__ __forceinline__ uint32_t min3_u16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_min3_u16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// 8 codes (fma results of channels 8d .. 8d + 7 of the lane) -> one packed word
__device__ __forceinline__ uint32_t pack8(const uint32_t (&b)[8]) {
  const uint32_t ev = __builtin_amdgcn_perm(b[2], b[0], 0x0C0C0602u) | __builtin_amdgcn_perm(b[6], b[4], 0x06020C0Cu);
  const uint32_t od = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0602u) | __builtin_amdgcn_perm(b[7], b[5], 0x06020C0Cu);
  return ((od << 4) | ev) ^ 0x88888888u;   // byte k = nibble(c_2k) | nibble(c_2k+1) << 4
}

template <int DT> __device__ __forceinline__ double widen64(uint32_t h) {
  return (double)(DT == DT_F16 ? f16_to_f32(h) : bf16_to_f32(h));
}

// Exact (fp64) parts of one token for the rare path: over this lane's R/4 input channels,
// the unnormalized rotated value of channel c (sum of +-x, exact) and the sum of squares.
struct ExactParts {
  double y, ss;
};
template <int DT, int R, int LG>
__device__ __noinline__ ExactParts exact_parts(const unsigned char* __restrict__ xrow, const int8_t* __restrict__ sgl,
                                               int c0, int c) {
  constexpr int n = 1 << LG;
  double y = 0.0, ss = 0.0;
#pragma unroll 1
  for (int q = 0; q < R / 32; ++q) {
    const u32x4 v = *(const u32x4*)(xrow + 16 * q);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = c0 + 8 * q + e;
      const double x = widen64<DT>((e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xffffu));
      ss = __builtin_fma(x, x, ss);
      if constexpr (LG == 0) {
        if (k == c) y = x;
      } else if ((k >> LG) == (c >> LG)) {
        const bool neg = ((__builtin_popcount(k & c & (n - 1)) & 1) != 0) != (sgl[k] < 0);
        y += neg ? -x : x;
      }
    }
  }
  return ExactParts{y, ss};
}

__device__ __forceinline__ uint32_t exact_nibble(double v) {
  return (uint32_t)(int)__builtin_rintf((float)v) & 0xfu;
}

template <int DT, int R, int LG, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3))) quant_pchan_mfma(QuantArgs a, int64_t ntiles) {
  constexpr int B = 32 * NW;
  constexpr int NK = R / 32;            // K steps per sub-tile
  constexpr int NI = R / 16;            // output blocks of 16 channels
  constexpr int CL = R / 4;             // channels per lane
  constexpr int NP = R / 32;            // packed code words per lane and sub-tile
  // per wave: its 32 input rows (staged by global_load_lds), later reused for its lane maxima
  constexpr int ROWB = 2 * R;           // input row bytes
  constexpr int CPR = ROWB / 16;        // 16-byte chunks per row
  constexpr int WSTAGE = 32 * ROWB;     // bytes per wave (= (R/4) quads x 16 slots x 16 B)
  __shared__ __attribute__((aligned(16))) unsigned char stage[NW * WSTAGE];
  __shared__ __attribute__((aligned(16))) float invs[R];
  __shared__ unsigned long long m64[R];
  __shared__ uint32_t chmask[R / 32];
  __shared__ uint32_t wflag[NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t h = tile % a.heads, sb = tile / a.heads;
  const int64_t nb = a.tokens / B;
  const int64_t seq = sb / nb;
  const int64_t row0 = seq * a.tokens + (sb - seq * nb) * B + 32 * w;   // first token of this wave

  // 1. signs and fragments (issued first: sub-tile 0 must not wait for them behind its input),
  //    then the input of both sub-tiles, 4 x 16 B per lane and sub-tile (R = 128)
  const int8_t* sgh = a.signs ? a.signs + h * R : nullptr;
  u32x4 fr[4], sm[NK];
  if constexpr (LG != 0) {
    fr[0] = hadamard_fragment<DT, R, LG>(0, lane);
    fr[1] = hadamard_fragment<DT, R, LG>(1, lane);
    fr[2] = fr[0] ^ 0x80008000u;
    fr[3] = fr[1] ^ 0x80008000u;
#pragma unroll
    for (int K = 0; K < NK; ++K) sm[K] = sign_masks<R>(sgh, g, K);
  }
  // the wave's 32 rows: instruction k moves 1 KiB (64 lanes x 16 B) into LDS; the chunk that
  // lane p fetches is XOR-swizzled with its row so that the MFMA-layout reads below are free
  // of bank conflicts (slot cc of row r holds chunk cc ^ (r mod CPR))
  unsigned char* wst = stage + w * WSTAGE;
  const unsigned char* xw = (const unsigned char*)a.x + ((row0 * a.heads + h) * R) * 2;
  const int64_t tok_bytes = a.heads * ROWB;
#pragma unroll
  for (int k = 0; k < WSTAGE / 1024; ++k) {
    const int p = 64 * k + lane, row = p / CPR, cc = p % CPR;
    __builtin_amdgcn_global_load_lds((const void*)(xw + row * tok_bytes + 16 * (cc ^ (row % CPR))),
                                     (__attribute__((address_space(3))) void*)(wst + k * 1024), 16, 0, 0);
  }
  if (tid < R) m64[tid] = 0ull;
  if (tid < R / 32) chmask[tid] = 0u;
  if (tid < NW) wflag[tid] = 0u;
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): the staged rows (and the signs) have landed
  asm volatile("" ::: "memory");
  u32x4 xin[2][NK];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int row = 16 * s + j;
#pragma unroll
    for (int K = 0; K < NK; ++K)
      xin[s][K] = *(const u32x4*)(wst + row * ROWB + 16 * (((R / 32) * g + K) ^ (row % CPR)));
  }

  // 2. norms and the rotation, sub-tile by sub-tile
  f32x4 u[2][NI];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float inv_nu = 1.f;
    if (a.nsep) {
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int K = 0; K < NK; ++K) {
        p0 = sumsq2<DT>(xin[s][K].x, p0);
        p1 = sumsq2<DT>(xin[s][K].y, p1);
        p0 = sumsq2<DT>(xin[s][K].z, p0);
        p1 = sumsq2<DT>(xin[s][K].w, p1);
      }
      float ss = p0 + p1;
      ss += shfl_xor_f(ss, 16);
      ss += shfl_xor_f(ss, 32);
      inv_nu = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
      if (g == 0) a.norms[(row0 + 16 * s + j) * a.heads + h] = (uint16_t)f32_to_f16(ss * inv_nu);
    }
    if constexpr (LG == 0) {
#pragma unroll
      for (int K = 0; K < NK; ++K) {
        const uint32_t q[4] = {xin[s][K].x, xin[s][K].y, xin[s][K].z, xin[s][K].w};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          u[s][2 * K + hh] = f32x4{lo_f32<DT>(q[2 * hh]), hi_f32<DT>(q[2 * hh]), lo_f32<DT>(q[2 * hh + 1]),
                                   hi_f32<DT>(q[2 * hh + 1])};
      }
    } else {
      u32x4 xs[NK];
#pragma unroll
      for (int K = 0; K < NK; ++K) xs[K] = xin[s][K] ^ sm[K];
#pragma unroll
      for (int I = 0; I < NI; ++I) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < NK; ++K) {
          const int bt = frag_beta<LG>(I, K);
          if (bt != 0) acc = mfma16<DT>(fr[(I & 1) + (bt < 0 ? 2 : 0)], xs[K], acc);
        }
        u[s][I] = acc;
      }
    }
    if (a.nsep) {
#pragma unroll
      for (int I = 0; I < NI; ++I) u[s][I] *= inv_nu;
    }
  }

  // 3. per-channel max over the block: lane maxima of the two tokens -> LDS (over the wave's own
  //    staged rows, which it has finished reading); TPQ threads then
  //    reduce channels 4 cq .. 4 cq + 3, each over R/16 of the 16 NW token slots, and finish
  //    with lane shuffles inside their aligned group
#pragma unroll
  for (int I = 0; I < NI; ++I) {
    const f32x4 m = {fmaxf(fabsf(u[0][I].x), fabsf(u[1][I].x)), fmaxf(fabsf(u[0][I].y), fabsf(u[1][I].y)),
                     fmaxf(fabsf(u[0][I].z), fabsf(u[1][I].z)), fmaxf(fabsf(u[0][I].w), fabsf(u[1][I].w))};
    ((f32x4*)wst)[(NI * g + I) * 16 + j] = m;   // slot (quad NI g + I, token j) of this wave
  }
  lds_barrier();
  {
    constexpr int TPQ = NW * 256 / R;     // threads per channel quad
    constexpr int SPT = R / 16;           // token slots per thread
    const int cq = tid / TPQ, part = tid % TPQ;
    const int slot0 = part * SPT;                     // of the 16 NW (wave, token) slots
    const f32x4* rp = (const f32x4*)(stage + (slot0 / 16) * WSTAGE) + cq * 16 + slot0 % 16;
    f32x4 mx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const f32x4 v = rp[(k + tid) % SPT];
      mx = f32x4{fmaxf(mx.x, v.x), fmaxf(mx.y, v.y), fmaxf(mx.z, v.z), fmaxf(mx.w, v.w)};
    }
#pragma unroll
    for (int o = 1; o < TPQ; o <<= 1) {
      mx.x = fmaxf(mx.x, shfl_xor_f(mx.x, o));
      mx.y = fmaxf(mx.y, shfl_xor_f(mx.y, o));
      mx.z = fmaxf(mx.z, shfl_xor_f(mx.z, o));
      mx.w = fmaxf(mx.w, shfl_xor_f(mx.w, o));
    }
    if (part == 0) {
      const float mm[4] = {mx.x, mx.y, mx.z, mx.w};
      f32x4 iv;
      uint16_t* sp = a.scales + (sb * a.heads + h) * R + 4 * cq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        iv[r] = mm[r] > 0.f ? a.q / mm[r] : 0.f;
        sp[r] = (uint16_t)f32_to_f16(mm[r] * a.scale_mul);
      }
      *(f32x4*)(invs + 4 * cq) = iv;
    }
  }
  lds_barrier();

  // 4. codes and near-tie flags
  f32x4 iv[NI];
#pragma unroll
  for (int I = 0; I < NI; ++I) iv[I] = *(const f32x4*)(invs + CL * g + 4 * I);
  uint32_t pk[2][NP];
  uint32_t fl = 0xffffffffu;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int d = 0; d < NP; ++d) {
      uint32_t b[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        b[r] = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[s][2 * d][r], iv[2 * d][r], CODE_MAGIC));
        b[4 + r] = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[s][2 * d + 1][r], iv[2 * d + 1][r], CODE_MAGIC));
      }
      fl = min3_u16(fl, b[0], b[1]);
      fl = min3_u16(fl, b[2], b[3]);
      fl = min3_u16(fl, b[4], b[5]);
      fl = min3_u16(fl, b[6], b[7]);
      pk[s][d] = pack8(b);
    }
  }
  if (__ballot((fl & 0xffffu) == 0u) != 0ull && lane == 0) wflag[w] = 1u;
  lds_barrier();
  uint32_t any = 0u;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) any |= wflag[ww];

  // 5. rare path: exact re-decision of the near-ties (whole workgroup, uniform control flow)
  if (any) {
    uint32_t cm[2] = {0u, 0u};
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int I = 0; I < NI; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t bb = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[s][I][r], iv[I][r], CODE_MAGIC));
          if ((bb & 0xffffu) == 0u) cm[s] |= 1u << (4 * I + r);
        }
    const uint32_t cml = cm[0] | cm[1];
    if (cml) atomicOr(&chmask[(CL * g) >> 5], cml << ((CL * g) & 31));
    lds_barrier();
    const double qd = (double)a.q;
    // pass 0: exact maxima of the flagged channels (from the tokens near the fp32 max);
    // pass 1: exact codes of the flagged values
    for (int pass = 0; pass < 2; ++pass) {
      for (int wd = 0; wd < R / 32; ++wd) {
        uint32_t bits = chmask[wd];
        while (bits) {
          const int c = 32 * wd + __builtin_ctz(bits);
          bits &= bits - 1u;
          const int gc = c / CL, k = c % CL;
          const float ivc = invs[c];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            bool need = false;
            if (g == gc) {
              float uv = 0.f;   // u[s][k / 4][k % 4] (k is uniform: selects, no indexed registers)
#pragma unroll
              for (int I = 0; I < NI; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (4 * I + r == k) uv = u[s][I][r];
              need = pass == 0 ? fabsf(uv) * ivc >= a.q * (1.f - 0x1p-12f) : ((cm[s] >> k) & 1u) != 0u;
            }
            need = __shfl(need ? 1 : 0, j + 16 * gc) != 0;
            double y = 0.0, ss = 0.0;
            if (need) {
              const unsigned char* xr =
                  (const unsigned char*)a.x + (((row0 + 16 * s + j) * a.heads + h) * R + CL * g) * 2;
              const ExactParts ep = exact_parts<DT, R, LG>(xr, sgh, CL * g, c);
              y = ep.y;
              ss = ep.ss;
            }
            y += __shfl_xor(y, 16);
            y += __shfl_xor(y, 32);
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            if (need && g == gc) {
              const double nu = sqrt(ss);
              const double uv = a.nsep ? (nu > 0.0 ? y / nu : 0.0) : y;
              if (pass == 0) {
                atomicMax(&m64[c], __builtin_bit_cast(unsigned long long, fabs(uv)));
              } else {
                const double mm = __builtin_bit_cast(double, m64[c]);
                const uint32_t nib = mm > 0.0 ? exact_nibble(qd * uv / mm) : 0u;
                const int sh = 4 * (k & 7);
#pragma unroll
                for (int d = 0; d < NP; ++d)
                  if (d == (k >> 3)) pk[s][d] = (pk[s][d] & ~(0xFu << sh)) | (nib << sh);
              }
            }
          }
        }
      }
      lds_barrier();
    }
  }

  // 6. codes: 16 bytes per lane and sub-tile (R = 128)
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    unsigned char* cp = a.codes + ((row0 + 16 * s + j) * a.heads + h) * (R / 2) + (R / 8) * g;
    if constexpr (NP == 4)
      __builtin_nontemporal_store(u32x4{pk[s][0], pk[s][1], pk[s][2], pk[s][3]}, (u32x4*)cp);
    else
      __builtin_nontemporal_store(u32x2{pk[s][0], pk[s][1]}, (u32x2*)cp);
  }
}

template <int DT, int R, int LG>
void launch_r(const QuantArgs& a, hipStream_t st) {
  const int64_t ntiles = a.seqs * (a.tokens / a.block) * a.heads;
  if (a.block == 64)
    hipLaunchKernelGGL((quant_pchan_mfma<DT, R, LG, 2>), dim3((unsigned)ntiles), dim3(128), 0, st, a, ntiles);
  else if (a.block == 128)
    hipLaunchKernelGGL((quant_pchan_mfma<DT, R, LG, 4>), dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles);
  else if constexpr (R == 64)
    hipLaunchKernelGGL((quant_pchan_mfma<DT, R, LG, 8>), dim3((unsigned)ntiles), dim3(512), 0, st, a, ntiles);
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
