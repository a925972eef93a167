// Dequantize kernels for gfx950: unpack nibbles -> code * scale (* norm) -> inverse
// randomized Hadamard -> convert, one pass over HBM.
//
// Method sources (page title, section): norm-separation post "the fix" (direction_q is the
// code times the scale; the norm multiplies back); Rotated Runtime Smooth analysis
// "term-by-term" (R^-1 = R^T); NSNQuant summary "implementation details" (a dedicated
// dequantization kernel that keeps DRAM traffic minimal).
//
// Main kernel (dequant_mfma, every per-channel mode and per-token token counts that are a multiple
// of 64): the inverse rotation is one matrix-core contraction per 16 tokens, codes (exact small
// integers in fp16) times H diag(scale) built from per-tile fragments; each lane ends with 8
// consecutive output channels of 4 tokens and the 16 lanes of a row store whole output rows.
// Fallback (per-token modes with other token counts): one thread owns one row of R channels in
// VGPRs, with a register butterfly, and codes come in and values go out through XOR-swizzled LDS
// tiles so both HBM streams are coalesced.
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_launch.h"

namespace kvq {

template <int R>
__device__ __forceinline__ void unsign(float (&y)[R], const int8_t* __restrict__ sg) {
#pragma unroll
  for (int c = 0; c < R / 16; ++c) {
    const u32x4 sv = *(const u32x4*)(sg + 16 * c);
    const uint32_t s4[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t neg = (s4[j >> 2] >> (8 * (j & 3) + 7)) & 1u;
      y[16 * c + j] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, y[16 * c + j]) ^ (neg << 31));
    }
  }
}

// signed 4-bit code e of a packed word, as float
__device__ __forceinline__ float nib_f(uint32_t word, int e) {
  return (float)((int)(((word >> (4 * e)) & 0xfu) ^ 8u) - 8);
}

// Write row `row` (R values) into the LDS output tile in the output dtype.
template <int ODT, int R>
__device__ __forceinline__ void stage_row(unsigned char* stage, int row, const float (&y)[R]) {
  constexpr int OB = ODT == DT_F32 ? 4 : 2;
  constexpr int ROWB = R * OB, CPR = ROWB / 16;
#pragma unroll
  for (int cc = 0; cc < CPR; ++cc) {
    u32x4 v;
    if constexpr (ODT == DT_F32) {
      v = u32x4{__builtin_bit_cast(uint32_t, y[4 * cc]), __builtin_bit_cast(uint32_t, y[4 * cc + 1]),
                __builtin_bit_cast(uint32_t, y[4 * cc + 2]), __builtin_bit_cast(uint32_t, y[4 * cc + 3])};
    } else {
      v = u32x4{pack2<ODT>(y[8 * cc], y[8 * cc + 1]), pack2<ODT>(y[8 * cc + 2], y[8 * cc + 3]),
                pack2<ODT>(y[8 * cc + 4], y[8 * cc + 5]), pack2<ODT>(y[8 * cc + 6], y[8 * cc + 7])};
    }
    *(u32x4*)(stage + row * ROWB + swz_chunk(row, cc, ROWB) * 16) = v;
  }
}

// ---------------------------------------------------------------------------------------
// Per-channel modes on the matrix cores.  The grid holds only as many workgroups (4 waves) as
// fit on the chip at once; each walks an equal share of the 64-token chunks of all head-major
// (sequence, head) streams, in order (a share may span streams), so no partly filled last
// round of workgroups is left.  Wave w takes tokens [16 w, 16 w + 16) of each chunk.  Three
// waves per SIMD keep enough loads in flight (an explicit prefetch of the next chunk measured
// no faster).
//
//   x^[t, c] = norm[t] * sigma[c] / sqrt(n) * sum_k H[c, k] * scale[k] * code[t, k]
//
// is D = A B with A = the codes (row i = token, fp16, exact) and B(I) = H diag(scale) for the
// output channels c = L j + I (L = R / 16 I-blocks; column j of the MFMA).  Lane (g, j) of a
// K step holds input channels k = (R/4) g + 8 K + nib(e) (its code load, converted in the
// [n0 n4 n1 n5 ...] order).  Since c and k share no bit below log2 L other than through I,
//   H[c, k] = [block(L j) == block(k)] (-1)^popcount(L j & k & (n-1)) * (-1)^popcount(I & k & (L-1))
// where the first two factors depend on the lane and K (and, for L = 4, on the parity of e) but
// not on I: B(I) = (scale pairs & keep mask ^ lane sign mask) ^ a constant sign pattern per I.  Lane (g, j) of the result
// holds tokens 4 g + r, channel L j + I; after all I it owns channels [L j, L j + L) of four
// tokens, so the 16 lanes of a row store whole output rows.  The products scale * code are
// exact in fp32 (11 x 4 bits).

template <int R, bool PT, bool NS>
struct DqPre {
  static constexpr int KS = R / 32;
  uint32_t wd[KS];          // packed codes of token j, channels (R/4) g ..
  uint32_t nw[2];           // fp16 norms of tokens 4 g + r, r = 0..3
  u32x4 sc[PT ? 1 : KS];    // per-channel: fp16 scales of channels (R/4) g + 8 K + [0, 8);
                            // per-token: sc[0].x, .y = fp16 scales of tokens 4 g + r
  uint32_t n2[NS ? 2 : 1];  // NSN: fp16 second scales s2 of tokens 4 g + r
  uint32_t of[NS ? R / 32 : 1];   // NSN: fp16 offsets of channels L j .. L j + L - 1 (pairs)
};

//
// Per-token scales (PT) use the same contraction with diag(scale) = I; the token's scale joins
// its norm in the row factor.  A vector of D = 2^lgL R channels is 2^lgL row segments, each
// walked as a stream of its own (the rotation is block-diagonal with blocks of at most R).
//
// NSN (NS): x^ = s1 (s2 R^T (c scale) + offset): the row factor is s1 s2 and s1 times the block's
// offset (original domain) is added per output channel.
template <int ODT, int R, int LG, bool PT, bool NS = false, int WPE = 3>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE)))
dequant_mfma(DequantArgs a, int64_t nchunks, int lgL, int vec) {
  constexpr int L = R / 16;                 // I-blocks: output channels per lane and token
  constexpr int KS = R / 32;                // K steps
  constexpr int LB = R / 8;                 // code bytes per lane and token
  constexpr int OB = ODT == DT_F32 ? 4 : 2;
  constexpr int NMASK = LG == 0 ? 0 : (1 << LG) - 1;
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int64_t nch = a.tokens / 64;                         // 64-token chunks per stream
  const int64_t nb = PT ? 0 : a.tokens / a.block;           // per-channel scale blocks per stream
  const int lgb = PT ? 0 : __builtin_ctz((unsigned)a.block); // block = 64, 128 or 256

  // lane constants: keep / sign masks of the base fragment per K; per I the constant pattern
  // with the lane's output sign folded in
  uint32_t keepm[KS], negm[KS];
#pragma unroll
  for (int K = 0; K < KS; ++K) {
    const int k0 = (R / 4) * g + 8 * K;                   // channel of e = 0 (nib 0); e odd: nib >= 4
    if constexpr (LG == 0) {
      keepm[K] = ((k0 & ~(L - 1)) == L * j ? 0x0000ffffu : 0u) | (((k0 + 4) & ~(L - 1)) == L * j ? 0xffff0000u : 0u);
      negm[K] = 0u;
    } else {
      keepm[K] = ((L * j) >> LG) == (k0 >> LG) ? 0xffffffffu : 0u;
      negm[K] = ((uint32_t)(__builtin_popcount((uint32_t)((L * j) & k0 & NMASK)) & 1) << 15) |
                ((uint32_t)(__builtin_popcount((uint32_t)((L * j) & (k0 + 4) & NMASK)) & 1) << 31);
    }
  }
  int64_t k = (int64_t)blockIdx.x * nchunks / gridDim.x;   // this workgroup's chunks [k, kend)
  const int64_t kend = ((int64_t)blockIdx.x + 1) * nchunks / gridDim.x;
  while (k < kend) {
    const int64_t vs = k / nch;                                // (s * heads + h) 2^lgL + segment
    const int64_t ch0 = k - vs * nch;
    const int nt = (int)(kend - k < nch - ch0 ? kend - k : nch - ch0);
    k += nt;
    const int64_t hs = vs >> lgL, seg = vs & ((1 << lgL) - 1);
    const int64_t s = hs / a.heads, h = hs - s * a.heads;
    uint32_t sgn = 0u;                                         // bit I: sigma[L j + I] < 0
    if constexpr (LG != 0) {
      const int8_t* sp = a.signs + h * a.dim + seg * R + L * j;
      if constexpr (L == 8) {
        const u32x2 v = *(const u32x2*)sp;
#pragma unroll
        for (int I = 0; I < 8; ++I) sgn |= (((I < 4 ? v.x : v.y) >> (8 * (I & 3) + 7)) & 1u) << I;
      } else {
        const uint32_t v = *(const uint32_t*)sp;
#pragma unroll
        for (int I = 0; I < 4; ++I) sgn |= ((v >> (8 * I + 7)) & 1u) << I;
      }
    }

    const size_t cstride = (size_t)(R / 2) << lgL;             // code bytes between tokens
    const unsigned char* cstream = a.codes + hs * a.tokens * cstride + seg * (R / 2);
    const uint16_t* nstream = a.nsep ? a.norms + hs * a.tokens : nullptr;
    const uint16_t* sstream = PT ? a.scales + hs * a.tokens : a.scales + hs * nb * R;
    auto load = [&](int i, DqPre<R, PT, NS>& p) {
      const uint32_t t = (uint32_t)((ch0 + i) * 64) + 16 * w;   // stream token of the wave's first row
      const unsigned char* cp = cstream + (size_t)(t + j) * cstride + LB * g;
      if constexpr (KS == 4) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)cp);
        p.wd[0] = v.x; p.wd[1] = v.y; p.wd[2] = v.z; p.wd[3] = v.w;
      } else {
        const u32x2 v = __builtin_nontemporal_load((const u32x2*)cp);
        p.wd[0] = v.x; p.wd[1] = v.y;
      }
      if (a.nsep) {
        const uint16_t* np = nstream + t + 4 * g;
        if (vec) {
          const u32x2 v = *(const u32x2*)np;
          p.nw[0] = v.x; p.nw[1] = v.y;
        } else {
          p.nw[0] = np[0] | ((uint32_t)np[1] << 16);
          p.nw[1] = np[2] | ((uint32_t)np[3] << 16);
        }
      }
      if constexpr (NS) {
        const uint16_t* np = a.s2 + hs * a.tokens + t + 4 * g;
        if (vec) {
          const u32x2 v = *(const u32x2*)np;
          p.n2[0] = v.x; p.n2[1] = v.y;
        } else {
          p.n2[0] = np[0] | ((uint32_t)np[1] << 16);
          p.n2[1] = np[2] | ((uint32_t)np[3] << 16);
        }
        const uint16_t* op = a.offsets + (hs * nb + (t >> lgb)) * R + L * j;
        if constexpr (R == 128) {
          const u32x4 v = *(const u32x4*)op;
          p.of[0] = v.x; p.of[1] = v.y; p.of[2] = v.z; p.of[3] = v.w;
        } else {
          const u32x2 v = *(const u32x2*)op;
          p.of[0] = v.x; p.of[1] = v.y;
        }
      }
      if constexpr (PT) {
        const uint16_t* sp = sstream + t + 4 * g;
        if (vec) {
          const u32x2 v = *(const u32x2*)sp;
          p.sc[0].x = v.x; p.sc[0].y = v.y;
        } else {
          p.sc[0].x = sp[0] | ((uint32_t)sp[1] << 16);
          p.sc[0].y = sp[2] | ((uint32_t)sp[3] << 16);
        }
      } else {
        const uint16_t* srow = sstream + (size_t)(t >> lgb) * R + (R / 4) * g;
#pragma unroll
        for (int K = 0; K < KS; ++K) {
          if (vec) {
            p.sc[K] = *(const u32x4*)(srow + 8 * K);
          } else {
            uint32_t t4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) t4[q] = srow[8 * K + 2 * q] | ((uint32_t)srow[8 * K + 2 * q + 1] << 16);
            p.sc[K] = u32x4{t4[0], t4[1], t4[2], t4[3]};
          }
        }
      }
    };

    const size_t orow = (size_t)a.heads * a.dim * OB;          // bytes between x rows
    unsigned char* const ybase =
        (unsigned char*)a.y + ((s * a.tokens) * a.heads + h) * a.dim * OB + (seg * R + L * j) * OB;
    DqPre<R, PT, NS> cur;
    for (int i = 0; i < nt; ++i) {
      load(i, cur);

      // base fragments: scale pairs in the [n0 n4 n1 n5 ...] order, lane keep and sign masks.
      // Per-token scales make every B fragment loop-invariant; the opaque fp16 pair of ones
      // keeps the compiler from holding all L KS of them in registers across chunks.
      uint32_t one = 0x3C003C00u;
      if constexpr (PT) asm volatile("" : "+v"(one));
      u32x4 base[KS];
#pragma unroll
      for (int K = 0; K < KS; ++K) {
        const u32x4 v = PT ? u32x4{one, one, one, one} : cur.sc[PT ? 0 : K];   // (s0 s1) (s2 s3) (s4 s5) (s6 s7)
        const uint32_t p0 = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);   // (s0 s4)
        const uint32_t p1 = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);   // (s1 s5)
        const uint32_t p2 = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);   // (s2 s6)
        const uint32_t p3 = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);   // (s3 s7)
        base[K] = (u32x4{p0, p1, p2, p3} & keepm[K]) ^ negm[K];
      }
      // A operand: codes as fp16 pairs (c_q, c_{q+4}) = ((word ^ 0x88888888) >> 4 q & 0x000F000F | 0x64006400) - 1032
      u32x4 av[KS];
#pragma unroll
      for (int K = 0; K < KS; ++K) {
        const uint32_t xb = cur.wd[K] ^ 0x88888888u;
        uint32_t q4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x2 hv2 = __builtin_bit_cast(f16x2, ((xb >> (4 * q)) & 0x000F000Fu) | 0x64006400u) -
                            f16x2{(_Float16)1032.0f, (_Float16)1032.0f};
          q4[q] = __builtin_bit_cast(uint32_t, hv2);
        }
        av[K] = u32x4{q4[0], q4[1], q4[2], q4[3]};
      }
      float nu[4], s1v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s1v[r] = a.nsep ? f16_to_f32(cur.nw[r >> 1] >> (16 * (r & 1))) : 1.f;
        nu[r] = s1v[r] * a.inv_sqrt_n;
        if constexpr (PT) {
          const uint32_t sw = r < 2 ? cur.sc[0].x : cur.sc[0].y;
          nu[r] *= f16_to_f32(sw >> (16 * (r & 1)));
        }
        if constexpr (NS) nu[r] *= f16_to_f32(cur.n2[r >> 1] >> (16 * (r & 1)));
      }

      // results: lane (g, j) owns channels [L j, L j + L) of tokens 4 g + r; f16/bf16 outputs are
      // packed as each pair of I-blocks completes (fp32 outputs keep L floats per token)
      constexpr int OW = ODT == DT_F32 ? L : L / 2;            // output words per token row
      uint32_t ow[4][OW];
#pragma unroll
      for (int I = 0; I < L; ++I) {
        const uint32_t sbit = ((sgn >> I) & 1u) << 31;              // sigma of column j's channel
        uint32_t m[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n0 = q, n1 = q + 4;                       // nib of e = 2 q and 2 q + 1
          if constexpr (LG == 0)
            m[q] = ((n0 & (L - 1)) == I ? 0x0000ffffu : 0u) | ((n1 & (L - 1)) == I ? 0xffff0000u : 0u);
          else
            m[q] = ((__builtin_popcount(I & n0 & (L - 1)) & 1) ? 0x00008000u : 0u) |
                   ((__builtin_popcount(I & n1 & (L - 1)) & 1) ? 0x80000000u : 0u);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < KS; ++K) {
          const u32x4 bI = LG == 0 ? (base[K] & u32x4{m[0], m[1], m[2], m[3]}) : (base[K] ^ u32x4{m[0], m[1], m[2], m[3]});
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av[K]), __builtin_bit_cast(f16x8, bI), acc,
                                                       0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, acc[r] * nu[r]) ^ sbit);
          if constexpr (NS) v = __builtin_fmaf(s1v[r], f16_to_f32(cur.of[I >> 1] >> (16 * (I & 1))), v);
          if constexpr (ODT == DT_F32)
            ow[r][I] = __builtin_bit_cast(uint32_t, v);
          else if ((I & 1) == 0)
            ow[r][I / 2] = __builtin_bit_cast(uint32_t, v);   // held until its partner arrives
          else
            ow[r][I / 2] = pack2<ODT>(__builtin_bit_cast(float, ow[r][I / 2]), v);
        }
        // one I-block's fragments live at a time
        __builtin_amdgcn_sched_barrier(0);
      }

      // whole output rows: lanes j = 0..15 of a row cover the R channels of token 4 g + r
      unsigned char* yw = ybase + (size_t)((ch0 + i) * 64 + 16 * w + 4 * g) * orow;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        unsigned char* op = yw + r * orow;
#pragma unroll
        for (int q = 0; q < OW / 4; ++q)
          __builtin_nontemporal_store(u32x4{ow[r][4 * q], ow[r][4 * q + 1], ow[r][4 * q + 2], ow[r][4 * q + 3]},
                                      (u32x4*)(op + 16 * q));
        if constexpr (OW % 4 == 2)
          __builtin_nontemporal_store(u32x2{ow[r][OW - 2], ow[r][OW - 1]}, (u32x2*)(op + 16 * (OW / 4)));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per-token modes: one wave per 64 consecutive row segments of R channels.
template <int ODT, int R, int LG>
__global__ void __launch_bounds__(64) dequant_ptok_kernel(DequantArgs a, int64_t nseg, int64_t ntiles, int lgL) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int CRB = R / 2, CCR = CRB / 16;
  constexpr int OB = ODT == DT_F32 ? 4 : 2;
  constexpr int OROWB = R * OB, OCPR = OROWB / 16;
  unsigned char* stage = smem;
  const int lane = threadIdx.x;
  const int64_t seg0 = xcd_tile(blockIdx.x, ntiles) * 64;
  const int nvalid = (int)(nseg - seg0 < 64 ? nseg - seg0 : 64);

  const int L = 1 << lgL;
  // codes are head-major: segment `sg` (x order) is segment head_major(vector) L + part
#pragma unroll
  for (int k = 0; k < CCR; ++k) {
    const int q = lane + k * 64;
    const int row = q / CCR, cc = q % CCR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < nvalid) {
      const int64_t sg = seg0 + row;
      const int64_t src = a.heads == 1 ? sg : (head_major(a.heads, a.tokens, sg >> lgL) << lgL) + (sg & (L - 1));
      v = __builtin_nontemporal_load((const u32x4*)(a.codes + src * CRB + cc * 16));
    }
    *(u32x4*)(stage + row * CRB + swz_chunk(row, cc, CRB) * 16) = v;
  }
  const int64_t seg = seg0 + lane;
  const int64_t vec = seg >> lgL;
  const int part = (int)(seg & (L - 1));
  const int64_t h = vec % a.heads;
  float f = 0.f;
  if (lane < nvalid) {
    const int64_t vh = head_major(a.heads, a.tokens, vec);
    f = f16_to_f32(a.scales[vh]);
    if (a.nsep) f *= f16_to_f32(a.norms[vh]);
  }
  wave_lds_sync();
  uint32_t cw[R / 8];
#pragma unroll
  for (int cc = 0; cc < CCR; ++cc) {
    const u32x4 v = *(const u32x4*)(stage + lane * CRB + swz_chunk(lane, cc, CRB) * 16);
    cw[4 * cc] = v.x; cw[4 * cc + 1] = v.y; cw[4 * cc + 2] = v.z; cw[4 * cc + 3] = v.w;
  }
  float y[R];
#pragma unroll
  for (int i = 0; i < R / 8; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[8 * i + e] = nib_f(cw[i], e) * f;
  }
  if (LG) {
    fwht_blocks<R>(y, LG);
#pragma unroll
    for (int i = 0; i < R; ++i) y[i] *= a.inv_sqrt_n;
    unsign<R>(y, a.signs + h * a.dim + part * R);
  }
  wave_lds_sync();   // every lane has read its codes
  stage_row<ODT, R>(stage, lane, y);
  wave_lds_sync();
  unsigned char* ob = (unsigned char*)a.y + seg0 * OROWB;
#pragma unroll
  for (int k = 0; k < OCPR; ++k) {
    const int q = lane + k * 64;
    const int row = q / OCPR, cc = q % OCPR;
    if (row < nvalid) {
      const u32x4 v = *(const u32x4*)(stage + row * OROWB + swz_chunk(row, cc, OROWB) * 16);
      __builtin_nontemporal_store(v, (u32x4*)(ob + row * OROWB + cc * 16));
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int ODT, int R, int LG, bool PT, bool NS = false>
static void dq_mfma_k(const DequantArgs& a, hipStream_t st, int lgL) {
  const int64_t nchunks = (a.seqs * a.heads << lgL) * (a.tokens / 64);
  const int64_t grid = persistent_grid(dequant_mfma<ODT, R, LG, PT, NS>, 256, nchunks);
  const int vec = ((uintptr_t)a.scales & (PT ? 7u : 15u)) == 0 && (!a.norms || ((uintptr_t)a.norms & 7u) == 0) &&
                  (!NS || ((uintptr_t)a.s2 & 7u) == 0);
  hipLaunchKernelGGL((dequant_mfma<ODT, R, LG, PT, NS>), dim3((unsigned)grid), dim3(256), 0, st, a, nchunks, lgL, vec);
}

template <int ODT, int R, int LG>
static void dq_pchan_k(const DequantArgs& a, hipStream_t st) {
  dq_mfma_k<ODT, R, LG, false>(a, st, 0);               // blocks are multiples of 64 tokens
}

template <int ODT, int R, int LG>
static void dq_ptok_k(const DequantArgs& a, hipStream_t st) {
  constexpr int OB = ODT == DT_F32 ? 4 : 2;
  int lgL = 0;
  while ((R << lgL) < a.dim) ++lgL;
  if (a.tokens % 64 == 0 && !rotation_butterfly()) {   // whole 64-token chunks: matrix cores
    dq_mfma_k<ODT, R, LG, true>(a, st, lgL);
    return;
  }
  const int64_t nseg = a.seqs * a.tokens * a.heads * (a.dim / R);
  const int64_t ntiles = (nseg + 63) / 64;
  hipLaunchKernelGGL((dequant_ptok_kernel<ODT, R, LG>), dim3((unsigned)ntiles), dim3(64), (size_t)64 * R * OB, st, a,
                     nseg, ntiles, lgL);
}

template <int ODT, int R, int LG>
static void dq_nsn_k(const DequantArgs& a, hipStream_t st) {
  dq_mfma_k<ODT, R, LG, false, true>(a, st, 0);
}

// compile-time Hadamard size: LG = log2(n) in {0 (none), 4, 5, 6, 7}
template <int ODT, int R, int KIND>    // KIND: 0 per-token, 1 per-channel, 2 NSN
static void dq_by_lg(const DequantArgs& a, hipStream_t st) {
#define KVQ_DQ(LGV) (KIND == 1 ? dq_pchan_k<ODT, R, LGV>(a, st) : KIND == 2 ? dq_nsn_k<ODT, R, LGV>(a, st) : dq_ptok_k<ODT, R, LGV>(a, st))
  switch (a.lg_had) {
    case 0: KVQ_DQ(0); break;
    case 4: KVQ_DQ(4); break;
    case 5: KVQ_DQ(5); break;
    case 6: KVQ_DQ(6); break;
    default: if constexpr (R >= 128) KVQ_DQ(7); break;
  }
#undef KVQ_DQ
}

template <int ODT, int KIND>
static void dq_odt(const DequantArgs& a, hipStream_t st) {
  const bool wide = KIND ? a.dim == 128 : a.dim >= 128;
  if (wide) dq_by_lg<ODT, 128, KIND>(a, st); else dq_by_lg<ODT, 64, KIND>(a, st);
}

template <int KIND>
static hipError_t dq_launch(const DequantArgs& a, hipStream_t st) {
  switch (a.out_dtype) {
    case DT_F16: dq_odt<DT_F16, KIND>(a, st); break;
    case DT_BF16: dq_odt<DT_BF16, KIND>(a, st); break;
    default: dq_odt<DT_F32, KIND>(a, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_dequantize_pchan(const DequantArgs& a, hipStream_t st) { return dq_launch<1>(a, st); }
hipError_t launch_dequantize_ptok(const DequantArgs& a, hipStream_t st) { return dq_launch<0>(a, st); }
hipError_t launch_dequantize_nsn(const DequantArgs& a, hipStream_t st) { return dq_launch<2>(a, st); }

}  // namespace kvq
