// Decode attention scores straight from the packed K cache (gfx950, MFMA).
//
// Method sources (page title, section): NSNQuant summary "implementation details" (scores
// computed from the quantized keys with the stored byproducts folded into the kernel;
// "latency": decoding gets faster because the memory-bound attention reads less);
// Rotated Runtime Smooth analysis "master equation" / "step-by-step flow" (a per-channel
// factor applied to partial products) and Figure 2 (Y = (XR)(R^-1 W^T) = X W^T, so the
// contraction may run in the rotated domain).
//
// scores[s, hq, t] = sum_d q[s,hq,d] k^[s,t,hq/G,d]
//                  = norm[t] * sum_d (R q)[d] * scale[blk(t), d] * code[t, d]
// and for the NSN variant (k^ = s1 (s2 R^T (c scale) + offset); NSNQuant summary, "implementation
// details": the byproducts folded into the score kernel)
//                  = s1[t] s2[t] * sum_d (R q)[d] scale[blk(t), d] code[t, d] + s1[t] (q . offset[blk(t)])
// where q . offset (original domain) is one dot product per unit and query head.
//
// Work: a workgroup takes a chunk of one head-major (sequence, KV head) stream; each wave
// walks units of U tokens (U = the scale block for per-channel modes, 128 otherwise).  The MFMA
// tile is 16 rows x 16 tokens: row i serves query head 4 hc + i / 4 of pass hc, and i % 4 picks
// the part of g = (R q) * scale it carries: bit 0 the fp16 high part hi (the fp32 value truncated
// to 11 significant bits) or the low part 2^10 (g - hi), bit 1 the even or the odd channels (the
// other parity's K slots are zero).  The B operand is 16 tokens x 32 channels of codes as fp16
// subnormals (c + 8) m 2^-24, the nibbles masked in place (m = 1 for even, 16 for odd channels);
// the K order inside a lane is [n0 n4 n1 n5 n2 n6 n3 n7].  Lane (g, j) of the result holds the
// four parts of head 4 hc + g for token j, and sums them with the factors 1, 2^-10, 2^-4, 2^-14.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

__device__ __forceinline__ int nib_of(int e) { return (e >> 1) + ((e & 1) << 2); }

// B operand of the 8 codes of one packed word, slots [n0 n4 | n1 n5 | n2 n6 | n3 n7] (one 32-bit
// word per pair, low half first): the xor turns each two's-complement nibble into c + 8, and the
// nibbles are masked where they sit (bits 0-3 or 4-7 of a 16-bit half, after one 8-bit shift), so
// even channels read (c + 8) 2^-24 and odd channels (c + 8) 16 2^-24, all exact fp16 subnormals
__device__ __forceinline__ u32x4 codes_to_sub16(uint32_t word) {
  // a rotate rather than a shift keeps the bias constant (0x88888888 rotated is itself), so each
  // output is one xor-and of three operands
  const uint32_t ws = __builtin_amdgcn_alignbit(word, word, 8);
  constexpr uint32_t B8 = 0x88888888u;
  return u32x4{(word ^ B8) & 0x000F000Fu, (word ^ B8) & 0x00F000F0u, (ws ^ B8) & 0x000F000Fu, (ws ^ B8) & 0x00F000F0u};
}

constexpr int SCORE_UNITS_PER_BLOCK = 16;

constexpr uint32_t HI_MASK = 0xFFFFE000u;      // fp32 bits that survive truncation to fp16 precision

// U: tokens per unit (the scale block, or 128 per token).  WHOLE: every unit lies inside the stream
// and the fp32 score rows take 16-byte stores (the launcher checks T % U, T % 4 and alignment).
template <int R, bool NS, int U, bool WHOLE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) score_kernel(ScoreArgs a, int64_t ntiles, int64_t nchunks,
                                                    int vec_scales) {
  constexpr int KS = R / 32;               // MFMA K steps of 32 channels
  constexpr int LB = R / 8;                // code bytes per lane and token (lanes 16 g + j: bytes LB g ..)
  constexpr int SROW = U + 16;                              // staged score row (padded: no bank conflicts)
  // rotated queries of this KV head's group: [head][parity][R / 2] (zero past G)
  __shared__ __attribute__((aligned(16))) float qa[16 * R];
  // the rotation's work area, then per wave the scores of one unit and pass: [4 heads][SROW]
  __shared__ __attribute__((aligned(16))) float qs[4 * 4 * SROW > 16 * R ? 4 * 4 * SROW : 16 * R];
  float* const qr = qs;
  __shared__ float qob[NS ? SCORE_UNITS_PER_BLOCK : 1][16];  // NSN: q . offset per (unit, query head)
  __shared__ __attribute__((aligned(16))) uint16_t qh[NS ? 16 * R : 8];   // NSN: fp16 queries (zero rows past G)
  __shared__ float tokf[4][2][256];   // per wave, the unit's tokens: norm 2^24 token-scale s2, and norm
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int G = (int)(a.q_heads / a.heads);
  const int64_t T = a.tokens;

  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t ci = tile % nchunks;
  const int64_t sh = tile / nchunks;                        // head-major stream: s * heads + kvh
  const int64_t kvh = sh % a.heads, s = sh / a.heads;
  const int NHC = (G + 3) / 4;                              // passes of 4 query heads

  // 1. rotated queries R q = (1/sqrt n) H (sigma * q), once per workgroup (butterflies in LDS)
  for (int e = tid; e < G * R; e += 256) {
    const int hh = e / R, d = e % R;
    float v = f16_to_f32(a.q[(s * a.q_heads + kvh * G + hh) * R + d]);
    if (a.lg_had && a.signs[kvh * R + d] < 0) v = -v;
    qr[e] = v;
  }
  __syncthreads();
  for (int st = 0; st < a.lg_had; ++st) {
    const int half = 1 << st;
    for (int p = tid; p < G * R / 2; p += 256) {
      const int hh = p / (R / 2), pp = p % (R / 2);
      const int i = ((pp >> st) << (st + 1)) | (pp & (half - 1));   // index with bit st clear
      const float u = qr[hh * R + i], v = qr[hh * R + i + half];
      qr[hh * R + i] = u + v;
      qr[hh * R + i + half] = u - v;
    }
    __syncthreads();
  }
  // the A-operand table, the channels split by parity
  for (int e = tid; e < 4 * NHC * R; e += 256) {
    const int hh = e / R, d = e % R;
    qa[hh * R + (d & 1) * (R / 2) + (d >> 1)] = hh < G ? (a.lg_had ? qr[e] * a.inv_sqrt_n : qr[e]) : 0.f;
  }

  // NSN: the original-domain fp16 queries, the A operand of q . offset on the matrix cores (row i =
  // query head i of the group, zero rows past G)
  if constexpr (NS)
    for (int e = tid; e < 16 * R; e += 256) qh[e] = e / R < G ? a.q[(s * a.q_heads + kvh * G) * R + e] : (uint16_t)0;
  __syncthreads();

  const int64_t nunits = (T + U - 1) / U;
  const int64_t u_begin = ci * SCORE_UNITS_PER_BLOCK;
  const int64_t u_end = u_begin + SCORE_UNITS_PER_BLOCK < nunits ? u_begin + SCORE_UNITS_PER_BLOCK : nunits;
  const unsigned char* cstream = a.codes + sh * T * (R / 2);
  const int64_t tstream = sh * T;                           // index of the stream's first token
  const int64_t nb = a.per_channel ? T / a.block : 0;
  const uint16_t* nrm_p = a.nsep ? a.norms + tstream : kF16One;              // per-token norms
  const uint16_t* tsc_p = a.per_channel ? kF16One : a.scales + tstream;      // per-token scales

  // NSN: q . offset for every (unit, query head) of the workgroup, all offset loads in flight at
  // once: B holds a unit's offset vector in every column (lane 16 g + j: channels 32 K + 8 g +
  // [0, 8)), so D[i][*] = q_i . offset and lane 16 g (column 0) holds heads 4 g .. 4 g + 3 (exact
  // fp16 products, fp32 sums).  Wave w takes the units it walks below.
  if constexpr (NS) {
    constexpr int UW = SCORE_UNITS_PER_BLOCK / 4;           // units per wave
    u32x4 ov[UW][KS];
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      const int64_t un = u_begin + w + 4 * i;
      const uint16_t* orow = a.offsets + (sh * nb + (un < u_end ? un : u_begin)) * R + 8 * g;
#pragma unroll
      for (int K = 0; K < KS; ++K) {
        if (vec_scales) {                                   // scales and offsets 16-byte aligned
          ov[i][K] = *(const u32x4*)(orow + 32 * K);
        } else {
          uint32_t o4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (uint32_t)orow[32 * K + 2 * e] | ((uint32_t)orow[32 * K + 2 * e + 1] << 16);
          ov[i][K] = u32x4{o4[0], o4[1], o4[2], o4[3]};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      f32x4 qo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < KS; ++K) {
        const f16x8 qv = __builtin_bit_cast(f16x8, *(const u32x4*)(qh + j * R + 32 * K + 8 * g));
        qo = __builtin_amdgcn_mfma_f32_16x16x32_f16(qv, __builtin_bit_cast(f16x8, ov[i][K]), qo, 0, 0, 0);
      }
      if (j == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) qob[w + 4 * i][4 * g + r] = qo[r];
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  }

  // this lane's A row: part (j & 1: hi or 2^10 lo), channel parity p = (j >> 1) & 1
  const int par = (j >> 1) & 1;
  const uint32_t lo_mask = (j & 1) ? HI_MASK : 0u;          // g - (g & mask): g itself, or its low part
  const float part = (j & 1) ? 0x1p10f : 1.f;               // the low part's exact scaling
  float* const stg = qs + w * 4 * SROW;                     // this wave's score staging rows
  const uint32_t keep = par ? 0u : 0xFFFFFFFFu;             // even rows fill words 0, 2; odd rows 1, 3

  // A pass's scores stay in the staging rows until the next pass has issued its first code loads:
  // loads and stores retire in order through one counter, so a store issued before a load would be
  // waited for with it.  With WHOLE units the stores are unconditional and fixed in number (lanes
  // past the pass's last head rewrite that head's row with the same values), so the compiler's
  // counter waits for the next loads do not include them.
  float* pend = nullptr;                                    // head row 0 of the pending pass
  int pend_lim = U - 1, pend_heads = 4;
  auto flush = [&]() {
#pragma unroll
    for (int c = 0; c < U / 64; ++c) {
      const int e = 256 * c + 4 * lane, tk = e % U;
      const int hh = WHOLE ? (e / U < pend_heads ? e / U : pend_heads - 1) : e / U;
      const f32x4 v = *(const f32x4*)(stg + hh * SROW + tk);
      float* op = pend + hh * T + tk;
      if constexpr (WHOLE) {
        __builtin_nontemporal_store(v, (f32x4*)op);
      } else if (hh < pend_heads) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tk + r <= pend_lim) op[r] = v[r];
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  };

  const int64_t first = u_begin + w;
  const int nsteps = first < u_end ? (int)((u_end - first + 3) / 4) * NHC : 0;   // (unit, pass) steps
  float sc[KS][4];
  // one (unit, pass) step; the first step of the wave has no pending scores to write
  auto step = [&](int it, auto flush_tag) {
    constexpr bool FLUSH = decltype(flush_tag)::value;
    const int hc = it % NHC;
    const int64_t un = first + 4 * (it / NHC);
    const int64_t t0 = un * U;
    // A unit's first pass loads its per-token factors (coalesced 2-byte loads by all lanes, token
    // t0 + lane + 64 k clamped to the last token) and the scales of this lane's channels of its
    // parity ((R / 4) g + 8 K + 2 i + par), then every code load of the unit, then the pending
    // stores; only then does it wait, for the factors and scales alone.
    uint16_t nv[4], sv[4], s2v[4];
    uint32_t sraw[KS][4];                                   // scale bits (shifted by sshift)
    const int sshift = vec_scales ? 16 * par : 0;
    if (hc == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t tt = t0 + lane + 64 * k;
        const int64_t tc = tt < T ? tt : T - 1;
        nv[k] = ld_global(nrm_p + (a.nsep ? tc : 0));
        sv[k] = ld_global(tsc_p + (a.per_channel ? 0 : tc));
        if constexpr (NS) s2v[k] = ld_global(a.s2 + tstream + tc);
      }
      if (a.per_channel) {
        const uint16_t* srow = a.scales + (sh * nb + un) * R + (R / 4) * g;
        if (vec_scales) {
#pragma unroll
          for (int K = 0; K < KS; ++K) {
            const u32x4 v = ld_global((const u32x4*)(srow + 8 * K));
            sraw[K][0] = v.x; sraw[K][1] = v.y; sraw[K][2] = v.z; sraw[K][3] = v.w;
          }
        } else {
#pragma unroll
          for (int K = 0; K < KS; ++K)
#pragma unroll
            for (int i = 0; i < 4; ++i) sraw[K][i] = ld_global(srow + 8 * K + 2 * i + par);
        }
      }
    }
    // tokens of this unit past the stream's end read the last token (their scores are not stored)
    const int lim = WHOLE ? U - 1 : (T - t0 < U ? (int)(T - 1 - t0) : U - 1);
    const unsigned char* cu = cstream + t0 * (R / 2) + LB * g;
    // the unit's 16-token groups (ascending, so each group waits only for its own); a whole unit
    // loads at fixed offsets from the lane's token, a partial last unit clamps each token to the
    // stream's last one
    constexpr int NG = U / 16;
    const unsigned char* cj = cu + j * (R / 2);
    uint32_t wd[NG][KS];
#pragma unroll
    for (int b = 0; b < NG; ++b) {
      const uint32_t lt = 16u * b + j;
      const unsigned char* cp = (WHOLE || lim == U - 1) ? cj + 16 * (R / 2) * b
                                                        : cu + (lt < (uint32_t)lim ? lt : (uint32_t)lim) * (R / 2);
      if constexpr (KS == 4) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)cp);
        wd[b][0] = v.x; wd[b][1] = v.y; wd[b][2] = v.z; wd[b][3] = v.w;
      } else {
        const u32x2 v = __builtin_nontemporal_load((const u32x2*)cp);
        wd[b][0] = v.x; wd[b][1] = v.y;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FLUSH) flush();
    __builtin_amdgcn_sched_barrier(0);
    if (hc == 0) {
      if (a.per_channel) {
#pragma unroll
        for (int K = 0; K < KS; ++K)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[K][i] = f16_to_f32((sraw[K][i] >> sshift) & 0xffffu) * part;
      } else {
#pragma unroll
        for (int K = 0; K < KS; ++K)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[K][i] = part;
      }
      // f = norm 2^24 token-scale (s2), f1 = norm (a mode without the value reads the constant 1.0)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (64 * k < U) {
          const float n1 = f16_to_f32(nv[k]);
          float fk = n1 * 0x1p24f * f16_to_f32(sv[k]);
          if constexpr (NS) fk *= f16_to_f32(s2v[k]);
          tokf[w][0][lane + 64 * k] = fk;
          tokf[w][1][lane + 64 * k] = n1;
        }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    }
    // A operand of row j: g (x 2^10 for the low part) of the lane's parity, its high part
    // truncated by the fp16 conversion or its low part left after the mask
    const float* qp = qa + (4 * hc + (j >> 2)) * R + par * (R / 2) + (R / 8) * g;
    f16x8 av[KS];
#pragma unroll
    for (int K = 0; K < KS; ++K) {
      const f32x4 q4 = *(const f32x4*)(qp + 4 * K);
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = q4[i] * sc[K][i];
        v[i] = gv - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, gv) & lo_mask);
      }
      const uint32_t w02 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(v[0], v[2]));
      const uint32_t w13 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(v[1], v[3]));
      av[K] = __builtin_bit_cast(f16x8, u32x4{w02 & keep, w02 & ~keep, w13 & keep, w13 & ~keep});
    }
    // NSN: q . offset of this lane's head for the unit
    float qo = 0.f;
    if constexpr (NS) qo = qob[un - u_begin][4 * hc + g < 16 ? 4 * hc + g : 15];
    // accumulator start: -8 2^-24 sum_k A[i][k] m_k, from one more product with B = m (1 for the
    // even-channel slots, 16 for the odd ones; lane (g, j) receives rows 4 g + r)
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = 0; K < KS; ++K)
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          av[K], __builtin_bit_cast(f16x8, u32x4{0x3C003C00u, 0x4C004C00u, 0x3C003C00u, 0x4C004C00u}), acc0, 0, 0, 0);
    acc0 *= -8.f * 0x1p-24f;
    float* const srow_l = stg + g * SROW + j;               // this lane's head of the pass, token j
#pragma unroll
    for (int b = 0; b < NG; ++b) {
      const float f = tokf[w][0][16 * b + j];
      f32x4 acc = acc0;
#pragma unroll
      for (int K = 0; K < KS; ++K)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[K], __builtin_bit_cast(f16x8, codes_to_sub16(wd[b][K])), acc, 0, 0, 0);
      // rows 4 g + r: even hi, even 2^10 lo, odd 16 hi, odd 16 2^10 lo of head 4 hc + g
      const float sum = __builtin_fmaf(__builtin_fmaf(acc.w, 0x1p-10f, acc.z), 0x1p-4f,
                                       __builtin_fmaf(acc.y, 0x1p-10f, acc.x));
      if constexpr (NS) srow_l[16 * b] = __builtin_fmaf(sum, f, tokf[w][1][16 * b + j] * qo);
      else srow_l[16 * b] = sum * f;
    }
    // this pass's 4 x U scores are written as whole rows (lane l of step c: 4 tokens of one head)
    // once the next pass has its first loads in flight
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    pend = a.scores + (s * a.q_heads + kvh * G + 4 * hc) * T + t0;
    pend_lim = lim;
    pend_heads = G - 4 * hc < 4 ? G - 4 * hc : 4;
  };
  if (nsteps > 0) {
    step(0, std::false_type{});
    for (int it = 1; it < nsteps; ++it) step(it, std::true_type{});
    flush();
  }
}

hipError_t launch_score_decode(const ScoreArgs& a, hipStream_t st) {
  const int U = a.per_channel ? a.block : 128;
  const int64_t nunits = (a.tokens + U - 1) / U;
  const int64_t nchunks = (nunits + SCORE_UNITS_PER_BLOCK - 1) / SCORE_UNITS_PER_BLOCK;
  const int64_t ntiles = a.seqs * a.heads * nchunks;
  const int vec_scales = ((uintptr_t)a.scales & 15u) == 0 && (!a.nsn || ((uintptr_t)a.offsets & 15u) == 0);
  const bool whole = a.tokens % U == 0 && a.tokens % 4 == 0 && ((uintptr_t)a.scores & 15u) == 0;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles, nchunks, vec_scales);
  };
  // per R and NSN flag: the unit size, then whole or partial units
  auto by_u = [&](auto r_tag, auto ns_tag) {
    constexpr int R = decltype(r_tag)::value;
    constexpr bool NS = decltype(ns_tag)::value;
    if (U == 64) {
      if (whole) go(score_kernel<R, NS, 64, true>); else go(score_kernel<R, NS, 64, false>);
    } else if (U == 128) {
      if (whole) go(score_kernel<R, NS, 128, true>); else go(score_kernel<R, NS, 128, false>);
    } else if constexpr (R == 64) {
      if (whole) go(score_kernel<R, NS, 256, true>); else go(score_kernel<R, NS, 256, false>);
    }
  };
  if (a.nsn) {
    if (a.dim == 128) by_u(std::integral_constant<int, 128>{}, std::true_type{});
    else by_u(std::integral_constant<int, 64>{}, std::true_type{});
  } else {
    if (a.dim == 128) by_u(std::integral_constant<int, 128>{}, std::false_type{});
    else by_u(std::integral_constant<int, 64>{}, std::false_type{});
  }
  return hipGetLastError();
}

}  // namespace kvq
