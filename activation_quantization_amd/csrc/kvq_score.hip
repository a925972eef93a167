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
// walks units of U tokens (U = the scale block for per-channel modes, 128 otherwise).  Per unit
// the wave issues all of its loads at once (16 bytes of codes per lane and 16-token group, the
// unit's scale row, the norms), then builds the MFMA A operand: g = (R q) * scale in fp32, split
// into an fp16 hi/lo pair, rows 2 h + {0, 1} = (hi, lo) of query head h (8 heads per pass).
// The B operand is 16 tokens x 32 channels of codes as fp16 subnormals (c + 8) 2^-24 (two bit
// operations per pair); the K order inside a lane is [n0 n4 n1 n5 n2 n6 n3 n7] and the A
// operand uses the same order.  Lane (g, j) of the
// result holds rows 4 g + r: heads 2 g and 2 g + 1 (hi and lo rows summed) of token j.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

__device__ __forceinline__ int nib_of(int e) { return (e >> 1) + ((e & 1) << 2); }

// B operand of the 8 codes of one packed word, in [n0 n4 n1 n5 n2 n6 n3 n7] order, as the fp16
// subnormals (c + 8) 2^-24: (word ^ 0x88888888) >> 4 q & 0x000F000F is the pair (c_q + 8,
// c_{q+4} + 8) in the mantissa bits, exact.  The bias 8 leaves through the accumulator's start
// value (-8 2^-24 times the row sums of A) and 2^24 through the epilogue factor.
__device__ __forceinline__ u32x4 codes_to_sub16(uint32_t word) {
  const uint32_t xb = word ^ 0x88888888u;
  return u32x4{xb & 0x000F000Fu, (xb >> 4) & 0x000F000Fu, (xb >> 8) & 0x000F000Fu, (xb >> 12) & 0x000F000Fu};
}

constexpr int SCORE_UNITS_PER_BLOCK = 16;


template <int R, bool NS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) score_kernel(ScoreArgs a, int64_t ntiles, int64_t nchunks, int U,
                                                    int vec_scales) {
  constexpr int KS = R / 32;               // MFMA K steps of 32 channels
  constexpr int LB = R / 8;                // code bytes per lane and token (lanes 16 g + j: bytes LB g ..)
  __shared__ __attribute__((aligned(16))) float qr[16 * R];   // rotated queries of this KV head's group
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
  if (a.lg_had) {
    for (int e = tid; e < G * R; e += 256) qr[e] *= a.inv_sqrt_n;
    __syncthreads();
  }

  // NSN: the original-domain fp16 queries, the A operand of q . offset on the matrix cores (row i =
  // query head i of the group, zero rows past G)
  if constexpr (NS) {
    for (int e = tid; e < 16 * R; e += 256) qh[e] = e / R < G ? a.q[(s * a.q_heads + kvh * G) * R + e] : (uint16_t)0;
    __syncthreads();
  }

  const int NHC = (G + 7) / 8;                              // passes of 8 query heads
  const int64_t nunits = (T + U - 1) / U;
  const int64_t u_begin = ci * SCORE_UNITS_PER_BLOCK;
  const int64_t u_end = u_begin + SCORE_UNITS_PER_BLOCK < nunits ? u_begin + SCORE_UNITS_PER_BLOCK : nunits;
  const unsigned char* cstream = a.codes + sh * T * (R / 2);
  const int64_t tstream = sh * T;                           // index of the stream's first token
  const int64_t nb = a.per_channel ? T / a.block : 0;
  const int ngr = U / 16;                                   // 16-token groups per unit
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
        const f16x8 qa = __builtin_bit_cast(f16x8, *(const u32x4*)(qh + j * R + 32 * K + 8 * g));
        qo = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, __builtin_bit_cast(f16x8, ov[i][K]), qo, 0, 0, 0);
      }
      if (j == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) qob[w + 4 * i][4 * g + r] = qo[r];
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  }

  for (int64_t un = u_begin + w; un < u_end; un += 4) {
    const int64_t t0 = un * U;
    // the unit's per-token factors: coalesced 2-byte loads by all lanes (token t0 + lane + 64 k,
    // clamped to the last token), issued before the scale loads, into this wave's LDS table
    uint16_t nv[4], sv[4], s2v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t tt = t0 + lane + 64 * k;
      const int64_t tc = tt < T ? tt : T - 1;
      nv[k] = nrm_p[a.nsep ? tc : 0];
      sv[k] = tsc_p[a.per_channel ? 0 : tc];
      if constexpr (NS) s2v[k] = a.s2[tstream + tc];
    }
    // scales of this lane's channels (LB g .. as fp16), loaded with the unit
    float sc[KS * 8];
    if (a.per_channel) {
      const uint16_t* srow = a.scales + (sh * nb + un) * R + (R / 4) * g;
      if (vec_scales) {
#pragma unroll
        for (int K = 0; K < KS; ++K) {
          const u32x4 v = *(const u32x4*)(srow + 8 * K);
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int n = nib_of(e);
            sc[8 * K + e] = f16_to_f32((n & 1) ? wv[n >> 1] >> 16 : wv[n >> 1] & 0xffffu);
          }
        }
      } else {
#pragma unroll
        for (int K = 0; K < KS; ++K)
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[8 * K + e] = f16_to_f32(srow[8 * K + nib_of(e)]);
      }
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
    for (int hc = 0; hc < NHC; ++hc) {
      // A operand: row i = lane & 15 -> head hc 8 + i / 2, hi (i even) or lo (i odd) part
      const int hl = hc * 8 + (j >> 1);
      const bool live = hl < G;
      f16x8 av[KS];
#pragma unroll
      for (int K = 0; K < KS; ++K) {
        const float* qp = qr + hl * R + (R / 4) * g + 8 * K;   // inside qr even when not live
        const f32x4 q0 = *(const f32x4*)qp, q1 = *(const f32x4*)(qp + 4);
        // rows of even j take hi = fp16(g), odd j take lo = fp16(g - hi); hi + lo = g to ~2^-21
        // relative with any rounding, so the packed round-toward-zero conversion serves
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int n0 = nib_of(e), n1 = nib_of(e + 1);
          float g0 = n0 < 4 ? q0[n0] : q1[n0 - 4], g1 = n1 < 4 ? q0[n1] : q1[n1 - 4];
          if (a.per_channel) {
            g0 *= sc[8 * K + e];
            g1 *= sc[8 * K + e + 1];
          }
          const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(g0, g1));
          const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(g0 - (float)hi[0], g1 - (float)hi[1]));
          const f16x2 pv = live ? ((j & 1) ? lo : hi) : f16x2{(_Float16)0.f, (_Float16)0.f};
          av[K][e] = pv[0];
          av[K][e + 1] = pv[1];
        }
      }
      // NSN: q . offset of this lane's two heads for the unit
      float qo0 = 0.f, qo1 = 0.f;
      if constexpr (NS) {
        const int h0 = hc * 8 + 2 * g;
        qo0 = qob[un - u_begin][h0 < 16 ? h0 : 15];
        qo1 = qob[un - u_begin][h0 + 1 < 16 ? h0 + 1 : 15];
      }
      // accumulator start: -8 2^-24 sum_k A[i][k], from one more product with B = ones (lane (g, j)
      // receives rows 4 g + r)
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < KS; ++K)
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            av[K], __builtin_bit_cast(f16x8, u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}), acc0, 0, 0, 0);
      acc0 *= -8.f * 0x1p-24f;
      // 16-token groups, four at a time: every load of the four first, then the products
      for (int gr0 = 0; gr0 < ngr; gr0 += 4) {
        uint32_t wd[4][KS];
        float f[4], f1[4];
        // the four groups' code loads are all issued before any is used (a token past the end
        // reads the last token; its scores are not stored)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t t = t0 + 16 * (gr0 + b) + j;
          const int64_t tc = t < T ? t : T - 1;
          const unsigned char* cp = cstream + tc * (R / 2) + LB * g;
          if constexpr (KS == 4) {
            const u32x4 v = __builtin_nontemporal_load((const u32x4*)cp);
            wd[b][0] = v.x; wd[b][1] = v.y; wd[b][2] = v.z; wd[b][3] = v.w;
          } else {
            const u32x2 v = __builtin_nontemporal_load((const u32x2*)cp);
            wd[b][0] = v.x; wd[b][1] = v.y;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          f[b] = tokf[w][0][16 * (gr0 + b) + j];
          f1[b] = tokf[w][1][16 * (gr0 + b) + j];
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t t = t0 + 16 * (gr0 + b) + j;
          f32x4 acc = acc0;
#pragma unroll
          for (int K = 0; K < KS; ++K)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[K], __builtin_bit_cast(f16x8, codes_to_sub16(wd[b][K])), acc, 0, 0, 0);
          // rows 4 g + r: (head 2 g, hi), (2 g, lo), (2 g + 1, hi), (2 g + 1, lo) of this pass
          if (t < T) {
            const int h0 = hc * 8 + 2 * g;
            float* sp = a.scores + (s * a.q_heads + kvh * G + h0) * T + t;
            if constexpr (NS) {
              if (h0 < G) sp[0] = __builtin_fmaf(acc.x + acc.y, f[b], f1[b] * qo0);
              if (h0 + 1 < G) sp[T] = __builtin_fmaf(acc.z + acc.w, f[b], f1[b] * qo1);
            } else {
              if (h0 < G) sp[0] = (acc.x + acc.y) * f[b];
              if (h0 + 1 < G) sp[T] = (acc.z + acc.w) * f[b];
            }
          }
        }
      }
    }
  }
}

hipError_t launch_score_decode(const ScoreArgs& a, hipStream_t st) {
  const int U = a.per_channel ? a.block : 128;
  const int64_t nunits = (a.tokens + U - 1) / U;
  const int64_t nchunks = (nunits + SCORE_UNITS_PER_BLOCK - 1) / SCORE_UNITS_PER_BLOCK;
  const int64_t ntiles = a.seqs * a.heads * nchunks;
  const int vec_scales = ((uintptr_t)a.scales & 15u) == 0 && (!a.nsn || ((uintptr_t)a.offsets & 15u) == 0);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles, nchunks, U, vec_scales);
  };
  if (a.nsn) {
    if (a.dim == 128) go(score_kernel<128, true>); else go(score_kernel<64, true>);
  } else {
    if (a.dim == 128) go(score_kernel<128, false>); else go(score_kernel<64, false>);
  }
  return hipGetLastError();
}

}  // namespace kvq
