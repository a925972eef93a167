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
// The rotated query times the block's per-channel scales (g, split into an fp16 hi/lo pair)
// is the MFMA A operand (rows = the G query heads of one KV head, padded to 16); the codes
// are the B operand (columns = 16 tokens), converted from nibbles to fp16 with two bit ops
// per pair: (word ^ 0x88888888) >> 4j & 0x000F000F | 0x64006400 is the fp16 pair
// (1032 + c_j, 1032 + c_{j+4}); subtracting 1032 is exact.  The K order inside a lane is
// therefore [n0 n4 n1 n5 n2 n6 n3 n7]; the A operand uses the same order.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

__device__ __forceinline__ int nib_of(int e) { return (e >> 1) + ((e & 1) << 2); }

// fp16x8 B operand (8 codes of one packed word) in [n0 n4 n1 n5 n2 n6 n3 n7] order
__device__ __forceinline__ f16x8 codes_to_f16(uint32_t word) {
  const uint32_t xb = word ^ 0x88888888u;
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t p = ((xb >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
    f16x2 hv = __builtin_bit_cast(f16x2, p);
    hv = hv - f16x2{(_Float16)1032.0f, (_Float16)1032.0f};
    r[2 * j] = hv[0];
    r[2 * j + 1] = hv[1];
  }
  return r;
}

template <int R>
__global__ void __launch_bounds__(256) score_kernel(ScoreArgs a, int64_t ntiles, int64_t nchunks, int chunk) {
  constexpr int KS = R / 32;               // MFMA K steps of 32 channels
  __shared__ float qr[16 * R];             // rotated queries of this KV head's group
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = (int)(a.q_heads / a.heads);

  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t ci = tile % nchunks;
  const int64_t sh = tile / nchunks;
  const int64_t kvh = sh % a.heads, s = sh / a.heads;

  // 1. rotated queries R q = (1/sqrt n) H (sigma * q), once per workgroup
  for (int e = tid; e < G * R; e += 256) {
    const int g = e / R, d = e % R;
    float v = f16_to_f32(a.q[(s * a.q_heads + kvh * G + g) * R + d]);
    if (a.lg_had && a.signs[kvh * R + d] < 0) v = -v;
    qr[e] = v;
  }
  __syncthreads();
  for (int st = 0; st < a.lg_had; ++st) {
    const int half = 1 << st;
    for (int p = tid; p < G * R / 2; p += 256) {
      const int g = p / (R / 2), pp = p % (R / 2);
      const int i = ((pp >> st) << (st + 1)) | (pp & (half - 1));   // index with bit st clear
      const float u = qr[g * R + i], v = qr[g * R + i + half];
      qr[g * R + i] = u + v;
      qr[g * R + i + half] = u - v;
    }
    __syncthreads();
  }

  // 2. this lane's slice of the A operand: row i = lane & 15 (query head), K group lane >> 4
  const int ri = lane & 15, grp = lane >> 4;
  const bool live = ri < G;
  float qv[KS * 8];
#pragma unroll
  for (int sk = 0; sk < KS; ++sk)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      qv[sk * 8 + e] = live ? qr[ri * R + 8 * (KS * grp + sk) + nib_of(e)] * a.inv_sqrt_n : 0.f;

  f16x8 ahi[KS], alo[KS];
  auto build = [&](const uint16_t* sc) {
#pragma unroll
    for (int sk = 0; sk < KS; ++sk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float g = qv[sk * 8 + e];
        if (sc) g *= f16_to_f32(sc[8 * (KS * grp + sk) + nib_of(e)]);
        const _Float16 hi = (_Float16)g;
        ahi[sk][e] = hi;
        alo[sk][e] = (_Float16)(g - (float)hi);
      }
  };
  if (!a.per_channel) build(nullptr);

  const int64_t T = a.tokens;
  const int64_t per_wave = chunk / 4;
  const int64_t t_begin = ci * chunk + w * per_wave;
  int64_t t_end = t_begin + per_wave;
  if (t_end > T) t_end = T;
  const int64_t nb = a.per_channel ? T / a.block : 1;
  int64_t cur = -1;
  const int64_t rowbase = (s * a.heads + kvh) * T;   // head-major (sequence, KV head) stream
  constexpr int CRB = R / 2;

  for (int64_t t0 = t_begin; t0 < t_end; t0 += 64) {
    if (a.per_channel) {
      const int64_t blk = t0 / a.block;
      if (blk != cur) {
        build(a.scales + ((s * a.heads + kvh) * nb + blk) * R);
        cur = blk;
      }
    }
    f32x4 acc[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      acc[tg] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int64_t t = t0 + 16 * tg + (lane & 15);
      uint32_t wd[KS];
      if (t < T) {
        const unsigned char* cp = a.codes + (rowbase + t) * CRB + grp * (KS * 4);
        if constexpr (KS == 4) {
          const u32x4 v = __builtin_nontemporal_load((const u32x4*)cp);
          wd[0] = v.x; wd[1] = v.y; wd[2] = v.z; wd[3] = v.w;
        } else {
          const u32x2 v = __builtin_nontemporal_load((const u32x2*)cp);
          wd[0] = v.x; wd[1] = v.y;
        }
      } else {
#pragma unroll
        for (int k = 0; k < KS; ++k) wd[k] = 0x88888888u;   // code 0
      }
#pragma unroll
      for (int sk = 0; sk < KS; ++sk) {
        const f16x8 b = codes_to_f16(wd[sk]);
        acc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[sk], b, acc[tg], 0, 0, 0);
        acc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[sk], b, acc[tg], 0, 0, 0);
      }
    }
    // 3. epilogue: lane holds D[4*grp + r][lane & 15] = (head 4*grp + r, token lane & 15)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int64_t t = t0 + 16 * tg + (lane & 15);
      if (t >= T) continue;
      float f = 1.f;
      const int64_t rix = rowbase + t;
      if (a.nsep) f = f16_to_f32(a.norms[rix]);
      if (!a.per_channel) f *= f16_to_f32(a.scales[rix]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * grp + r;
        if (i < G) a.scores[((s * a.q_heads + kvh * G + i) * T) + t] = acc[tg][r] * f;
      }
    }
  }
}

hipError_t launch_score_decode(const ScoreArgs& a, hipStream_t st) {
  const int chunk = a.tokens >= 4096 ? 1024 : 256;
  const int64_t nchunks = (a.tokens + chunk - 1) / chunk;
  const int64_t ntiles = a.seqs * a.heads * nchunks;
  if (a.dim == 128)
    hipLaunchKernelGGL((score_kernel<128>), dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles, nchunks, chunk);
  else
    hipLaunchKernelGGL((score_kernel<64>), dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles, nchunks, chunk);
  return hipGetLastError();
}

}  // namespace kvq
