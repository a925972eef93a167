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
// The statistics (two token norms, the block's channel means and maxima) are taken in fp64, so the
// codes are the same rounding decisions as the fp64 definition without a near-tie path: fp16 inputs
// rotate exactly in fp64, and what differs is summation order at the 2^-53 level.
//
// Layout: one workgroup of 2 B threads per tile (one sequence, one head, B tokens); thread
// 2 t + half holds channels [half D/2, half D/2 + D/2) of token t in registers.  When the rotation
// spans the whole row, its top butterfly stage pairs channel c with c + D/2: each thread reads the
// whole row and forms its half of that stage directly (the stages commute), so no exchange is
// needed.  Column statistics over the block's tokens reduce across the lanes of equal parity,
// then across waves through LDS.
#include "kvq_device.h"
#include "kvq_internal.h"

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

// sum (MAX = false) or maximum over the lanes of equal parity (the threads holding the same
// channels of different tokens) of one wave
template <bool MAX>
__device__ __forceinline__ double parity_reduce(double x) {
#pragma unroll
  for (int m = 2; m < 64; m <<= 1) {
    const double y = __shfl_xor(x, m);
    x = MAX ? fmax(x, y) : x + y;
  }
  return x;
}

template <int DT, int D, int LG, int B>
__global__ void __launch_bounds__(2 * B) quant_nsn_tile(NsnArgs a, int64_t ntiles) {
  constexpr int RH = D / 2, NW = 2 * B / 64, LGD = D == 128 ? 7 : 6;
  constexpr bool CROSS = LG == LGD;                    // the rotation's top stage crosses the halves
  __shared__ double part[NW][D];                       // per-wave column sums / maxima
  __shared__ double mean[D];                           // the block's column mean of u1
  __shared__ double col[D];                            // the block's column scale
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = tid & 1, t = tid >> 1;
  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t nb = a.tokens / B, hs = tile / nb, blk = tile - hs * nb;
  const int64_t seq = hs / a.heads, h = hs - seq * a.heads;
  const uint16_t* xr = (const uint16_t*)a.x + ((seq * a.tokens + blk * B + t) * a.heads + h) * D;
  const int8_t* sg = LG ? a.signs + h * D : nullptr;
  const int c0 = half * RH;
  auto ld = [&](int c) -> double {
    const uint32_t b = xr[c];
    double v = DT == DT_F16 ? (double)f16_to_f32(b) : (double)bf16_to_f32(b);
    if (LG != 0 && sg[c] < 0) v = -v;
    return v;
  };

  // 1. y = R x on this thread's half row (exact for fp16 inputs), then / sqrt(n)
  double v[RH];
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    if constexpr (CROSS) {
      const double own = ld(c0 + i), oth = ld((c0 ^ RH) + i);
      v[i] = half == 0 ? own + oth : oth - own;
    } else {
      v[i] = ld(c0 + i);
    }
  }
  fwht64<RH>(v, CROSS ? LG - 1 : LG);
  if (LG) {
    const double rn = sqrt((double)(1 << LG));
#pragma unroll
    for (int i = 0; i < RH; ++i) v[i] /= rn;
  }
  const double rd = sqrt((double)D);

  // 2. s1 = ||y|| / sqrt(D), u1 = y / s1
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < RH; ++i) ss = __builtin_fma(v[i], v[i], ss);
  ss += __shfl_xor(ss, 1);
  const double s1 = sqrt(ss) / rd;
#pragma unroll
  for (int i = 0; i < RH; ++i) v[i] = s1 > 0.0 ? v[i] / s1 : 0.0;

  // 3. o = the block's channel means of u1
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    const double r = parity_reduce<false>(v[i]);
    if (lane < 2) part[w][c0 + i] = r;
  }
  __syncthreads();
  if (tid < D) {
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < NW; ++k) sum += part[k][tid];
    mean[tid] = sum / (double)B;
  }
  __syncthreads();

  // 4. u2 = u1 - o, s2 = ||u2|| / sqrt(D) (0 when ||u2|| < 2^-16 sqrt(D)), u3 = u2 / s2
  double ss2 = 0.0;
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    v[i] -= mean[c0 + i];
    ss2 = __builtin_fma(v[i], v[i], ss2);
  }
  ss2 += __shfl_xor(ss2, 1);
  const double n2 = sqrt(ss2);
  const double s2 = n2 < 0x1p-16 * rd ? 0.0 : n2 / rd;
#pragma unroll
  for (int i = 0; i < RH; ++i) v[i] = s2 > 0.0 ? v[i] / s2 : 0.0;

  // 5. per-channel absmax of u3 over the block, scale = amax / Q
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    const double r = parity_reduce<true>(fabs(v[i]));
    if (lane < 2) part[w][c0 + i] = r;
  }
  __syncthreads();
  if (tid < D) {
    double m = 0.0;
#pragma unroll
    for (int k = 0; k < NW; ++k) m = fmax(m, part[k][tid]);
    const double sc = m / (double)a.q;
    col[tid] = sc;
    a.scales[(hs * nb + blk) * D + tid] = (uint16_t)f32_to_f16((float)sc);
  }
  __syncthreads();

  // 6. codes c = rne(fp32(u3 / scale)), packed two per byte; the token scales
  uint32_t cw[RH / 8];
#pragma unroll
  for (int k = 0; k < RH / 8; ++k) cw[k] = 0u;
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    const double sc = col[c0 + i];
    int c = sc > 0.0 ? (int)__builtin_rintf((float)(v[i] / sc)) : 0;
    c = c > a.q ? a.q : (c < -a.q ? -a.q : c);
    cw[i >> 3] |= ((uint32_t)c & 0xFu) << (4 * (i & 7));
  }
  const int64_t tok = hs * a.tokens + blk * B + t;     // head-major token index
  uint32_t* cp = (uint32_t*)(a.codes + tok * (D / 2) + c0 / 2);
#pragma unroll
  for (int k = 0; k < RH / 8; ++k) cp[k] = cw[k];
  if (half == 0) {
    a.s1[tok] = (uint16_t)f32_to_f16((float)s1);
    a.s2[tok] = (uint16_t)f32_to_f16((float)s2);
  }

  // 7. the offset R^T o (original domain) of this block: threads 0 and 1 (token 0), from mean[]
  if (t == 0) {
    double of[RH];
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      if constexpr (CROSS) {
        const double own = mean[c0 + i], oth = mean[(c0 ^ RH) + i];
        of[i] = half == 0 ? own + oth : oth - own;
      } else {
        of[i] = mean[c0 + i];
      }
    }
    fwht64<RH>(of, CROSS ? LG - 1 : LG);
    uint16_t* op = a.offsets + (hs * nb + blk) * D + c0;
    const double rn = sqrt((double)(1 << LG));
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      double x = of[i];
      if (LG) {
        x /= rn;
        if (sg[c0 + i] < 0) x = -x;
      }
      op[i] = (uint16_t)f32_to_f16((float)x);
    }
  }
}

template <int DT, int D, int LG, int B>
void launch_nsn_k(const NsnArgs& a, hipStream_t st) {
  const int64_t ntiles = a.seqs * (a.tokens / B) * a.heads;
  hipLaunchKernelGGL((quant_nsn_tile<DT, D, LG, B>), dim3((unsigned)ntiles), dim3(2 * B), 0, st, a, ntiles);
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
