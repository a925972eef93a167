// Quantize kernels for gfx950: randomized Hadamard -> norm separation -> absmax scale ->
// round-half-even -> nibble packing, one pass over HBM.
//
// Method sources (page title, section): norm-separation post "the fix" (fp16 L2 norm + unit
// direction, absmax / 7, round and clamp to +-7) and "root cause" (per-row absmax);
// Rotated Runtime Smooth analysis "problem definition" (alpha = max|X| / (2^(N-1)-1)) and
// "term-by-term" (R = (1/sqrt K)[+-1]; runtime scale s_j = max over tokens of column j);
// NSNQuant summary "Hadamard transform" (randomized Hadamard before quantization).
//
// Layout in registers: one thread owns one row of R = min(head_dim, 128) channels of one
// (token, head) and keeps it in VGPRs from load to store, so the 128-point transform needs
// no cross-lane traffic.  Tiles are loaded with coalesced 16-byte loads into LDS and read
// back row-wise through an XOR swizzle; codes leave the same way.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// y[i] <- -y[i] where the sign byte is negative
template <int R>
__device__ __forceinline__ void apply_signs(float (&y)[R], const int8_t* __restrict__ sg) {
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

template <int R>
__device__ __forceinline__ float sum_squares(const float (&y)[R]) {
  float p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = y[k] * y[k];
#pragma unroll
  for (int i = 8; i < R; ++i) p[i & 7] = fmaf(y[i], y[i], p[i & 7]);
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

template <int R>
__device__ __forceinline__ float abs_max(const float (&y)[R]) {
  float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < R; ++i) m[i & 3] = fmaxf(m[i & 3], fabsf(y[i]));
  return fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
}

// code = clamp(rne(u * inv_scale), -q, q) as a two's-complement nibble
__device__ __forceinline__ uint32_t code_nibble(float u, float inv_scale, float q) {
  float v = __builtin_rintf(u * inv_scale);
  v = fminf(fmaxf(v, -q), q);
  return (uint32_t)(int)v & 0xfu;
}

// ---------------------------------------------------------------------------------------
// Per-channel modes (PCHAN, NSEP_PCHAN): one workgroup of B threads per (sequence, token
// block, head) tile; thread t owns token t of the block.
template <int DT, int R>
__global__ void __launch_bounds__(256) quant_pchan_kernel(QuantArgs a, int64_t ntiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int ROWB = R * 2;        // input row bytes
  constexpr int CPR = ROWB / 16;     // input 16-byte chunks per row
  constexpr int CRB = R / 2;         // code row bytes
  constexpr int CCR = CRB / 16;      // code chunks per row
  const int B = a.block;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = B >> 6;
  unsigned char* stage = smem;                                  // B * ROWB
  float* colmax = (float*)(smem + (size_t)B * ROWB);           // nw * R
  float* invs = colmax + nw * R;                                // R

  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t nb = a.tokens / B;
  const int64_t h = tile % a.heads;
  const int64_t sb = tile / a.heads;                            // seq * nb + block
  const int64_t s = sb / nb, blk = sb - s * nb;
  const int64_t row0 = s * a.tokens + blk * B;
  const int64_t tok_stride = a.heads * ROWB;                    // bytes between tokens
  const unsigned char* xb = (const unsigned char*)a.x + (row0 * a.heads + h) * ROWB;

  // 1. coalesced tile load -> LDS
#pragma unroll
  for (int k = 0; k < CPR; ++k) {
    const int q = tid + k * B;
    const int row = q / CPR, cc = q % CPR;
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(xb + row * tok_stride + cc * 16));
    *(u32x4*)(stage + row * ROWB + swz_chunk(row, cc, ROWB) * 16) = v;
  }
  __syncthreads();
  float y[R];
#pragma unroll
  for (int cc = 0; cc < CPR; ++cc) {
    const u32x4 v = *(const u32x4*)(stage + tid * ROWB + swz_chunk(tid, cc, ROWB) * 16);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y[8 * cc + 2 * j] = lo_f32<DT>(wv[j]);
      y[8 * cc + 2 * j + 1] = hi_f32<DT>(wv[j]);
    }
  }
  __syncthreads();   // the staging buffer is free from here on

  // 2. randomized Hadamard rotation (orthonormal)
  if (a.lg_had) {
    apply_signs<R>(y, a.signs + h * R);
    fwht_blocks<R>(y, a.lg_had);
#pragma unroll
    for (int i = 0; i < R; ++i) y[i] *= a.inv_sqrt_n;
  }

  // 3. norm separation
  if (a.nsep) {
    const float nu = sqrtf(sum_squares<R>(y));
    const float inv_nu = nu > 0.f ? 1.f / nu : 0.f;
    a.norms[(row0 + tid) * a.heads + h] = (uint16_t)f32_to_f16(nu);
#pragma unroll
    for (int i = 0; i < R; ++i) y[i] *= inv_nu;
  }

  // 4. per-channel absmax over the B tokens: each wave transposes 16 channels at a time
  //    through a 4 KiB LDS scratch (64 tokens x 16 fp32), reduces 16 tokens per lane and
  //    finishes across the 4 lane groups with two lane shuffles.
  float* scr = (float*)(stage + w * 4096);
  const int ch = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int j = 0; j < R / 16; ++j) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 v = {y[16 * j + 4 * jj], y[16 * j + 4 * jj + 1], y[16 * j + 4 * jj + 2], y[16 * j + 4 * jj + 3]};
      *(f32x4*)(scr + lane * 16 + 4 * (jj ^ ((lane >> 2) & 3))) = v;
    }
    wave_lds_sync();
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int t = 4 * k + grp;   // (t >> 2) & 3 == k & 3
      m = fmaxf(m, fabsf(scr[t * 16 + 4 * ((ch >> 2) ^ (k & 3)) + (ch & 3)]));
    }
    m = fmaxf(m, shfl_xor_f(m, 16));
    m = fmaxf(m, shfl_xor_f(m, 32));
    if (lane < 16) colmax[w * R + 16 * j + lane] = m;
    wave_lds_sync();
  }
  __syncthreads();
  for (int c = tid; c < R; c += B) {
    float m = colmax[c];
    for (int ww = 1; ww < nw; ++ww) m = fmaxf(m, colmax[ww * R + c]);
    invs[c] = m > 0.f ? a.q / m : 0.f;
    a.scales[(sb * a.heads + h) * R + c] = (uint16_t)f32_to_f16(m / a.q);
  }
  __syncthreads();

  // 5. codes, staged through LDS for coalesced 16-byte stores
  uint32_t cw[R / 8];
#pragma unroll
  for (int i = 0; i < R / 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= code_nibble(y[8 * i + e], invs[8 * i + e], a.q) << (4 * e);
    cw[i] = word;
  }
#pragma unroll
  for (int cc = 0; cc < CCR; ++cc) {
    const u32x4 v = {cw[4 * cc], cw[4 * cc + 1], cw[4 * cc + 2], cw[4 * cc + 3]};
    *(u32x4*)(stage + tid * CRB + swz_chunk(tid, cc, CRB) * 16) = v;
  }
  __syncthreads();
  unsigned char* cb = a.codes + (row0 * a.heads + h) * CRB;
#pragma unroll
  for (int k = 0; k < CCR; ++k) {
    const int q = tid + k * B;
    const int row = q / CCR, cc = q % CCR;
    const u32x4 v = *(const u32x4*)(stage + row * CRB + swz_chunk(row, cc, CRB) * 16);
    __builtin_nontemporal_store(v, (u32x4*)(cb + (int64_t)row * a.heads * CRB + cc * 16));
  }
}

// ---------------------------------------------------------------------------------------
// Per-token modes (NAIVE, NSEP): one wave per 64 consecutive row segments of R channels.
// A (token, head) vector of D = L * R channels spans L = 2^lgL neighbouring lanes.
template <int DT, int R>
__global__ void __launch_bounds__(64) quant_ptok_kernel(QuantArgs a, int64_t nseg, int64_t ntiles, int lgL) {
  constexpr int ROWB = R * 2, CPR = ROWB / 16, CRB = R / 2, CCR = CRB / 16;
  __shared__ __attribute__((aligned(16))) unsigned char stage[64 * ROWB];
  const int lane = threadIdx.x;
  const int64_t seg0 = xcd_tile(blockIdx.x, ntiles) * 64;
  const int nvalid = (int)(nseg - seg0 < 64 ? nseg - seg0 : 64);
  const unsigned char* xb = (const unsigned char*)a.x + seg0 * ROWB;

#pragma unroll
  for (int k = 0; k < CPR; ++k) {
    const int q = lane + k * 64;
    const int row = q / CPR, cc = q % CPR;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < nvalid) v = __builtin_nontemporal_load((const u32x4*)(xb + row * ROWB + cc * 16));
    *(u32x4*)(stage + row * ROWB + swz_chunk(row, cc, ROWB) * 16) = v;
  }
  wave_lds_sync();
  float y[R];
#pragma unroll
  for (int cc = 0; cc < CPR; ++cc) {
    const u32x4 v = *(const u32x4*)(stage + lane * ROWB + swz_chunk(lane, cc, ROWB) * 16);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y[8 * cc + 2 * j] = lo_f32<DT>(wv[j]);
      y[8 * cc + 2 * j + 1] = hi_f32<DT>(wv[j]);
    }
  }
  const int L = 1 << lgL;
  const int64_t seg = seg0 + lane;
  const int64_t vec = seg >> lgL;
  const int part = (int)(seg & (L - 1));
  const int64_t h = vec % a.heads;

  if (a.lg_had) {
    apply_signs<R>(y, a.signs + h * a.dim + part * R);
    fwht_blocks<R>(y, a.lg_had);
#pragma unroll
    for (int i = 0; i < R; ++i) y[i] *= a.inv_sqrt_n;
  }
  float nu = 0.f;
  if (a.nsep) {
    float ss = sum_squares<R>(y);
    for (int o = 1; o < L; o <<= 1) ss += shfl_xor_f(ss, o);
    nu = sqrtf(ss);
    const float inv_nu = nu > 0.f ? 1.f / nu : 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) y[i] *= inv_nu;
  }
  float m = abs_max<R>(y);
  for (int o = 1; o < L; o <<= 1) m = fmaxf(m, shfl_xor_f(m, o));
  const float inv_scale = m > 0.f ? a.q / m : 0.f;

  uint32_t cw[R / 8];
#pragma unroll
  for (int i = 0; i < R / 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= code_nibble(y[8 * i + e], inv_scale, a.q) << (4 * e);
    cw[i] = word;
  }
  wave_lds_sync();   // every lane has read its input row
#pragma unroll
  for (int cc = 0; cc < CCR; ++cc) {
    const u32x4 v = {cw[4 * cc], cw[4 * cc + 1], cw[4 * cc + 2], cw[4 * cc + 3]};
    *(u32x4*)(stage + lane * CRB + swz_chunk(lane, cc, CRB) * 16) = v;
  }
  wave_lds_sync();
  unsigned char* cb = a.codes + seg0 * CRB;
#pragma unroll
  for (int k = 0; k < CCR; ++k) {
    const int q = lane + k * 64;
    const int row = q / CCR, cc = q % CCR;
    if (row < nvalid) {
      const u32x4 v = *(const u32x4*)(stage + row * CRB + swz_chunk(row, cc, CRB) * 16);
      __builtin_nontemporal_store(v, (u32x4*)(cb + row * CRB + cc * 16));
    }
  }
  if (part == 0 && lane < nvalid) {
    if (a.nsep) a.norms[vec] = (uint16_t)f32_to_f16(nu);
    a.scales[vec] = (uint16_t)f32_to_f16(m / a.q);
  }
}

// ---------------------------------------------------------------------------------------
template <int DT>
static hipError_t launch_pchan_dt(const QuantArgs& a, hipStream_t st) {
  const int64_t ntiles = a.seqs * (a.tokens / a.block) * a.heads;
  const int nw = a.block / 64;
  if (a.dim == 128) {
    const size_t lds = (size_t)a.block * 256 + (size_t)nw * 128 * 4 + 128 * 4;
    hipLaunchKernelGGL((quant_pchan_kernel<DT, 128>), dim3((unsigned)ntiles), dim3(a.block), lds, st, a, ntiles);
  } else {
    const size_t lds = (size_t)a.block * 128 + (size_t)nw * 64 * 4 + 64 * 4;
    hipLaunchKernelGGL((quant_pchan_kernel<DT, 64>), dim3((unsigned)ntiles), dim3(a.block), lds, st, a, ntiles);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_pchan(const QuantArgs& a, hipStream_t st) {
  return a.dtype == DT_F16 ? launch_pchan_dt<DT_F16>(a, st) : launch_pchan_dt<DT_BF16>(a, st);
}

template <int DT>
static hipError_t launch_ptok_dt(const QuantArgs& a, hipStream_t st) {
  const int R = a.dim >= 128 ? 128 : 64;
  int lgL = 0;
  while ((R << lgL) < a.dim) ++lgL;
  const int64_t nseg = a.seqs * a.tokens * a.heads * (a.dim / R);
  const int64_t ntiles = (nseg + 63) / 64;
  if (R == 128)
    hipLaunchKernelGGL((quant_ptok_kernel<DT, 128>), dim3((unsigned)ntiles), dim3(64), 0, st, a, nseg, ntiles, lgL);
  else
    hipLaunchKernelGGL((quant_ptok_kernel<DT, 64>), dim3((unsigned)ntiles), dim3(64), 0, st, a, nseg, ntiles, lgL);
  return hipGetLastError();
}

hipError_t launch_quantize_ptok(const QuantArgs& a, hipStream_t st) {
  return a.dtype == DT_F16 ? launch_ptok_dt<DT_F16>(a, st) : launch_ptok_dt<DT_BF16>(a, st);
}

}  // namespace kvq
