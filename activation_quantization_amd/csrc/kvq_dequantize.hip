// Dequantize kernels for gfx950: unpack nibbles -> code * scale (* norm) -> inverse
// randomized Hadamard -> convert, one pass over HBM.
//
// Method sources (page title, section): norm-separation post "the fix" (direction_q is the
// code times the scale; the norm multiplies back); Rotated Runtime Smooth analysis
// "term-by-term" (R^-1 = R^T); NSNQuant summary "implementation details" (a dedicated
// dequantization kernel that keeps DRAM traffic minimal).
//
// Same layout as quantize: a thread owns one row of R channels in VGPRs; codes come in and
// values go out through XOR-swizzled LDS tiles so both HBM streams are coalesced.
#include "kvq_device.h"
#include "kvq_internal.h"

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
  return (float)((int)((word >> (4 * e)) & 0xfu ^ 8u) - 8);
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
// Per-channel modes: one workgroup of B threads per (sequence, token block, head) tile.
template <int ODT, int R, int LG>
__global__ void __launch_bounds__(256) dequant_pchan_kernel(DequantArgs a, int64_t ntiles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int CRB = R / 2, CCR = CRB / 16;
  constexpr int OB = ODT == DT_F32 ? 4 : 2;
  constexpr int OROWB = R * OB, OCPR = OROWB / 16;
  const int B = a.block;
  const int tid = threadIdx.x;
  unsigned char* stage = smem;

  // tiles numbered along the head-major streams (block fastest)
  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t nb = a.tokens / B;
  const int64_t hs = tile / nb, blk = tile - hs * nb;   // hs = s * heads + h
  const int64_t s = hs / a.heads, h = hs - s * a.heads;
  const int64_t row0 = s * a.tokens + blk * B;
  const int64_t tok0 = hs * a.tokens + blk * B;

  const unsigned char* cbase = a.codes + tok0 * CRB;  // the tile's codes: one contiguous block
#pragma unroll
  for (int k = 0; k < CCR; ++k) {
    const int q = tid + k * B;
    const int row = q / CCR, cc = q % CCR;
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(cbase + q * 16));
    *(u32x4*)(stage + row * CRB + swz_chunk(row, cc, CRB) * 16) = v;
  }
  const float nrm = a.nsep ? f16_to_f32(a.norms[tok0 + tid]) : 1.f;
  __syncthreads();
  uint32_t cw[R / 8];
#pragma unroll
  for (int cc = 0; cc < CCR; ++cc) {
    const u32x4 v = *(const u32x4*)(stage + tid * CRB + swz_chunk(tid, cc, CRB) * 16);
    cw[4 * cc] = v.x; cw[4 * cc + 1] = v.y; cw[4 * cc + 2] = v.z; cw[4 * cc + 3] = v.w;
  }
  __syncthreads();

  const uint16_t* sc = a.scales + (hs * nb + blk) * R;
  float y[R];
#pragma unroll
  for (int i = 0; i < R / 8; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[8 * i + e] = nib_f(cw[i], e) * f16_to_f32(sc[8 * i + e]);
  }
  if (a.nsep) {
#pragma unroll
    for (int i = 0; i < R; ++i) y[i] *= nrm;
  }
  if (LG) {
    fwht_blocks<R>(y, LG);
#pragma unroll
    for (int i = 0; i < R; ++i) y[i] *= a.inv_sqrt_n;
    unsign<R>(y, a.signs + h * R);
  }

  stage_row<ODT, R>(stage, tid, y);
  __syncthreads();
  unsigned char* ob = (unsigned char*)a.y + (row0 * a.heads + h) * OROWB;
#pragma unroll
  for (int k = 0; k < OCPR; ++k) {
    const int q = tid + k * B;
    const int row = q / OCPR, cc = q % OCPR;
    const u32x4 v = *(const u32x4*)(stage + row * OROWB + swz_chunk(row, cc, OROWB) * 16);
    __builtin_nontemporal_store(v, (u32x4*)(ob + (int64_t)row * a.heads * OROWB + cc * 16));
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
template <int ODT, int R, int LG>
static void dq_pchan_k(const DequantArgs& a, hipStream_t st) {
  constexpr int OB = ODT == DT_F32 ? 4 : 2;
  const int64_t ntiles = a.seqs * (a.tokens / a.block) * a.heads;
  const size_t lds = (size_t)a.block * R * OB;     // >= the code tile
  hipLaunchKernelGGL((dequant_pchan_kernel<ODT, R, LG>), dim3((unsigned)ntiles), dim3(a.block), lds, st, a, ntiles);
}

template <int ODT, int R, int LG>
static void dq_ptok_k(const DequantArgs& a, hipStream_t st) {
  constexpr int OB = ODT == DT_F32 ? 4 : 2;
  int lgL = 0;
  while ((R << lgL) < a.dim) ++lgL;
  const int64_t nseg = a.seqs * a.tokens * a.heads * (a.dim / R);
  const int64_t ntiles = (nseg + 63) / 64;
  hipLaunchKernelGGL((dequant_ptok_kernel<ODT, R, LG>), dim3((unsigned)ntiles), dim3(64), (size_t)64 * R * OB, st, a,
                     nseg, ntiles, lgL);
}

// compile-time Hadamard size: LG = log2(n) in {0 (none), 4, 5, 6, 7}
template <int ODT, int R, bool PCHAN>
static void dq_by_lg(const DequantArgs& a, hipStream_t st) {
#define KVQ_DQ(LGV) (PCHAN ? dq_pchan_k<ODT, R, LGV>(a, st) : dq_ptok_k<ODT, R, LGV>(a, st))
  switch (a.lg_had) {
    case 0: KVQ_DQ(0); break;
    case 4: KVQ_DQ(4); break;
    case 5: KVQ_DQ(5); break;
    case 6: KVQ_DQ(6); break;
    default: if constexpr (R >= 128) KVQ_DQ(7); break;
  }
#undef KVQ_DQ
}

template <int ODT, bool PCHAN>
static void dq_odt(const DequantArgs& a, hipStream_t st) {
  const bool wide = PCHAN ? a.dim == 128 : a.dim >= 128;
  if (wide) dq_by_lg<ODT, 128, PCHAN>(a, st); else dq_by_lg<ODT, 64, PCHAN>(a, st);
}

template <bool PCHAN>
static hipError_t dq_launch(const DequantArgs& a, hipStream_t st) {
  switch (a.out_dtype) {
    case DT_F16: dq_odt<DT_F16, PCHAN>(a, st); break;
    case DT_BF16: dq_odt<DT_BF16, PCHAN>(a, st); break;
    default: dq_odt<DT_F32, PCHAN>(a, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_dequantize_pchan(const DequantArgs& a, hipStream_t st) { return dq_launch<true>(a, st); }
hipError_t launch_dequantize_ptok(const DequantArgs& a, hipStream_t st) { return dq_launch<false>(a, st); }

}  // namespace kvq
