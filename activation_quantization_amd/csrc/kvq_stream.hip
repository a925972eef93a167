// Token copies for the streaming append (gfx950): the cache is a quantized part plus a
// full-precision residual of fewer than B tokens per sequence (NSNQuant summary, "implementation
// details"); new tokens move into the residual, and a residual that fills is quantized by the
// per-channel quantize kernel straight from there.
//
// Both sides are token-major [seqs, tokens, heads, head_dim]: the k tokens of a sequence form one
// contiguous run of k * rowb bytes on each side, so the copy is a plain 16-byte stream.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

// dst_p[s, i] = src_p[s, i] for i < k tokens of rowb bytes (a multiple of 16), for the npairs (1 or
// 2) pairs p; sequence s starts src_seq tokens after sequence s - 1 in src and dst_seq tokens in dst
__global__ void __launch_bounds__(256) copy_tokens(const unsigned char* __restrict__ src0, unsigned char* __restrict__ dst0,
                                                   const unsigned char* __restrict__ src1, unsigned char* __restrict__ dst1,
                                                   int npairs, int64_t total, int64_t per_seq, int64_t src_stride,
                                                   int64_t dst_stride) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < npairs * total; i += step) {
    const bool second = i >= total;
    const int64_t ii = second ? i - total : i;
    const int64_t s = ii / per_seq, o = ii - s * per_seq;
    const unsigned char* src = second ? src1 : src0;
    unsigned char* dst = second ? dst1 : dst0;
    *(u32x4*)(dst + s * dst_stride + 16 * o) = *(const u32x4*)(src + s * src_stride + 16 * o);
  }
}

}  // namespace

hipError_t launch_copy_tokens(const void* const* src, void* const* dst, int npairs, int64_t seqs, int64_t k, int64_t rowb,
                              int64_t src_seq, int64_t dst_seq, hipStream_t st) {
  const int64_t per_seq = k * rowb / 16;                 // 16-byte pieces per sequence
  const int64_t total = seqs * per_seq;
  if (total <= 0 || npairs < 1) return hipSuccess;
  if (npairs > 2) return hipErrorInvalidValue;
  int64_t blocks = (npairs * total + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(copy_tokens, dim3((unsigned)blocks), dim3(256), 0, st, (const unsigned char*)src[0],
                     (unsigned char*)dst[0], (const unsigned char*)src[npairs - 1], (unsigned char*)dst[npairs - 1],
                     npairs, total, per_seq, src_seq * rowb, dst_seq * rowb);
  return hipGetLastError();
}

}  // namespace kvq
