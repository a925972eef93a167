// Device-side building blocks shared by the gfx950 kernels (HIP, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}
// low / high 16-bit element of a packed pair -> fp32
template <int DT> __device__ __forceinline__ float lo_f32(uint32_t w) {
  if constexpr (DT == DT_F16) return f16_to_f32(w & 0xffffu);
  else return __builtin_bit_cast(float, w << 16);
}
template <int DT> __device__ __forceinline__ float hi_f32(uint32_t w) {
  if constexpr (DT == DT_F16) return f16_to_f32(w >> 16);
  else return __builtin_bit_cast(float, w & 0xffff0000u);
}
// fp32 -> fp16 bits, round to nearest even (hardware default rounding mode)
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// two fp32 -> one word of two fp16 / bf16 (a low), round to nearest even: one packed
// conversion instruction on gfx950
template <int DT> __device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == DT_F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, b2{(__bf16)a, (__bf16)b});
  }
}

// ------------------------------------------------------------------ launch geometry
// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs (each with its
// own L2).  Remap so that every XCD walks a contiguous range of tiles: neighbouring tiles
// (which share cache lines of the codes, norms and scales outputs) then run on one L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t n) {
  const int64_t x = bid & 7, k = bid >> 3;
  const int64_t per = n >> 3, rem = n & 7;
  return x * per + (x < rem ? x : rem) + k;
}

// Outputs are head-major: the (token, head) vector at x row `row` = s T + t, head h (x index
// row * heads + h) is entry (s heads + h) T + t of the codes / norms / scales streams.
__device__ __forceinline__ int64_t head_major(int64_t heads, int64_t tokens, int64_t vec) {
  if (heads == 1) return vec;
  const int64_t h = vec % heads, row = vec / heads;
  const int64_t s = row / tokens;
  return (s * heads + h) * tokens + (row - s * tokens);
}

// 16-byte-chunk XOR swizzle for LDS tiles of `row_bytes` per row (power of two, >= 16):
// consecutive rows land on different bank groups for both row-wise and chunk-wise access.
__device__ __forceinline__ int swz_chunk(int row, int cc, int row_bytes) {
  const int cpr = row_bytes >> 4;                         // chunks per row
  const int rows_per_256 = row_bytes >= 256 ? 1 : 256 / row_bytes;
  return cc ^ ((row / rows_per_256) & (cpr - 1));
}

// ------------------------------------------------------------------ wave helpers
// Orders this wave's LDS accesses.  LDS executes one wave's instructions in order, so only
// the compiler must be kept from reordering; no memory fence (a fence would also wait for
// every global access in flight, the asynchronous tile prefetch included).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}
// Workgroup barrier for LDS data only: waits for this wave's LDS operations, then s_barrier.
// Global loads in flight (the prefetch into a different LDS array) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ float shfl_xor_f(float v, int m) {
  const int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float shfl_f(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

// fp16 1.0: the per-token norm or scale of a mode that has none, read like a real one (no branch
// between the load and its use)
static __device__ const uint16_t kF16One[1] = {0x3C00u};
// four fp16 ones, 8-byte aligned: the per-token factors of a mode that stores none
// cache policy of an LDS-DMA load (global_load_lds) that streams data read exactly once: the
// nontemporal bit (encoded where older targets kept SLC)
constexpr int KVQ_LOAD_NT = 2;
static __device__ __attribute__((aligned(8))) const uint16_t kF16Ones4[4] = {0x3C00u, 0x3C00u, 0x3C00u, 0x3C00u};

// A load through a global-address-space pointer.  A pointer that may be a kernel argument or a
// device constant is generic to the compiler, and a load through it is a flat load, which the
// compiler can only wait for together with every other load and store in flight.
template <typename V>
__device__ __forceinline__ V ld_global(const V* p) {
  return *(const __attribute__((address_space(1))) V*)p;
}

// ------------------------------------------------------------------ code packing
// Codes by one fma into [128, 256), where the fp32 ulp is 2^-16: b = bits(v + 136.5) has code + 8
// in byte 2 (v rounded half up), and b & 0xffff == 0 marks a value within 2^-17 of a tie.
constexpr float CODE_MAGIC = 136.5f;

__device__ __forceinline__ uint32_t min3_u16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_min3_u16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// 8 magic-biased codes (channels 8d .. 8d + 7) -> one packed word
__device__ __forceinline__ uint32_t pack8(const uint32_t (&b)[8]) {
  const uint32_t ev = __builtin_amdgcn_perm(b[2], b[0], 0x0C0C0602u) | __builtin_amdgcn_perm(b[6], b[4], 0x06020C0Cu);
  const uint32_t od = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0602u) | __builtin_amdgcn_perm(b[7], b[5], 0x06020C0Cu);
  return ((od << 4) | ev) ^ 0x88888888u;   // byte k = nibble(c_2k) | nibble(c_2k+1) << 4
}

// ------------------------------------------------------------------ Walsh-Hadamard
// In-register fast Walsh-Hadamard transform (unnormalized, natural Sylvester order) on
// independent blocks of n = 2^lg consecutive elements of v[R]; lg is wave-uniform.
// One butterfly stage per index bit: (a, b) -> (a + b, a - b).
template <int R>
__device__ __forceinline__ void fwht_blocks(float (&v)[R], int lg) {
#pragma unroll
  for (int s = 0; (1 << s) < R; ++s) {
    if (s < lg) {
      const int st = 1 << s;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if ((i & st) == 0) {
          const float a = v[i], b = v[i + st];
          v[i] = a + b;
          v[i + st] = a - b;
        }
      }
    }
  }
}

}  // namespace kvq
