// RRS INT4 GEMM for gfx950: Y = sum over channel groups of the group's smoothing scale times the
// group's integer product of INT4 activations and INT4 weights.
//
// Method source (page title, section): Rotated Runtime Smooth analysis, "master equation"
// (Y = sum_j (X'_quant)_j (W'_quant)_j^T s_j), "step-by-step flow" (the per-channel partial products
// scaled by s_j, then summed) and Figure 4 (channels grouped to the matrix multiplication's block
// size, one runtime scale per group, applied to the interim result of each block).  With the
// per-token activation scale a_t and the per-output-channel weight scale b_m,
//   y[t, m] = a_t b_m sum_g s_g P_g[t, m],   P_g[t, m] = sum_{j in group g} cx[t, j] cw[m, j],
// each P_g an exact int32 from the int8 matrix cores, scaled and summed in fp32.
//
// Work split: a workgroup (4 waves) owns a 128 x 128 output tile, wave (wr, wc) its 64 x 64
// quarter as 4 x 4 blocks of v_mfma_i32_16x16x64_i8.  Per group of 128 channels the two operand
// tiles (128 rows x 64 packed bytes each) stream into a ring of four LDS stages with
// global_load_lds, three groups ahead of the one computed; in LDS, 16-byte chunk c of row r sits in slot c ^ ((r / 4) mod 4), so the 16
// lanes reading 8 bytes of 16 consecutive rows hit 32 different banks.  A lane's 8 packed bytes
// (16 codes) become the 16 int8 operand bytes without sign extension: a code byte's high nibble
// masked in place, w & 0xF0, is 16 times that two's-complement nibble as an int8, and the low
// nibble shifted up, (w << 4) & 0xF0, likewise; the odd and even codes go to separate words (the
// same channel order in both operands, so the dot product is unchanged).  Three ALU operations per
// 8 codes; every product carries 16 x 16 = 256, exact in int32 (|P| <= 128 49 256 < 2^21) and in
// its fp32 conversion, and removed with the group scale (s_g / 256, a power-of-two factor).  The
// int32 group products are scaled into fp32 accumulators; the epilogue applies a_t b_m.  Rows or columns past n or m read the last row
// (addresses stay inside the operands) and are not stored.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int TT = 128;        // output tile rows (tokens) and columns (output channels)
constexpr int KG = 128;        // channels per smoothing group = the K block
constexpr int GB = KG / 2;     // packed bytes of one row in one group
constexpr int NST = 4;         // LDS stages: the group computed and three in flight
constexpr int LPG = 4;         // global_load_lds instructions per wave and group
constexpr int GM = 8;          // tile rows per group of the tile order

// 16 packed codes (8 bytes) -> the 16 int8 bytes of one MFMA operand lane, each 16 times its code
__device__ __forceinline__ i32x4 unpack16x16(u32x2 p) {
  return i32x4{(int)((p.x << 4) & 0xF0F0F0F0u), (int)(p.x & 0xF0F0F0F0u), (int)((p.y << 4) & 0xF0F0F0F0u),
               (int)(p.y & 0xF0F0F0F0u)};
}

__global__ void __launch_bounds__(256) rrs_gemm_kernel(RrsGemmArgs a, int64_t tiles_m, int64_t ntiles) {
  __shared__ __attribute__((aligned(16))) unsigned char sa[NST][TT * GB];   // activation codes of a group
  __shared__ __attribute__((aligned(16))) unsigned char sb[NST][TT * GB];   // weight codes of a group
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w >> 1, wc = w & 1;
  // each XCD takes a contiguous range of tiles, walked in groups of GM tile rows with the row
  // fastest: the tiles in flight on one XCD share GM row tiles of A and a few column tiles of B,
  // a working set its L2 holds (row-major order would sweep all of B once per tile row)
  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t tiles_n = ntiles / tiles_m;
  const int64_t grp = tile / (GM * tiles_m), in_grp = tile - grp * (GM * tiles_m);
  const int64_t first_n = grp * GM;
  const int64_t gsz = tiles_n - first_n < GM ? tiles_n - first_n : GM;
  const int64_t tn = first_n + in_grp % gsz, tm = in_grp / gsz;
  const int64_t r0 = tn * TT, c0 = tm * TT;
  const int64_t kb = a.k / 2;                                   // packed bytes per row
  const int ng = (int)(a.k / KG);

  // group g's operand tiles into buffer buf: 512 16-byte pieces each, wave w issuing pieces
  // 64 (2 w + i) + lane (row p / 4, chunk p mod 4 of the row's group slice); the per-lane source
  // addresses of group 0, computed once
  const unsigned char* xsrc[2];
  const unsigned char* wsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = 64 * (2 * w + i) + lane, row = p >> 2, ch = p & 3;
    const int phys = ch ^ ((row >> 2) & 3);
    const int64_t xr = r0 + row < a.n ? r0 + row : a.n - 1;
    const int64_t mr = c0 + row < a.m ? c0 + row : a.m - 1;
    xsrc[i] = a.x_codes + xr * kb + 16 * phys;
    wsrc[i] = a.w_codes + mr * kb + 16 * phys;
  }
  auto issue = [&](int g, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(xsrc[i] + g * GB),
                                       (__attribute__((address_space(3))) void*)(sa[buf] + 1024 * (2 * w + i)), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + g * GB),
                                       (__attribute__((address_space(3))) void*)(sb[buf] + 1024 * (2 * w + i)), 16, 0, 0);
    }
  };
  // 8 packed bytes of row r at byte offset o of its group slice (o a multiple of 8)
  auto frag = [&](const unsigned char* t, int r, int o) {
    return *(const u32x2*)(t + r * GB + 16 * ((o >> 4) ^ ((r >> 2) & 3)) + (o & 8));
  };

  f32x4 accf[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) accf[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int p = 0; p < NST - 1 && p < ng; ++p) issue(p, p);
  // group g in LDS stage BUF = g mod NST; the loop is unrolled over the NST stages so that each
  // stage's base is an immediate and the fragment addresses stay loop-invariant
  auto group = [&](const int g, auto stage) {
    constexpr int BUF = decltype(stage)::value;
    // the group's scale (the operands carry 16 x 16), read through the scalar unit: a vector load
    // here would be waited for with vmcnt(0), which also drains the operand loads in flight
    const float sg = ((const __attribute__((address_space(4))) float*)a.s)[g] * (1.f / 256.f);
    // group g has landed once at most the loads of the groups issued after it are in flight
    // (LPG per group; vmcnt(n) immediates: expcnt and lgkmcnt left unconstrained)
    const int later = ng - 1 - g < NST - 2 ? ng - 1 - g : NST - 2;
    if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * LPG));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | LPG);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
    lds_barrier();                                            // and every wave is done with group g - 1's stage
    if (g + NST - 1 < ng) issue(g + NST - 1, (g + NST - 1) % NST);
    i32x4 acc[4][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int o = 32 * ks + 8 * (lane >> 4);               // K position of this lane's 16 codes
      i32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = unpack16x16(frag(sa[BUF], 64 * wr + 16 * i + (lane & 15), o));
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) bf[jj] = unpack16x16(frag(sb[BUF], 64 * wc + 16 * jj + (lane & 15), o));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[jj], ks == 0 ? i32x4{0, 0, 0, 0} : acc[i][jj], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) accf[i][jj][r] = __builtin_fmaf((float)acc[i][jj][r], sg, accf[i][jj][r]);
  };
  for (int g0 = 0; g0 < ng; g0 += NST) {
    group(g0, std::integral_constant<int, 0>{});
    if (g0 + 1 < ng) group(g0 + 1, std::integral_constant<int, 1>{});
    if (g0 + 2 < ng) group(g0 + 2, std::integral_constant<int, 2>{});
    if (g0 + 3 < ng) group(g0 + 3, std::integral_constant<int, 3>{});
  }
  static_assert(NST == 4, "the group loop is unrolled over four stages");

  // epilogue: lane (q, j) holds rows 4 q + r, column j of every 16 x 16 block.  Every scale load is
  // issued first, at clamped indices (a row or column past the end is loaded, not stored), so none
  // waits for another.
  const int q4 = lane >> 4, j = lane & 15;
  uint16_t bh[4], ah[4][4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int64_t m = c0 + 64 * wc + 16 * jj + j;
    bh[jj] = a.w_scales[m < a.m ? m : a.m - 1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = r0 + 64 * wr + 16 * i + 4 * q4 + r;
      ah[i][r] = a.x_scales[t < a.n ? t : a.n - 1];
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = r0 + 64 * wr + 16 * i + 4 * q4 + r;
      const float at = f16_to_f32(ah[i][r]);
      float* yr = a.y + t * a.m;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t m = c0 + 64 * wc + 16 * jj + j;
        if (t < a.n && m < a.m) __builtin_nontemporal_store(accf[i][jj][r] * at * f16_to_f32(bh[jj]), yr + m);
      }
    }
}

}  // namespace

hipError_t launch_rrs_gemm(const RrsGemmArgs& a, hipStream_t st) {
  const int64_t tiles_n = (a.n + TT - 1) / TT, tiles_m = (a.m + TT - 1) / TT;
  const int64_t ntiles = tiles_n * tiles_m;
  if (ntiles > 0)
    hipLaunchKernelGGL(rrs_gemm_kernel, dim3((unsigned)ntiles), dim3(256), 0, st, a, tiles_m, ntiles);
  return hipGetLastError();
}

}  // namespace kvq
