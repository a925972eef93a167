// Fused decode attention over a packed K/V cache (gfx950): the scores never leave the chip.
//
// Method sources (page title, section): NSNQuant summary "implementation details" (attention
// computed from the quantized cache with the stored byproducts folded into the kernel) and
// "latency" (decode time falls because the memory-bound attention reads less); norm-separation
// post "longer contexts get worse" (error accumulates in attention as the cache grows); Rotated
// Runtime Smooth analysis, Figure 2 (a rotation cancels inside a product, so the value sum may
// run in the rotated domain and be rotated back once).
//
//   out[s, hq] = sum_t p_t v^_t,  p = softmax_t(q . k^_t / sqrt(D)),
//   v^_t = sigma_v (1/sqrt n) H (norm_v[t] scale_v[blk(t)] (.) c_v[t])
// so  out = sigma_v (1/sqrt n) H  sum_blk scale_v[blk] (.) sum_{t in blk} p_t norm_v[t] c_v[t].
//
// Pass 1 (one workgroup of 4 waves per chunk of 16 scale blocks of one (sequence, KV head)
// stream; every wave walks its own blocks): per block, the scores of the G query heads come from
// the matrix cores exactly as in the decode-score kernel (query times K scales as an fp16 hi/lo
// A operand, codes as fp16 subnormals), an online softmax keeps the running max m and sum l per
// head, and the value sum runs on the int8 matrix cores in exact integers: the block's V codes
// (loaded into registers with the block's other loads, then written to LDS) are regrouped so each
// lane holds one channel of 16 tokens as bytes c + 8, against the value weights p' = p norm_v of
// each head as 24-bit integers (against the block's largest) split into three byte planes.  The
// four waves' (m, l, partial sum) are merged in LDS and the workgroup writes one partial per query
// head to the caller's workspace.  Pass 2 merges the partials of a head (log-sum-exp weights),
// rotates the result back and writes it.
#include <mutex>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int ATT_UNITS_PER_GROUP = 16;   // scale blocks per workgroup (4 per wave)

__device__ __forceinline__ int att_nib(int e) { return (e >> 1) + ((e & 1) << 2); }

__device__ __forceinline__ u32x4 att_codes_sub16(uint32_t word) {
  const uint32_t xb = word ^ 0x88888888u;
  return u32x4{xb & 0x000F000Fu, (xb >> 4) & 0x000F000Fu, (xb >> 8) & 0x000F000Fu, (xb >> 12) & 0x000F000Fu};
}

// max / sum over the 16 lanes of each row (DPP row rotations), every lane gets the result
__device__ __forceinline__ float row_max16f(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ float row_sum16f(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896340736f); }

// Pass 1.  R = 128 channels; U = the scale block (64 or 128 tokens); at most GM = 4 query heads
// per KV head (value sums of GM heads per lane).
template <int U>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
attn_partial(AttnArgs a, int64_t ntiles, int64_t nchunks) {
  constexpr int R = 128, KS = 4, LB = 16, GM = 4, NGR = U / 16;
  __shared__ __attribute__((aligned(16))) float qr[GM * R];                 // rotated queries
  __shared__ __attribute__((aligned(16))) unsigned char vbuf[4][U * 64];    // per wave: one block of V codes
  __shared__ __attribute__((aligned(16))) unsigned char wbuf[4][U / 64][16][64];   // per wave: MFMA A operand (weight planes)
  __shared__ float tokf[4][2][U];   // per wave, the block's tokens: K norm 2^24 / sqrt(D) (log2 e), V norm
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);    // wave index, in a scalar register
  const int g = lane >> 4, j = lane & 15;
  const int G = (int)(a.q_heads / a.heads);
  const int64_t T = a.tokens;

  const int64_t tile = xcd_tile(blockIdx.x, ntiles);
  const int64_t ci = tile % nchunks;
  const int64_t sh = tile / nchunks;                                      // stream: s * heads + kvh
  const int64_t kvh = sh % a.heads, s = sh / a.heads;

  // 1. rotated queries R q = (1/sqrt n) H (sigma_k q), once per workgroup
  for (int e = tid; e < G * R; e += 256) {
    const int hh = e / R, d = e % R;
    float v = f16_to_f32(a.q[(s * a.q_heads + kvh * G + hh) * R + d]);
    if (a.lg_had && a.k_signs[kvh * R + d] < 0) v = -v;
    qr[e] = v;
  }
  __syncthreads();
  for (int st = 0; st < a.lg_had; ++st) {
    const int half = 1 << st;
    for (int p = tid; p < G * R / 2; p += 256) {
      const int hh = p / (R / 2), pp = p % (R / 2);
      const int i = ((pp >> st) << (st + 1)) | (pp & (half - 1));
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

  const int64_t nunits = T / U;
  const int64_t u_begin = ci * ATT_UNITS_PER_GROUP;
  const int64_t u_end = u_begin + ATT_UNITS_PER_GROUP < nunits ? u_begin + ATT_UNITS_PER_GROUP : nunits;
  const int64_t TS = a.stream_tokens;                                       // stream length (capacity)
  const unsigned char* kstream = a.k_codes + sh * TS * (R / 2);
  const unsigned char* vstream = a.v_codes + sh * TS * (R / 2);
  const int64_t tstream = sh * TS;
  const int64_t nb = TS / U;                                                // scale rows per stream
  const float zscale = 1.f / sqrtf((float)R);

  // per-lane softmax state of the row's heads 2 g, 2 g + 1 (replicated over the row), and the
  // value sums: lane 16 g + b owns channels 8 b .. 8 b + 7 of head g
  float m_row[2] = {-INFINITY, -INFINITY}, l_row[2] = {0.f, 0.f};
  float o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = 0.f;
  const int vb = lane & 15;
  unsigned char* vw = &vbuf[w][0];
  unsigned char* ww = &wbuf[w][0][0][0];

  const uint16_t* knp = a.nsep ? a.k_norms + tstream : kF16One;      // per-token norms (1.0 without)
  const uint16_t* vnp = a.nsep ? a.v_norms + tstream : kF16One;
  for (int64_t un = u_begin + w; un < u_end; un += 4) {
    const int64_t t0 = un * U;
    // Every load of the block is issued before any is waited for, into registers and in the order
    // they are needed: the K and V norms (coalesced 2-byte loads by all lanes, token t0 + lane +
    // 64 k), the K and V scales, all of the block's K code groups (each group waited for on its
    // own), and the V codes (U * 64 bytes, 16 per lane and KiB; written to LDS only when the value
    // sum needs them).  All through
    // global-address-space pointers, so the compiler counts the loads in flight exactly (copies
    // into LDS, or flat loads, would make it wait for every load before the first LDS access).
    uint16_t kn[U / 64], vn[U / 64];
#pragma unroll
    for (int k = 0; k < U / 64; ++k) {
      const int64_t tt = t0 + lane + 64 * k;
      kn[k] = ld_global(knp + (a.nsep ? tt : 0));
      vn[k] = ld_global(vnp + (a.nsep ? tt : 0));
    }
    // K scales of this lane's channels (R/4) g + 8 K + nib(e); V scales of channels 8 vb ..
    // (scale rows are 16-byte aligned: the entry point requires it)
    const uint16_t* ksrow = a.k_scales + (sh * nb + un) * R + (R / 4) * g;
    u32x4 ksw[KS];
#pragma unroll
    for (int K = 0; K < KS; ++K) ksw[K] = ld_global((const u32x4*)(ksrow + 8 * K));
    const u32x4 vsw = ld_global((const u32x4*)(a.v_scales + (sh * nb + un) * R + 8 * vb));
    uint32_t wd[NGR][KS];
#pragma unroll
    for (int b = 0; b < NGR; ++b) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)(kstream + (t0 + 16 * b + j) * (R / 2) + LB * g));
      wd[b][0] = v.x; wd[b][1] = v.y; wd[b][2] = v.z; wd[b][3] = v.w;
    }
    u32x4 vcw[NGR];                                         // V codes: lane's 16 bytes of each KiB
#pragma unroll
    for (int k = 0; k < NGR; ++k) vcw[k] = __builtin_nontemporal_load((const u32x4*)(vstream + t0 * (R / 2) + k * 1024 + 16 * lane));
    __builtin_amdgcn_sched_barrier(0);
    float sc[KS * 8];
#pragma unroll
    for (int K = 0; K < KS; ++K) {
      const uint32_t wv[4] = {ksw[K].x, ksw[K].y, ksw[K].z, ksw[K].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int n = att_nib(e);
        sc[8 * K + e] = f16_to_f32((n & 1) ? wv[n >> 1] >> 16 : wv[n >> 1] & 0xffffu);
      }
    }
    float vs[8];
    {
      const uint32_t wv[4] = {vsw.x, vsw.y, vsw.z, vsw.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) vs[c] = f16_to_f32((c & 1) ? wv[c >> 1] >> 16 : wv[c >> 1] & 0xffffu);
    }

#pragma unroll
    for (int k = 0; k < U / 64; ++k) {
      tokf[w][0][lane + 64 * k] = f16_to_f32(kn[k]) * (0x1p24f * zscale);
      tokf[w][1][lane + 64 * k] = f16_to_f32(vn[k]);
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");

    // 2. scores of the block: A = (R q) * K scale as fp16 hi/lo rows (row i = lane & 15 -> head
    //    i / 2), B = K codes as fp16 subnormals (c + 8) 2^-24
    f16x8 av[KS];
    {
      const int hl = j >> 1;
      const bool live = hl < G;
#pragma unroll
      for (int K = 0; K < KS; ++K) {
        const float* qp = qr + hl * R + (R / 4) * g + 8 * K;
        const f32x4 q0 = *(const f32x4*)qp, q1 = *(const f32x4*)(qp + 4);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int n0 = att_nib(e), n1 = att_nib(e + 1);
          const float g0 = (n0 < 4 ? q0[n0] : q1[n0 - 4]) * sc[8 * K + e];
          const float g1 = (n1 < 4 ? q0[n1] : q1[n1 - 4]) * sc[8 * K + e + 1];
          const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(g0, g1));
          const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(g0 - (float)hi[0], g1 - (float)hi[1]));
          const f16x2 pv = live ? ((j & 1) ? lo : hi) : f16x2{(_Float16)0.f, (_Float16)0.f};
          av[K][e] = pv[0];
          av[K][e + 1] = pv[1];
        }
      }
    }
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = 0; K < KS; ++K)
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          av[K], __builtin_bit_cast(f16x8, u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}), acc0, 0, 0, 0);
    acc0 *= -8.f * 0x1p-24f;
    // z[gr][0/1]: scaled scores of heads 2 g, 2 g + 1 for token 16 gr + j; nv: V norm of it
    float z[NGR][2], nvv[NGR];
#pragma unroll
    for (int b = 0; b < NGR; ++b) {
      const float fk = tokf[w][0][16 * b + j];
      nvv[b] = tokf[w][1][16 * b + j];
      f32x4 acc = acc0;
#pragma unroll
      for (int K = 0; K < KS; ++K)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[K], __builtin_bit_cast(f16x8, att_codes_sub16(wd[b][K])), acc, 0, 0, 0);
      z[b][0] = (acc.x + acc.y) * fk;
      z[b][1] = (acc.z + acc.w) * fk;
    }

    // 3. online softmax for the row's two heads.  The value weights p' = p * norm_v become
    //    24-bit integers W = rint(p' 2^24 / wmax) (at most 2^24 - 1) against the block's largest
    //    weight wmax of the head (fp16 weights, 2^-12 relative, move a long, nearly cancelling value
    //    sum past 2e-3 of the output's rms), stored as three byte planes less 128 (signed int8):
    //    rows 4 h + b, b < 3, of the value MFMA's A operand; row 4 h + 3 is all ones, so the same
    //    products also give each channel's code sum, which puts the 128 back.  Token t sits at K
    //    position (lane group t % 4, byte 4 ((t / 4) % 4) + (t / 16) % 4) of K step t / 64, so this
    //    lane's four tokens of a K step fill one 32-bit word per plane (a byte transpose of their
    //    four weights).
    float alpha_row[2], wf_row[2];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      float mx = -INFINITY;
#pragma unroll
      for (int gr = 0; gr < NGR; ++gr) mx = fmaxf(mx, z[gr][q2]);
      mx = row_max16f(mx);
      const float mnew = fmaxf(m_row[q2], mx);
      alpha_row[q2] = exp_f(m_row[q2] - mnew);            // 0 on the first block (m = -inf)
      float ps = 0.f, wmax = 0.f;                          // sum of p, largest p'
      const int h = 2 * g + q2;
#pragma unroll
      for (int gr = 0; gr < NGR; ++gr) {
        const float p = exp_f(z[gr][q2] - mnew);
        ps += p;
        z[gr][q2] = p * nvv[gr];                            // p', in place of the score
        wmax = fmaxf(wmax, z[gr][q2]);
      }
      wmax = row_max16f(wmax);
      const float wscale = wmax > 0.f ? 0x1p24f / wmax : 0.f;
      if (h < GM) {
#pragma unroll
        for (int ks = 0; ks < NGR / 4; ++ks) {
          uint32_t wq[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float wv = __builtin_rintf(z[4 * ks + r][q2] * wscale);
            wq[r] = wv < 16777215.f ? (uint32_t)wv : 16777215u;                      // <= 2^24 - 1
          }
          // byte b of the four tokens' weights, side by side, each less 128 (a signed int8)
          const uint32_t l01 = __builtin_amdgcn_perm(wq[1], wq[0], 0x05010400u);   // w0.0 w1.0 w0.1 w1.1
          const uint32_t h01 = __builtin_amdgcn_perm(wq[3], wq[2], 0x05010400u);   // w2.0 w3.0 w2.1 w3.1
          const uint32_t l2 = __builtin_amdgcn_perm(wq[1], wq[0], 0x06020602u);    // w0.2 w1.2 (twice)
          const uint32_t h2 = __builtin_amdgcn_perm(wq[3], wq[2], 0x06020602u);    // w2.2 w3.2 (twice)
          const uint32_t pk[4] = {__builtin_amdgcn_perm(h01, l01, 0x05040100u) ^ 0x80808080u,
                                  __builtin_amdgcn_perm(h01, l01, 0x07060302u) ^ 0x80808080u,
                                  __builtin_amdgcn_perm(h2, l2, 0x05040100u) ^ 0x80808080u, 0x01010101u};
#pragma unroll
          for (int b = 0; b < 4; ++b)
            *(uint32_t*)(ww + ((ks * 16 + 4 * h + b) * 64 + 16 * (j & 3) + 4 * (j >> 2))) = pk[b];
        }
      }
      ps = row_sum16f(ps);
      wf_row[q2] = wmax * 0x1p-24f;
      l_row[q2] = l_row[q2] * alpha_row[q2] + ps;
      m_row[q2] = mnew;
    }
    // alpha and weight unit of this lane's head g (head h lives in row h / 2)
    float alpha_g = 0.f, wf_g = 0.f;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const int src = 16 * (h >> 1);
      const float ah = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha_row[h & 1]), src));
      const float fh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wf_row[h & 1]), src));
      if (g == h) {
        alpha_g = ah;
        wf_g = fh;
      }
    }

    // 4. value sums of the block on the matrix cores (v_mfma_i32_16x16x64_i8, exact integers):
    //    D[4 h + b][j] of group m = sum_t S_b(t) 16 c_t, column j = channel 8 j + m.  Lane (kg, j)
    //    reads word j (channels 8 j .. 8 j + 7) of its 16 tokens of the K step and takes nibble m
    //    of each as a byte.
#pragma unroll
    for (int k = 0; k < NGR; ++k) *(u32x4*)&vbuf[w][k * 1024 + 16 * lane] = vcw[k];
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    i32x4 acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = i32x4{0, 0, 0, 0};
    const int kg = lane >> 4;
    // bytes k of four words side by side: t[k] = (a0.k, a1.k, a2.k, a3.k)
    auto transpose4 = [](uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t (&t)[4]) {
      const uint32_t l01 = __builtin_amdgcn_perm(a1, a0, 0x05010400u), h01 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
      const uint32_t l23 = __builtin_amdgcn_perm(a3, a2, 0x05010400u), h23 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
      t[0] = __builtin_amdgcn_perm(l23, l01, 0x05040100u);
      t[1] = __builtin_amdgcn_perm(l23, l01, 0x07060302u);
      t[2] = __builtin_amdgcn_perm(h23, h01, 0x05040100u);
      t[3] = __builtin_amdgcn_perm(h23, h01, 0x07060302u);
    };
#pragma unroll
    for (int ks = 0; ks < NGR / 4; ++ks) {
      // the lane's 16 tokens of the K step, channels 8 vb .. 8 vb + 7 as 16 c (a code nibble in the
      // high half of a byte is 16 times its two's-complement value as an int8): even channels
      // shifted up, odd channels masked in place
      uint32_t ev[16], od[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 64 * ks + kg + 4 * (e >> 2) + 16 * (e & 3);
        const uint32_t x = *(const uint32_t*)(vw + t * 64 + 4 * vb);
        ev[e] = (x << 4) & 0xF0F0F0F0u;
        od[e] = x & 0xF0F0F0F0u;
      }
      const i32x4 av = *(const i32x4*)(ww + ((ks * 16 + (lane & 15)) * 64 + 16 * kg));
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const uint32_t* src = par ? od : ev;
        uint32_t bt[4][4];                                   // [q][k]: byte k of words 4 q .. 4 q + 3
#pragma unroll
        for (int q = 0; q < 4; ++q) transpose4(src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3], bt[q]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int m = 2 * k + par;                         // channel 8 vb + m
          acc[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              av, i32x4{(int)bt[0][k], (int)bt[1][k], (int)bt[2][k], (int)bt[3][k]}, acc[m], 0, 0, 0);
        }
      }
    }
    // lane (g, j): rows 4 g + b = the planes of head g and its row of ones; with S_b = W_b - 128
    // and B = 16 c, D_b = 16 sum_t S_b c_t and D_1 = 16 sum_t c_t, so
    // 16 sum_t W c_t = sum_b 256^b D_b + 128 (1 + 256 + 65536) D_1; every D below 2^24 (exact in fp32)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float v = (float)acc[m][2];
      v = __builtin_fmaf(v, 256.f, (float)acc[m][1]);
      v = __builtin_fmaf(v, 256.f, (float)acc[m][0]);
      v = __builtin_fmaf((float)acc[m][3], 128.f * 65793.f, v);
      o[m] = o[m] * alpha_g + vs[m] * (wf_g * 0.0625f * v);
    }
    // every lane of the wave is done with this block's LDS before the next block's copy
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  }

  // 6. merge the four waves' partials through LDS (each wave's V buffer is free now), then one
  // partial (max, sum, vector) per head for the workgroup
  float* mw = (float*)&vbuf[w][0];                         // [GM][R] sums, [GM] maxima, [GM] sums of p
#pragma unroll
  for (int c = 0; c < 8; ++c) mw[g * R + 8 * vb + c] = o[c];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    const float mh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_row[h & 1]), 16 * (h >> 1)));
    const float lh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_row[h & 1]), 16 * (h >> 1)));
    if (lane == 0) {
      mw[GM * R + h] = mh;
      mw[GM * R + GM + h] = lh;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * R; e += 256) {
    const int h = e / R, c = e - h * R;
    float mx[4], M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      mx[ww] = ((const float*)&vbuf[ww][0])[GM * R + h];
      M = fmaxf(M, mx[ww]);
    }
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float* pw4 = (const float*)&vbuf[ww][0];
      const float f = mx[ww] == -INFINITY ? 0.f : exp_f(mx[ww] - M);
      L += f * pw4[GM * R + GM + h];
      O += f * pw4[h * R + c];
    }
    float* wp = a.ws + ((s * a.q_heads + kvh * G + h) * nchunks + ci) * (R + 2);
    wp[c] = O;
    if (c == 0) {
      wp[R] = M;
      wp[R + 1] = L;
    }
  }
}

// Pass 2: one workgroup of R threads per (sequence, query head): merge the cached part's
// partials, rotate their value sum back, then merge the residual tokens (if any), which are
// attended at full precision in the original domain.
__global__ void __launch_bounds__(128) attn_combine(AttnArgs a, int64_t NP) {
  constexpr int R = 128;
  __shared__ float buf[R];
  __shared__ float red[R];
  const int c = threadIdx.x;
  const int64_t shq = blockIdx.x;                              // s * q_heads + hq
  const int64_t s = shq / a.q_heads, hq = shq - s * a.q_heads;
  const int64_t kvh = hq / (a.q_heads / a.heads);
  const float* wp = a.ws + shq * NP * (R + 2);
  float M = -INFINITY;
#pragma unroll 4
  for (int64_t p = 0; p < NP; ++p) M = fmaxf(M, wp[p * (R + 2) + R]);
  float L = 0.f, O = 0.f;
#pragma unroll 4
  for (int64_t p = 0; p < NP; ++p) {
    const float m = wp[p * (R + 2) + R];
    const float f = m == -INFINITY ? 0.f : exp_f(m - M);
    L += f * wp[p * (R + 2) + R + 1];
    O += f * wp[p * (R + 2) + c];
  }
  // inverse rotation of the (unnormalized) value sum: sigma_v (1/sqrt n) H, blocks of n = 2^lg_had
  buf[c] = O;
  __syncthreads();
  for (int st = 0; st < a.lg_had; ++st) {
    const int half = 1 << st;
    const float x = buf[c], y = buf[c ^ half];
    __syncthreads();
    buf[c] = (c & half) ? y - x : x + y;
    __syncthreads();
  }
  O = buf[c];
  if (a.lg_had) {
    O *= a.inv_sqrt_n;
    if (a.v_signs[kvh * R + c] < 0) O = -O;
  }
  if (a.nres == 0) {                                           // uniform over the workgroup
    a.out[shq * R + c] = L > 0.f ? O / L : 0.f;
    return;
  }

  // residual tokens t < nres: scores q . k_t / sqrt(D) (thread t), their max and sum, and the
  // value sum (thread c = channel)
  const int r = a.nres;
  const int64_t rrow = (int64_t)a.heads * R;                   // elements between residual tokens
  const int64_t rbase = (s * a.block * a.heads + kvh) * R;     // token 0 of this sequence and head
  auto res = [&](const void* base, int64_t i) -> float {
    const uint32_t h = ((const uint16_t*)base)[i];
    return a.res_dtype == DT_F16 ? f16_to_f32(h) : bf16_to_f32(h);
  };
  buf[c] = f16_to_f32(a.q[shq * R + c]);
  __syncthreads();
  float z = -INFINITY;
  if (c < r) {
    float acc = 0.f;
    for (int d = 0; d < R; ++d) acc = __builtin_fmaf(buf[d], res(a.k_res, rbase + c * rrow + d), acc);
    z = acc * (1.f / sqrtf((float)R));
  }
  red[c] = z;
  __syncthreads();
  for (int half = R / 2; half > 0; half >>= 1) {
    if (c < half) red[c] = fmaxf(red[c], red[c + half]);
    __syncthreads();
  }
  const float mr = red[0];
  __syncthreads();
  const float p = c < r ? exp_f(z - mr) : 0.f;
  buf[c] = p;                                                  // the query is no longer needed
  red[c] = p;
  __syncthreads();
  for (int half = R / 2; half > 0; half >>= 1) {
    if (c < half) red[c] += red[c + half];
    __syncthreads();
  }
  const float lr = red[0];
  float orr = 0.f;
  for (int t = 0; t < r; ++t) orr = __builtin_fmaf(buf[t], res(a.v_res, rbase + t * rrow + c), orr);
  const float mx = fmaxf(M, mr);
  const float fq = M == -INFINITY ? 0.f : exp_f(M - mx), fr = exp_f(mr - mx);
  a.out[shq * R + c] = (fq * O + fr * orr) / (fq * L + fr * lr);
}

}  // namespace

// Decode attention's per-workgroup partials for callers that cannot allocate (the no-alloc entry
// point): a file-scope device array, one per GPU, held until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol; its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address is
// passed to kernels.
static __device__ __align__(256) float scratch[ATTENTION_SCRATCH_BYTES / sizeof(float)];

hipError_t attention_scratch(float** ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static float* addr[MAX_DEVICES] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int64_t attention_partials(const AttnArgs& a) {
  const int64_t nunits = a.tokens / a.block;
  return (nunits + ATT_UNITS_PER_GROUP - 1) / ATT_UNITS_PER_GROUP;     // one per workgroup
}

hipError_t launch_attention_decode(const AttnArgs& a, hipStream_t st) {
  const int64_t nunits = a.tokens / a.block;
  const int64_t nchunks = (nunits + ATT_UNITS_PER_GROUP - 1) / ATT_UNITS_PER_GROUP;
  const int64_t ntiles = a.seqs * a.heads * nchunks;
  if (ntiles > 0) {                                            // no whole block cached: residual only
    if (a.block == 64)
      hipLaunchKernelGGL((attn_partial<64>), dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles, nchunks);
    else
      hipLaunchKernelGGL((attn_partial<128>), dim3((unsigned)ntiles), dim3(256), 0, st, a, ntiles, nchunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_combine, dim3((unsigned)(a.seqs * a.q_heads)), dim3(128), 0, st, a, nchunks);
  return hipGetLastError();
}

}  // namespace kvq
