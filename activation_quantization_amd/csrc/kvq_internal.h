// Host <-> kernel interface inside libkvq (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

enum { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2 };

struct QuantArgs {
  const void* x;            // [rows, heads, D] f16/bf16
  const int8_t* signs;      // [heads, D] or null
  uint8_t* codes;           // [rows, heads, D/2]
  uint16_t* norms;          // [rows, heads] or null
  uint16_t* scales;         // per token [rows, heads] or per channel [rows/B, heads, D]
  int64_t seqs, tokens, heads, dim;
  int32_t block;            // B (per-channel modes)
  int32_t lg_had;           // log2 n, 0 = no rotation
  float inv_sqrt_n;         // 1/sqrt(n) (1 when no rotation)
  float q;                  // Q = 2^(bits-1) - 1
  float scale_mul;          // 1 / (sqrt(n) Q): stored scale = max of the unnormalized |u| * scale_mul
  int32_t nsep;             // norm separation on/off
  int32_t dtype;            // DT_F16 / DT_BF16
  // per-channel kernel only (the streaming append writes blocks into a larger cache):
  int64_t in_seq_tokens;    // x rows (tokens) from one sequence to the next (= tokens for a plain call)
  int64_t out_tokens;       // tokens per head-major output stream (= tokens for a plain call)
  int64_t out_tok0;         // stream token of the first quantized token (a multiple of B; 0 for a plain call)
  // per-token kernel only (RRS activations): every 128-channel segment k of a row is divided by
  // seg_div[k] (a divisor of 0 gives 0) after the rotation, before the per-token absmax; null = 1
  const float* seg_div;
};

// RRS INT4 GEMM: y[t, m] = a_t b_m sum_g s_g sum_{j in g} cx[t, j] cw[m, j], groups of 128 channels
struct RrsGemmArgs {
  const uint8_t* x_codes;   // [n, k/2] packed INT4, channel 2i in the low nibble
  const uint16_t* x_scales; // [n] fp16 a_t
  const uint8_t* w_codes;   // [m, k/2]
  const uint16_t* w_scales; // [m] fp16 b_m
  const float* s;           // [k/128] group smoothing scales
  float* y;                 // [n, m] fp32
  int64_t n, m, k;
};

// NSN variant (normalize, shift, normalize before the per-channel quantizer)
struct NsnArgs {
  const void* x;            // [rows, heads, D] f16/bf16
  const int8_t* signs;      // [heads, D] or null
  uint8_t* codes;           // head-major, as for the other modes
  uint16_t* s1;             // [seqs, heads, tokens] fp16: ||x|| / sqrt(D)
  uint16_t* s2;             // [seqs, heads, tokens] fp16: ||u1 - o|| / sqrt(D)
  uint16_t* offsets;        // [seqs, heads, tokens/B, D] fp16: the block's channel mean, original domain
  uint16_t* scales;         // [seqs, heads, tokens/B, D] fp16
  int64_t seqs, tokens, heads, dim;
  int32_t block;
  int32_t lg_had;
  int32_t q;                // Q = 2^(bits-1) - 1
  int32_t dtype;
};

struct DequantArgs {
  const uint8_t* codes;
  const uint16_t* norms;    // NSN: s1
  const uint16_t* scales;
  const int8_t* signs;
  const uint16_t* s2;       // NSN only
  const uint16_t* offsets;  // NSN only
  void* y;
  int64_t seqs, tokens, heads, dim;
  int32_t block;
  int32_t lg_had;
  float inv_sqrt_n;
  int32_t nsep;
  int32_t per_channel;
  int32_t out_dtype;        // DT_F16 / DT_BF16 / DT_F32
};

struct ScoreArgs {
  const uint16_t* q;        // [seqs, q_heads, D] fp16
  const uint8_t* codes;
  const uint16_t* norms;    // NSN: s1
  const uint16_t* scales;
  const int8_t* signs;
  const uint16_t* s2;       // NSN only
  const uint16_t* offsets;  // NSN only
  float* scores;            // [seqs, q_heads, tokens]
  int64_t seqs, tokens, heads, dim, q_heads;
  int32_t block;
  int32_t lg_had;
  float inv_sqrt_n;
  int32_t nsep;
  int32_t per_channel;
  int32_t nsn;              // NSN: norms = s1, plus s2 and the block offsets
};

struct AttnArgs {
  const uint16_t* q;        // [seqs, q_heads, D] fp16
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint16_t* k_scales;
  const int8_t* k_signs;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  const uint16_t* v_scales;
  const int8_t* v_signs;
  float* out;               // [seqs, q_heads, D]
  float* ws;                // per (sequence, query head, partial): R sums, max, normalizer
  int64_t seqs, tokens, heads, dim, q_heads;   // tokens: cached whole-block tokens attended per sequence
  int64_t stream_tokens;    // tokens per head-major cache stream (the capacity; >= tokens)
  int32_t block;
  int32_t lg_had;
  float inv_sqrt_n;
  int32_t nsep;
  // full-precision residual after the cached tokens (streaming append): [seqs, block, heads, D]
  const void* k_res;
  const void* v_res;
  int32_t nres;             // residual tokens per sequence (0: none)
  int32_t res_dtype;        // DT_F16 / DT_BF16
};

// The 128-point rotation of the per-token kernels runs on the matrix cores unless the environment
// variable KVQ_ROTATION is "butterfly" (read at every call), which selects the register-butterfly
// kernels (the comparison the rotation choice rests on).
bool rotation_butterfly();

// Launchers: enqueue on `stream`, return hipGetLastError() of the launch.
hipError_t launch_quantize_pchan(const QuantArgs& a, hipStream_t stream);
hipError_t launch_quantize_ptok(const QuantArgs& a, hipStream_t stream);
// the matrix-core per-token kernel (head_dim a power of two in [128, 8192]); launch_quantize_ptok
// dispatches to it
hipError_t launch_quantize_ptok_mfma(const QuantArgs& a, hipStream_t stream);
// RRS: s[k] = max over the rows of |(x R)| over 128-channel segment k (fp32, orthonormal units), for
// a per-token QuantArgs with heads = 1 and dim a power of two >= 128
hipError_t launch_rrs_colmax(const QuantArgs& a, float* s, hipStream_t stream);
hipError_t launch_rrs_gemm(const RrsGemmArgs& a, hipStream_t stream);
hipError_t launch_dequantize_pchan(const DequantArgs& a, hipStream_t stream);
hipError_t launch_quantize_nsn(const NsnArgs& a, hipStream_t stream);
hipError_t launch_dequantize_nsn(const DequantArgs& a, hipStream_t stream);
hipError_t launch_dequantize_ptok(const DequantArgs& a, hipStream_t stream);
hipError_t launch_score_decode(const ScoreArgs& a, hipStream_t stream);
hipError_t launch_attention_decode(const AttnArgs& a, hipStream_t stream);
// k tokens of rowb bytes per sequence, token-major runs: src sequences src_seq tokens apart, dst dst_seq;
// npairs (1 or 2) such (src[i], dst[i]) copies of the same shape in one launch
hipError_t launch_copy_tokens(const void* const* src, void* const* dst, int npairs, int64_t seqs, int64_t k, int64_t rowb,
                              int64_t src_seq, int64_t dst_seq, hipStream_t stream);
int64_t attention_partials(const AttnArgs& a);   // partials per (sequence, query head)
// The static partials buffer of the no-alloc attention entry point (its device address on the
// current device, looked up once per device); ATTENTION_SCRATCH_BYTES is its size.
constexpr int64_t ATTENTION_SCRATCH_BYTES = int64_t(32) << 20;
hipError_t attention_scratch(float** ptr);

}  // namespace kvq
