/*
 * kvq.h -- C ABI of the MI355X (gfx950) KV-cache / activation quantizer.
 *
 * The method (sources, by page title and section):
 *   - "nsep+pchan" norm-separation post, "the fix": split each KV vector into an fp16 L2 norm
 *     and a unit direction, then quantize the direction with per-channel scales; symmetric
 *     round-to-nearest onto +-(2^(b-1)-1) (the snippet divides the absmax by 7 and clamps to
 *     +-7 at INT4; INT3 is discussed under "INT3 > INT4").
 *   - Rotated Runtime Smooth analysis, "problem definition" (alpha = max|X| / (2^(N-1)-1)) and
 *     "term-by-term" (rotation R = (1/sqrt K)[+-1], R R^T = I; runtime scale s_j = max over
 *     tokens of column j).
 *   - NSNQuant summary, "Hadamard transform" (randomized Hadamard before quantization) and
 *     "implementation details" (scores computed from the quantized cache with the stored
 *     parameters folded into the kernel).
 *   - Activation-guided compensation abstract: random +-1 signs before the Hadamard rotation.
 *
 * Conventions shared by every entry point
 *   - Tensor x is [rows, heads, head_dim], rows = seqs * tokens_per_seq, head_dim fastest,
 *     contiguous.  For a wide activation row use heads = 1, head_dim = hidden.
 *   - Every data pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA tensor's storage)
 *     on the current HIP device.  The caller allocates and owns every buffer; buffers must
 *     stay alive until the work enqueued on `stream` has completed.  The library keeps no
 *     pointer after a call returns and allocates nothing on these paths.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.  Every call only
 *     enqueues kernels and returns without synchronizing; device faults surface at the
 *     caller's next synchronization.
 *   - All validation happens before anything is enqueued: on any error status nothing is
 *     launched and no output is touched.  kvq_last_error() then describes the failure
 *     (thread-local string).  No C++ exception crosses this interface.
 *
 * Storage formats (outputs are head-major: every (sequence, head) is one contiguous stream,
 * so a cache block of one head is whole cache lines for every kernel that touches it)
 *   codes   uint8 [seqs, heads, tokens_per_seq, head_dim/2]: two 4-bit two's-complement codes
 *           per byte, channel 2i in the low nibble, 2i+1 in the high nibble.  INT3 and 2-bit
 *           codes use the same nibble layout.  Codes lie in [-Q, Q], Q = 2^(bits-1)-1.
 *   norms   fp16 bits [seqs, heads, tokens_per_seq]: the L2 norm of each (rotated) vector;
 *           NSEP modes only.
 *   scales  fp16 bits.  Per-token modes (NAIVE, NSEP): [seqs, heads, tokens_per_seq] =
 *           absmax / Q of the (rotated, normalized) vector.  Per-channel modes (PCHAN,
 *           NSEP_PCHAN): [seqs, heads, tokens_per_seq / block_tokens, head_dim] = max over the
 *           block's tokens of |u| / Q, one per channel.
 *   signs   int8 [heads, head_dim] of +-1 (any value < 0 counts as -1).  Block k of n
 *           channels of head h uses signs[h, k*n : (k+1)*n].  NULL iff hadamard == 0.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,        /* a required pointer is NULL, or a forbidden one is non-NULL     */
  KVQ_ERR_ALIGN = 2,       /* x, y, codes or signs not 16-byte aligned; norms, scales or q not
                              2-byte aligned; scores not 4-byte aligned                      */
  KVQ_ERR_SHAPE = 3,       /* negative seqs / tokens, heads or head_dim < 1, odd head_dim, n
                              does not divide head_dim, block does not divide tokens_per_seq,
                              q_heads not a positive multiple of heads                       */
  KVQ_ERR_UNSUPPORTED = 4, /* bits, dtype, head_dim, block or n outside the built kernels     */
  KVQ_ERR_HIP = 5          /* no HIP device, or the launch reported an error                 */
} kvq_status;

typedef enum {
  KVQ_NAIVE = 0,      /* per-token absmax of x (after the optional rotation)                 */
  KVQ_NSEP = 1,       /* norm separation, per-token absmax of the unit direction             */
  KVQ_PCHAN = 2,      /* per-channel absmax over a block of tokens, no norm separation       */
  KVQ_NSEP_PCHAN = 3, /* norm separation, then per-channel scales over the token block       */
  KVQ_NSN_PCHAN = 4   /* normalize-shift-normalize, then per-channel scales (the _nsn calls)  */
} kvq_mode;

typedef enum { KVQ_F16 = 0, KVQ_BF16 = 1, KVQ_F32 = 2 } kvq_dtype;

/* Shape and method parameters (all fields plain integers for a stable layout: 56 bytes). */
typedef struct {
  int64_t seqs;           /* number of sequences (>= 0)                                       */
  int64_t tokens_per_seq; /* tokens per sequence (>= 0); seqs or tokens_per_seq = 0 is an empty
                             input: calls return KVQ_OK without launching or reading pointers */
  int64_t heads;          /* KV heads (>= 1)                                                  */
  int64_t head_dim;       /* channels per head: 64 or 128; per-token modes also 256..8192
                             (powers of two)                                                  */
  int32_t bits;           /* 2, 3 or 4                                                        */
  int32_t mode;           /* kvq_mode                                                         */
  int32_t block_tokens;   /* per-channel token block B: 64, 128 or 256 (B <= 128 when
                             head_dim = 128); must divide tokens_per_seq; ignored (set 0) for
                             per-token modes                                                  */
  int32_t hadamard;       /* 0 = no rotation; else n in {16, 32, 64, 128}, n | head_dim       */
  int32_t dtype;          /* kvq_dtype of x: KVQ_F16 or KVQ_BF16                              */
  int32_t reserved;       /* must be 0                                                        */
} kvq_desc;

/* Checks a descriptor without touching the device.  KVQ_OK or the reason it is refused. */
kvq_status kvq_validate(const kvq_desc* d);

/* Buffer sizes for a valid descriptor (-1 if kvq_validate fails):
 *   codes bytes = rows*heads*head_dim/2; norms = rows*heads for NSEP modes and for each of s1 and s2
 *   of the NSN mode, else 0; scales = rows*heads (per-token) or
 *   seqs*(tokens_per_seq/block_tokens)*heads*head_dim (per-channel and NSN; also the NSN offsets). */
int64_t kvq_codes_bytes(const kvq_desc* d);
int64_t kvq_norms_count(const kvq_desc* d);
int64_t kvq_scales_count(const kvq_desc* d);

/*
 * Quantize x [rows, heads, head_dim] (dtype d->dtype) into packed codes, fp16 norms (NSEP
 * modes) and fp16 scales.  Sources: norm-separation post, "the fix" (an fp16 L2 norm per KV vector
 * and a unit direction; absmax / Q; round and clamp to +-Q) and per-channel scaling; Rotated Runtime
 * Smooth analysis, "problem definition" (alpha = max|X| / (2^(N-1) - 1)) and "term-by-term"
 * (R = (1/sqrt K)[+-1]); NSNQuant summary, "Hadamard transform" (random signs before the Hadamard
 * matrix).  Steps per (token, head) vector: optional signs then orthonormal block Hadamard
 * (1/sqrt n, natural Sylvester order); nu = ||y||_2 and u = y/nu (NSEP modes; nu = 0 gives u = 0);
 * scale = absmax / Q per token or per channel over the token block; code =
 * clamp(round_half_even(u / scale), -Q, Q) of the exact quotient (from the unrounded scale and norm;
 * scale = 0 gives code 0).  Stored norms and scales are the fp16 (round-to-nearest-even) values of
 * nu and scale.  Outputs are head-major: codes [seqs, heads, tokens, head_dim/2], norms and per-token
 * scales [seqs, heads, tokens], per-channel scales [seqs, heads, tokens/B, head_dim].
 *   norms must be NULL for NAIVE / PCHAN and non-NULL for NSEP modes.
 */
kvq_status kvq_quantize(const kvq_desc* d, const void* x, const int8_t* signs,
                        uint8_t* codes, uint16_t* norms, uint16_t* scales, void* stream);

/*
 * Dequantize: y^ = code * scale * (norm for NSEP modes), then the inverse rotation
 * sigma * (1/sqrt n) H y^, written to y [rows, heads, head_dim] in y_dtype (F16, BF16 or
 * F32, round-to-nearest-even).  Inputs are exactly the buffers kvq_quantize writes.  Sources:
 * norm-separation post, "the fix" (the quantized direction is code times scale, and the norm
 * multiplies back); Rotated Runtime Smooth analysis, "term-by-term" (R^-1 = R^T); NSNQuant summary,
 * "implementation details" (a dedicated dequantization kernel).
 */
kvq_status kvq_dequantize(const kvq_desc* d, const uint8_t* codes, const uint16_t* norms,
                          const uint16_t* scales, const int8_t* signs, void* y, int32_t y_dtype,
                          void* stream);

/*
 * Decode attention scores straight from the packed K cache described by d (head_dim 64 or
 * 128):  scores[s, hq, t] = sum_d q[s, hq, d] * k^[s*T + t, hq / G, d], G = q_heads/heads
 * (query heads grouped contiguously), k^ the dequantized key.  No 1/sqrt(d), no softmax.
 * The kernel works in the rotated domain: it rotates each query once and folds the stored
 * scales and norms into the contraction.  Sources: NSNQuant summary, "implementation details"
 * (scores computed from the quantized keys with the stored byproducts folded into the kernel) and
 * "latency"; Rotated Runtime Smooth analysis, Figure 2 (XR (R^-1 W^T) = X W^T: the product may run
 * in the rotated domain).
 *   q: fp16 bits [seqs, q_heads, head_dim]; scores: fp32 [seqs, q_heads, tokens_per_seq].
 */
kvq_status kvq_score_decode(const kvq_desc* d, const uint16_t* q, int64_t q_heads,
                            const uint8_t* codes, const uint16_t* norms, const uint16_t* scales,
                            const int8_t* signs, float* scores, void* stream);

/*
 * Fused decode attention over a packed K cache and a packed V cache, both written by
 * kvq_quantize with descriptor d (one decode step; the scores stay on the chip).  Source: NSNQuant
 * summary, "implementation details" and "latency"; norm-separation post, "longer contexts get
 * worse".
 *   out[s, hq, :] = sum_t p_t v^[s*T + t, hq / G, :],  p = softmax_t(q[s, hq] . k^_t / sqrt(D))
 * with G = q_heads / heads and k^, v^ the dequantized caches.  Requirements: a per-channel mode
 * (PCHAN or NSEP_PCHAN), head_dim 128, block_tokens 64 or 128, tokens_per_seq >= 1, G <= 4.
 *   q: fp16 bits [seqs, q_heads, head_dim]; out: fp32 [seqs, q_heads, head_dim].
 *   k_signs / v_signs: the signs each cache was quantized with (NULL iff hadamard == 0).
 *   workspace: device memory of at least kvq_attention_workspace_bytes(d, q_heads) bytes, 4-byte
 *   aligned, owned by the caller; its contents on entry do not matter and are overwritten.
 *   Codes and scales must be 16-byte aligned; q, norms 2-byte; out 4-byte.
 * The call enqueues two kernels (partial softmax sums per cache chunk, then their merge).
 */
int64_t kvq_attention_workspace_bytes(const kvq_desc* d, int64_t q_heads);
kvq_status kvq_attention_decode(const kvq_desc* d, const uint16_t* q, int64_t q_heads,
                                const uint8_t* k_codes, const uint16_t* k_norms, const uint16_t* k_scales,
                                const int8_t* k_signs, const uint8_t* v_codes, const uint16_t* v_norms,
                                const uint16_t* v_scales, const int8_t* v_signs, float* out, void* workspace,
                                int64_t workspace_bytes, void* stream);

/*
 * kvq_attention_decode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, requirements and
 * result as kvq_attention_decode, without the workspace: the partials live in a static device
 * array of KVQ_ATTENTION_SCRATCH_BYTES bytes per GPU, which the library holds until the process
 * ends.  A shape whose kvq_attention_workspace_bytes exceeds that returns KVQ_ERR_UNSUPPORTED (the
 * 64 x 32768-token, 8-head, 32-query-head decode step needs 17,039,360 bytes).  The call allocates
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and give wrong results.
 */
#define KVQ_ATTENTION_SCRATCH_BYTES 33554432
kvq_status kvq_attention_decode_noalloc(const kvq_desc* d, const uint16_t* q, int64_t q_heads,
                                        const uint8_t* k_codes, const uint16_t* k_norms, const uint16_t* k_scales,
                                        const int8_t* k_signs, const uint8_t* v_codes, const uint16_t* v_norms,
                                        const uint16_t* v_scales, const int8_t* v_signs, float* out, void* stream);

/*
 * Streaming append with a full-precision residual (NSNQuant summary, "implementation details": the
 * KV cache is a quantized part plus a full-precision residual; when the residual is full it is
 * quantized and moved into the quantized part).  Per-channel modes only: a per-channel scale needs
 * a whole block of block_tokens tokens, so the last tokens_cached mod B tokens of a sequence wait
 * at full precision (per-token codes need no residual: kvq_quantize on the new tokens appends them).
 *   d: the cache.  tokens_per_seq is its capacity C (a multiple of block_tokens); codes, norms and
 *      scales are head-major streams of C tokens, laid out exactly as kvq_quantize writes them.
 *   tokens_cached: tokens already appended to every sequence (the caller keeps count; the cache
 *      holds the first floor(tokens_cached / B) B tokens, the residual the rest in its first slots).
 *   x_new: [seqs, n_new, heads, head_dim] in d->dtype, the tokens to append to every sequence.
 *   residual: [seqs, block_tokens, heads, head_dim] in d->dtype, read and written.
 *   signs: as for kvq_quantize.
 * Afterwards every sequence holds tokens_cached + n_new tokens (must be <= C): each block that
 * filled has been quantized into the cache exactly as kvq_quantize quantizes it, and the tokens
 * after the last whole block sit in residual slots 0 .. (tokens_cached + n_new) mod B - 1.
 * Enqueues up to four launches (residual top-up, its quantization, whole blocks straight from
 * x_new, the new residual); allocates nothing.  x_new, residual, codes, signs 16-byte aligned.
 */
kvq_status kvq_append(const kvq_desc* d, int64_t tokens_cached, const void* x_new, int64_t n_new, void* residual,
                      const int8_t* signs, uint8_t* codes, uint16_t* norms, uint16_t* scales, void* stream);

/*
 * The streaming append of one decode step's keys and values in one call: exactly kvq_append on the
 * K cache (k_new, k_residual, k_signs, k_codes, k_norms, k_scales) followed by kvq_append on the V
 * cache (v_...), both described by d and holding the same tokens_cached, with the same results
 * (NSNQuant summary, "implementation details": the quantized part plus a full-precision residual,
 * for each of K and V).  The residual top-ups of both caches are one copy launch, and so are the new
 * residuals, so a decode step that appends one token enqueues one launch instead of two; a block
 * that fills is quantized per cache.  Arguments, layouts, alignment and ownership as for kvq_append,
 * per side; a check that fails names its side ("K side: ", "V side: ") and nothing is enqueued.
 */
kvq_status kvq_append_kv(const kvq_desc* d, int64_t tokens_cached, int64_t n_new, const void* k_new, void* k_residual,
                         const int8_t* k_signs, uint8_t* k_codes, uint16_t* k_norms, uint16_t* k_scales,
                         const void* v_new, void* v_residual, const int8_t* v_signs, uint8_t* v_codes,
                         uint16_t* v_norms, uint16_t* v_scales, void* stream);

/*
 * Fused decode attention over a streamed cache: kvq_attention_decode over the first tokens_cached
 * tokens of every sequence, where the whole blocks come from the packed caches (capacity
 * d->tokens_per_seq) and the last tokens_cached mod B tokens from the full-precision residuals that
 * kvq_append maintains (k_residual, v_residual: [seqs, block_tokens, heads, head_dim] in d->dtype,
 * 2-byte aligned; they may be NULL when tokens_cached is a multiple of B).  One softmax spans both
 * parts (NSNQuant summary, "implementation details").  1 <= tokens_cached <= tokens_per_seq; the
 * workspace is sized by kvq_attention_workspace_bytes(d, q_heads), as for kvq_attention_decode.
 */
kvq_status kvq_attention_decode_stream(const kvq_desc* d, int64_t tokens_cached, const uint16_t* q, int64_t q_heads,
                                       const uint8_t* k_codes, const uint16_t* k_norms, const uint16_t* k_scales,
                                       const int8_t* k_signs, const void* k_residual, const uint8_t* v_codes,
                                       const uint16_t* v_norms, const uint16_t* v_scales, const int8_t* v_signs,
                                       const void* v_residual, float* out, void* workspace, int64_t workspace_bytes,
                                       void* stream);

/*
 * The NSN variant (mode KVQ_NSN_PCHAN; NSNQuant summary, "Normalize-Shift-Normalize (NSN)" and
 * "Hadamard transform", "implementation details"): after the optional rotation y = R x, per token
 * s1 = ||y|| / sqrt(D) and u1 = y / s1; per block of block_tokens tokens the channel mean o of u1;
 * u2 = u1 - o, s2 = ||u2|| / sqrt(D) (0 when ||u2|| < 2^-16 sqrt(D)), u3 = u2 / s2; then per-channel
 * absmax scales of u3 over the block and rounded codes as for KVQ_NSEP_PCHAN.  Stored (head-major):
 *   codes  as for the other modes;
 *   s1, s2 fp16 [seqs, heads, tokens_per_seq];
 *   offsets fp16 [seqs, heads, tokens_per_seq / B, head_dim]: R^T o, the mean in the original domain;
 *   scales fp16 [seqs, heads, tokens_per_seq / B, head_dim].
 * Dequantization: x^ = s1 (s2 R^T (c * scale) + offset).  Decode score: q . x^ =
 * s1 s2 (R q) . (c * scale) + s1 (q . offset), the byproducts folded in.  Same shapes, dtypes,
 * head_dim (64, 128) and block sizes as the per-channel modes; x, codes, offsets and signs 16-byte
 * aligned; the other arrays 2-byte (scores 4-byte).  The plain quantize / dequantize / score calls
 * refuse this mode; attention and the streaming append do not support it.
 */
kvq_status kvq_quantize_nsn(const kvq_desc* d, const void* x, const int8_t* signs, uint8_t* codes, uint16_t* s1,
                            uint16_t* s2, uint16_t* offsets, uint16_t* scales, void* stream);
kvq_status kvq_dequantize_nsn(const kvq_desc* d, const uint8_t* codes, const uint16_t* s1, const uint16_t* s2,
                              const uint16_t* offsets, const uint16_t* scales, const int8_t* signs, void* y,
                              int32_t y_dtype, void* stream);
kvq_status kvq_score_decode_nsn(const kvq_desc* d, const uint16_t* q, int64_t q_heads, const uint8_t* codes,
                                const uint16_t* s1, const uint16_t* s2, const uint16_t* offsets,
                                const uint16_t* scales, const int8_t* signs, float* scores, void* stream);

/*
 * The RRS activation path into an INT4 GEMM (Rotated Runtime Smooth analysis, "master equation",
 * "term-by-term", "step-by-step flow" and Figure 4).  Activations x [n_tokens, k] and weights
 * w [m, k] (dtype KVQ_F16 or KVQ_BF16, row-major, 16-byte aligned) are rotated alike, row by row:
 * x_rot = x R, w_rot = w R with R the block Hadamard of the other calls (signs [k] int8 then the
 * orthonormal n-point Hadamard, n = hadamard; signs NULL iff hadamard == 0), so x w^T = x_rot w_rot^T.
 * Channels form groups of 128 (the GEMM's K block); k must be a power of two in [128, 8192] for the
 * three quantizer calls and a multiple of 128 for the GEMM.
 *
 * kvq_rrs_smooth_scales: s[g] = max over all n_tokens rows and the 128 channels of group g of
 *   |x_rot| (the runtime smoothing scale s_j = the column max, shared by the group), fp32 [k/128]
 *   (4-byte aligned); n_tokens = 0 gives zeros.
 * kvq_rrs_quantize_act: u = x_rot / s (each column divided by its group's scale; s = 0 gives 0),
 *   then per-token symmetric INT-b: a_t = max_j |u_tj| / Q, code = clamp(rne(u / a_t), -Q, Q)
 *   decided as for the other modes (from the unrounded fp32 a_t; near-ties exact in fp64).
 *   codes [n_tokens, k/2] packed like the cache codes (16-byte aligned); act_scales fp16 [n_tokens]
 *   (2-byte aligned) = a_t.  scales is the fp32 array of kvq_rrs_smooth_scales (any positive values
 *   are accepted).
 * kvq_rrs_quantize_weights: per-output-channel symmetric INT-b of w_rot, b_m = max_j |w_rot_mj| / Q:
 *   codes [m, k/2] and w_scales fp16 [m] (the NAIVE per-token quantizer with each row one token).
 * kvq_rrs_gemm: y[t, m] = a_t b_m sum_g s_g sum_{j in g} cx[t, j] cw[m, j] in fp32 [n_tokens, m]
 *   (4-byte aligned), from the stored fp16 a_t, b_m and the fp32 s: each group's integer product is
 *   exact (int8 matrix cores) and scaled by s_g as an interim result, the groups summed in fp32.
 */
kvq_status kvq_rrs_smooth_scales(const void* x, int64_t n_tokens, int64_t k, int32_t dtype, const int8_t* signs,
                                 int32_t hadamard, float* scales, void* stream);
kvq_status kvq_rrs_quantize_act(const void* x, int64_t n_tokens, int64_t k, int32_t dtype, const int8_t* signs,
                                int32_t hadamard, const float* scales, int32_t bits, uint8_t* codes,
                                uint16_t* act_scales, void* stream);
kvq_status kvq_rrs_quantize_weights(const void* w, int64_t m, int64_t k, int32_t dtype, const int8_t* signs,
                                    int32_t hadamard, int32_t bits, uint8_t* codes, uint16_t* w_scales, void* stream);
kvq_status kvq_rrs_gemm(const uint8_t* x_codes, const uint16_t* act_scales, int64_t n_tokens, const uint8_t* w_codes,
                        const uint16_t* w_scales, int64_t m, int64_t k, const float* scales, float* y, void* stream);

/* Static description of a status code. */
const char* kvq_status_str(kvq_status s);

/* Thread-local description of the last error returned on this thread ("" if none). */
const char* kvq_last_error(void);

/* ABI version: 10000 * major + 100 * minor + patch (1.1: fused decode attention; 1.2: streaming
 * append and attention over a streamed cache; 1.3: the NSN variant; 1.4: the RRS INT4 GEMM path;
 * 1.5: the K and V streaming append in one call). */
int32_t kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
