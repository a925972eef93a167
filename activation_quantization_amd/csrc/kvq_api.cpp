// C ABI of libkvq: argument validation (before any HIP call), sizing and dispatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/kvq.h"
#include "kvq_internal.h"

static_assert(KVQ_ATTENTION_SCRATCH_BYTES == kvq::ATTENTION_SCRATCH_BYTES, "scratch size in the header");

bool kvq::rotation_butterfly() {
  const char* e = std::getenv("KVQ_ROTATION");
  return e != nullptr && std::strcmp(e, "butterfly") == 0;
}

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kvq_status ok() {
  g_last_error.clear();
  return KVQ_OK;
}

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}
bool nsep_mode(int m) { return m == KVQ_NSEP || m == KVQ_NSEP_PCHAN; }
bool pchan_mode(int m) { return m == KVQ_PCHAN || m == KVQ_NSEP_PCHAN; }
bool nsn_mode(int m) { return m == KVQ_NSN_PCHAN; }
bool blocked_mode(int m) { return pchan_mode(m) || nsn_mode(m); }   // per-channel scales over token blocks
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

kvq_status check_desc(const kvq_desc* d) {
  if (!d) return fail(KVQ_ERR_NULL, "descriptor is NULL");
  if (d->seqs < 0 || d->tokens_per_seq < 0)
    return fail(KVQ_ERR_SHAPE, "seqs (%lld) and tokens_per_seq (%lld) must be >= 0",
                (long long)d->seqs, (long long)d->tokens_per_seq);
  if (d->heads <= 0 || d->head_dim <= 0)
    return fail(KVQ_ERR_SHAPE, "heads (%lld) and head_dim (%lld) must be >= 1",
                (long long)d->heads, (long long)d->head_dim);
  if (d->head_dim & 1) return fail(KVQ_ERR_SHAPE, "head_dim %lld is odd", (long long)d->head_dim);
  if (d->reserved != 0) return fail(KVQ_ERR_UNSUPPORTED, "reserved field must be 0");
  if (d->bits < 2 || d->bits > 4) return fail(KVQ_ERR_UNSUPPORTED, "bits %d not in {2, 3, 4}", d->bits);
  if (d->mode < KVQ_NAIVE || d->mode > KVQ_NSN_PCHAN) return fail(KVQ_ERR_UNSUPPORTED, "unknown mode %d", d->mode);
  if (d->dtype != KVQ_F16 && d->dtype != KVQ_BF16)
    return fail(KVQ_ERR_UNSUPPORTED, "input dtype %d must be KVQ_F16 or KVQ_BF16", d->dtype);
  const int64_t D = d->head_dim;
  if (d->hadamard != 0) {
    if (d->hadamard < 0 || !pow2(d->hadamard) || D % d->hadamard != 0)
      return fail(KVQ_ERR_SHAPE, "hadamard %d must be a power of two dividing head_dim %lld", d->hadamard, (long long)D);
    if (d->hadamard < 16 || d->hadamard > 128)
      return fail(KVQ_ERR_UNSUPPORTED, "hadamard %d not in {16, 32, 64, 128}", d->hadamard);
  }
  if (blocked_mode(d->mode)) {
    if (D != 64 && D != 128) return fail(KVQ_ERR_UNSUPPORTED, "per-channel modes need head_dim 64 or 128 (got %lld)", (long long)D);
    if (d->block_tokens <= 0) return fail(KVQ_ERR_SHAPE, "block_tokens %d must be >= 1", d->block_tokens);
    if (d->block_tokens != 64 && d->block_tokens != 128 && d->block_tokens != 256)
      return fail(KVQ_ERR_UNSUPPORTED, "block_tokens %d not in {64, 128, 256}", d->block_tokens);
    if (d->block_tokens == 256 && D == 128)
      return fail(KVQ_ERR_UNSUPPORTED, "block_tokens 256 needs head_dim 64");
    if (d->tokens_per_seq % d->block_tokens != 0)
      return fail(KVQ_ERR_SHAPE, "block_tokens %d does not divide tokens_per_seq %lld", d->block_tokens,
                  (long long)d->tokens_per_seq);
  } else {
    if (!pow2(D) || D < 64 || D > 8192)
      return fail(KVQ_ERR_UNSUPPORTED, "per-token modes need head_dim a power of two in [64, 8192] (got %lld)", (long long)D);
  }
  // grid limits (one workgroup per tile; ids below 2^31)
  const int64_t rows = d->seqs * d->tokens_per_seq;
  if (rows > (int64_t(1) << 40) || d->heads > (int64_t(1) << 20))
    return fail(KVQ_ERR_UNSUPPORTED, "tensor too large");
  const int64_t tiles = blocked_mode(d->mode) ? rows / d->block_tokens * d->heads
                                            : (rows * d->heads * (D / (D >= 128 ? 128 : 64)) + 63) / 64;
  if (tiles >= (int64_t(1) << 31)) return fail(KVQ_ERR_UNSUPPORTED, "too many tiles (%lld)", (long long)tiles);
  return KVQ_OK;
}

bool empty_work(const kvq_desc* d) { return d->seqs == 0 || d->tokens_per_seq == 0; }

kvq_status device_ready() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(KVQ_ERR_HIP, "no HIP device available");
  }
  return KVQ_OK;
}

kvq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

float qmax(int bits) { return float((1 << (bits - 1)) - 1); }

}  // namespace

extern "C" {

kvq_status kvq_validate(const kvq_desc* d) {
  const kvq_status s = check_desc(d);
  return s == KVQ_OK ? ok() : s;
}

int64_t kvq_codes_bytes(const kvq_desc* d) {
  if (check_desc(d) != KVQ_OK) return -1;
  return d->seqs * d->tokens_per_seq * d->heads * d->head_dim / 2;
}

int64_t kvq_norms_count(const kvq_desc* d) {
  if (check_desc(d) != KVQ_OK) return -1;
  return nsep_mode(d->mode) || nsn_mode(d->mode) ? d->seqs * d->tokens_per_seq * d->heads : 0;
}

int64_t kvq_scales_count(const kvq_desc* d) {
  if (check_desc(d) != KVQ_OK) return -1;
  const int64_t rows = d->seqs * d->tokens_per_seq;
  return blocked_mode(d->mode) ? rows / d->block_tokens * d->heads * d->head_dim : rows * d->heads;
}

namespace {
kvq::QuantArgs quant_args(const kvq_desc* d, const void* x, const int8_t* signs, uint8_t* codes, uint16_t* norms,
                          uint16_t* scales) {
  kvq::QuantArgs a{};
  a.x = x; a.signs = signs; a.codes = codes; a.norms = norms; a.scales = scales;
  a.seqs = d->seqs; a.tokens = d->tokens_per_seq; a.heads = d->heads; a.dim = d->head_dim;
  a.block = d->block_tokens;
  a.lg_had = d->hadamard ? ilog2(d->hadamard) : 0;
  a.inv_sqrt_n = d->hadamard ? float(1.0 / std::sqrt(double(d->hadamard))) : 1.f;
  a.q = qmax(d->bits);
  a.scale_mul = float((d->hadamard ? 1.0 / std::sqrt(double(d->hadamard)) : 1.0) / double(qmax(d->bits)));
  a.nsep = nsep_mode(d->mode);
  a.dtype = d->dtype == KVQ_F16 ? kvq::DT_F16 : kvq::DT_BF16;
  a.in_seq_tokens = d->tokens_per_seq;
  a.out_tokens = d->tokens_per_seq;
  a.out_tok0 = 0;
  return a;
}
}  // namespace

kvq_status kvq_quantize(const kvq_desc* d, const void* x, const int8_t* signs, uint8_t* codes,
                        uint16_t* norms, uint16_t* scales, void* stream) {
  kvq_status s = check_desc(d);
  if (s != KVQ_OK) return s;
  if (nsn_mode(d->mode)) return fail(KVQ_ERR_UNSUPPORTED, "mode KVQ_NSN_PCHAN has its own entry points (the _nsn calls)");
  if (empty_work(d)) return ok();
  if (!x || !codes || !scales) return fail(KVQ_ERR_NULL, "x, codes and scales are required");
  if (nsep_mode(d->mode) != (norms != nullptr))
    return fail(KVQ_ERR_NULL, nsep_mode(d->mode) ? "NSEP modes need a norms buffer" : "norms must be NULL without NSEP");
  if ((d->hadamard != 0) != (signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "hadamard needs a signs buffer" : "signs must be NULL when hadamard == 0");
  if (!aligned(x, 16) || !aligned(codes, 16) || (signs && !aligned(signs, 16)))
    return fail(KVQ_ERR_ALIGN, "x, codes and signs must be 16-byte aligned");
  if (!aligned(scales, 2) || (norms && !aligned(norms, 2)))
    return fail(KVQ_ERR_ALIGN, "norms and scales must be 2-byte aligned");
  if ((s = device_ready()) != KVQ_OK) return s;

  const kvq::QuantArgs a = quant_args(d, x, signs, codes, norms, scales);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(pchan_mode(d->mode) ? kvq::launch_quantize_pchan(a, st) : kvq::launch_quantize_ptok(a, st),
                  "quantize");
}

namespace {

// one cache side of a streaming append
struct AppendSide {
  const void* x_new;
  void* residual;
  const int8_t* signs;
  uint8_t* codes;
  uint16_t* norms;
  uint16_t* scales;
};

kvq_status check_append_side(const kvq_desc* d, const AppendSide& c, const char* which) {
  if (!c.x_new || !c.residual || !c.codes || !c.scales)
    return fail(KVQ_ERR_NULL, "%sx_new, residual, codes and scales are required", which);
  if (nsep_mode(d->mode) != (c.norms != nullptr))
    return fail(KVQ_ERR_NULL, nsep_mode(d->mode) ? "%sNSEP modes need a norms buffer" : "%snorms must be NULL without NSEP",
                which);
  if ((d->hadamard != 0) != (c.signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "%shadamard needs a signs buffer" : "%ssigns must be NULL when hadamard == 0",
                which);
  if (!aligned(c.x_new, 16) || !aligned(c.residual, 16) || !aligned(c.codes, 16) || (c.signs && !aligned(c.signs, 16)))
    return fail(KVQ_ERR_ALIGN, "%sx_new, residual, codes and signs must be 16-byte aligned", which);
  if (!aligned(c.scales, 2) || (c.norms && !aligned(c.norms, 2)))
    return fail(KVQ_ERR_ALIGN, "%snorms and scales must be 2-byte aligned", which);
  return KVQ_OK;
}

// the streaming append of n_new tokens to nc (1 or 2) caches of the same shape: the residual
// top-ups and the new residuals of all caches are one copy launch each; a block that fills is
// quantized per cache
kvq_status append_impl(const kvq_desc* d, int64_t tokens_cached, int64_t n_new, const AppendSide* cs, int nc,
                       void* stream) {
  kvq_status s = check_desc(d);
  if (s != KVQ_OK) return s;
  if (!pchan_mode(d->mode))
    return fail(KVQ_ERR_UNSUPPORTED, "the streaming append is for per-channel modes (per-token codes need no residual)");
  if (tokens_cached < 0 || n_new < 0 || tokens_cached > d->tokens_per_seq - n_new)
    return fail(KVQ_ERR_SHAPE, "tokens_cached %lld + n_new %lld must stay within the capacity tokens_per_seq %lld",
                (long long)tokens_cached, (long long)n_new, (long long)d->tokens_per_seq);
  if (d->seqs == 0 || n_new == 0) return ok();
  for (int i = 0; i < nc; ++i)
    if ((s = check_append_side(d, cs[i], nc == 1 ? "" : i == 0 ? "K side: " : "V side: ")) != KVQ_OK) return s;
  if ((s = device_ready()) != KVQ_OK) return s;

  // the residual holds tokens [whole, tokens_cached) of every sequence in its first slots
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t B = d->block_tokens, S = d->seqs;
  const int64_t rowb = d->heads * d->head_dim * 2;              // bytes per token (fp16 / bf16)
  auto quantize_blocks = [&](const AppendSide& c, const void* x, int64_t tokens, int64_t in_seq_tokens, int64_t out_tok0) {
    kvq::QuantArgs a = quant_args(d, x, c.signs, c.codes, c.norms, c.scales);
    a.tokens = tokens; a.in_seq_tokens = in_seq_tokens; a.out_tok0 = out_tok0;
    return kvq::launch_quantize_pchan(a, st);
  };
  const void* src[2];
  void* dst[2];
  int64_t whole = tokens_cached - tokens_cached % B, r = tokens_cached % B, used = 0;
  hipError_t e = hipSuccess;
  if (r > 0) {                                                   // top up the residuals
    const int64_t k = n_new < B - r ? n_new : B - r;
    for (int i = 0; i < nc; ++i) {
      src[i] = cs[i].x_new;
      dst[i] = static_cast<unsigned char*>(cs[i].residual) + r * rowb;
    }
    e = kvq::launch_copy_tokens(src, dst, nc, S, k, rowb, n_new, B, st);
    used = k;
    r += k;
    if (r == B) {                                                // they filled: quantize them into the caches
      for (int i = 0; i < nc && e == hipSuccess; ++i) e = quantize_blocks(cs[i], cs[i].residual, B, B, whole);
      whole += B;
      r = 0;
    }
  }
  const int64_t full = (n_new - used) / B * B;                   // whole blocks straight from x_new
  if (full > 0) {
    for (int i = 0; i < nc && e == hipSuccess; ++i)
      e = quantize_blocks(cs[i], static_cast<const unsigned char*>(cs[i].x_new) + used * rowb, full, n_new, whole);
    used += full;
  }
  if (e == hipSuccess && used < n_new) {                         // the tails start new residuals
    for (int i = 0; i < nc; ++i) {
      src[i] = static_cast<const unsigned char*>(cs[i].x_new) + used * rowb;
      dst[i] = cs[i].residual;
    }
    e = kvq::launch_copy_tokens(src, dst, nc, S, n_new - used, rowb, n_new, B, st);
  }
  return launched(e, "append");
}

}  // namespace

kvq_status kvq_append(const kvq_desc* d, int64_t tokens_cached, const void* x_new, int64_t n_new, void* residual,
                      const int8_t* signs, uint8_t* codes, uint16_t* norms, uint16_t* scales, void* stream) {
  const AppendSide c{x_new, residual, signs, codes, norms, scales};
  return append_impl(d, tokens_cached, n_new, &c, 1, stream);
}

kvq_status kvq_append_kv(const kvq_desc* d, int64_t tokens_cached, int64_t n_new, const void* k_new, void* k_residual,
                         const int8_t* k_signs, uint8_t* k_codes, uint16_t* k_norms, uint16_t* k_scales,
                         const void* v_new, void* v_residual, const int8_t* v_signs, uint8_t* v_codes,
                         uint16_t* v_norms, uint16_t* v_scales, void* stream) {
  const AppendSide c[2] = {{k_new, k_residual, k_signs, k_codes, k_norms, k_scales},
                           {v_new, v_residual, v_signs, v_codes, v_norms, v_scales}};
  return append_impl(d, tokens_cached, n_new, c, 2, stream);
}

kvq_status kvq_dequantize(const kvq_desc* d, const uint8_t* codes, const uint16_t* norms,
                          const uint16_t* scales, const int8_t* signs, void* y, int32_t y_dtype, void* stream) {
  kvq_status s = check_desc(d);
  if (s != KVQ_OK) return s;
  if (nsn_mode(d->mode)) return fail(KVQ_ERR_UNSUPPORTED, "mode KVQ_NSN_PCHAN has its own entry points (the _nsn calls)");
  if (y_dtype != KVQ_F16 && y_dtype != KVQ_BF16 && y_dtype != KVQ_F32)
    return fail(KVQ_ERR_UNSUPPORTED, "output dtype %d not in {F16, BF16, F32}", y_dtype);
  if (empty_work(d)) return ok();
  if (!codes || !scales || !y) return fail(KVQ_ERR_NULL, "codes, scales and y are required");
  if (nsep_mode(d->mode) != (norms != nullptr))
    return fail(KVQ_ERR_NULL, nsep_mode(d->mode) ? "NSEP modes need a norms buffer" : "norms must be NULL without NSEP");
  if ((d->hadamard != 0) != (signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "hadamard needs a signs buffer" : "signs must be NULL when hadamard == 0");
  if (!aligned(y, 16) || !aligned(codes, 16) || (signs && !aligned(signs, 16)))
    return fail(KVQ_ERR_ALIGN, "y, codes and signs must be 16-byte aligned");
  if (!aligned(scales, 2) || (norms && !aligned(norms, 2)))
    return fail(KVQ_ERR_ALIGN, "norms and scales must be 2-byte aligned");
  if ((s = device_ready()) != KVQ_OK) return s;

  kvq::DequantArgs a{};
  a.codes = codes; a.norms = norms; a.scales = scales; a.signs = signs; a.y = y;
  a.seqs = d->seqs; a.tokens = d->tokens_per_seq; a.heads = d->heads; a.dim = d->head_dim;
  a.block = d->block_tokens;
  a.lg_had = d->hadamard ? ilog2(d->hadamard) : 0;
  a.inv_sqrt_n = d->hadamard ? float(1.0 / std::sqrt(double(d->hadamard))) : 1.f;
  a.nsep = nsep_mode(d->mode);
  a.per_channel = pchan_mode(d->mode);
  a.out_dtype = y_dtype == KVQ_F16 ? kvq::DT_F16 : y_dtype == KVQ_BF16 ? kvq::DT_BF16 : kvq::DT_F32;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(a.per_channel ? kvq::launch_dequantize_pchan(a, st) : kvq::launch_dequantize_ptok(a, st),
                  "dequantize");
}

kvq_status kvq_score_decode(const kvq_desc* d, const uint16_t* q, int64_t q_heads, const uint8_t* codes,
                            const uint16_t* norms, const uint16_t* scales, const int8_t* signs, float* scores,
                            void* stream) {
  kvq_status s = check_desc(d);
  if (s != KVQ_OK) return s;
  if (nsn_mode(d->mode)) return fail(KVQ_ERR_UNSUPPORTED, "mode KVQ_NSN_PCHAN has its own entry points (the _nsn calls)");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "decode score needs head_dim 64 or 128 (got %lld)", (long long)d->head_dim);
  if (q_heads <= 0 || q_heads % d->heads != 0)
    return fail(KVQ_ERR_SHAPE, "q_heads %lld must be a positive multiple of heads %lld", (long long)q_heads,
                (long long)d->heads);
  if (q_heads / d->heads > 16) return fail(KVQ_ERR_UNSUPPORTED, "at most 16 query heads per KV head");
  if (empty_work(d)) return ok();
  if (!q || !codes || !scales || !scores) return fail(KVQ_ERR_NULL, "q, codes, scales and scores are required");
  if (nsep_mode(d->mode) != (norms != nullptr))
    return fail(KVQ_ERR_NULL, nsep_mode(d->mode) ? "NSEP modes need a norms buffer" : "norms must be NULL without NSEP");
  if ((d->hadamard != 0) != (signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "hadamard needs a signs buffer" : "signs must be NULL when hadamard == 0");
  if (!aligned(codes, 16)) return fail(KVQ_ERR_ALIGN, "codes must be 16-byte aligned");
  if (!aligned(q, 2) || !aligned(scales, 2) || (norms && !aligned(norms, 2)) || !aligned(scores, 4))
    return fail(KVQ_ERR_ALIGN, "q, norms, scales must be 2-byte and scores 4-byte aligned");
  if ((s = device_ready()) != KVQ_OK) return s;

  kvq::ScoreArgs a{};
  a.q = q; a.codes = codes; a.norms = norms; a.scales = scales; a.signs = signs; a.scores = scores;
  a.seqs = d->seqs; a.tokens = d->tokens_per_seq; a.heads = d->heads; a.dim = d->head_dim; a.q_heads = q_heads;
  a.block = d->block_tokens;
  a.lg_had = d->hadamard ? ilog2(d->hadamard) : 0;
  a.inv_sqrt_n = d->hadamard ? float(1.0 / std::sqrt(double(d->hadamard))) : 1.f;
  a.nsep = nsep_mode(d->mode);
  a.per_channel = pchan_mode(d->mode);
  return launched(kvq::launch_score_decode(a, static_cast<hipStream_t>(stream)), "score_decode");
}

kvq_status kvq_quantize_nsn(const kvq_desc* d, const void* x, const int8_t* signs, uint8_t* codes, uint16_t* s1,
                            uint16_t* s2, uint16_t* offsets, uint16_t* scales, void* stream) {
  kvq_status s = check_desc(d);
  if (s != KVQ_OK) return s;
  if (!nsn_mode(d->mode)) return fail(KVQ_ERR_UNSUPPORTED, "the _nsn calls need mode KVQ_NSN_PCHAN");
  if (empty_work(d)) return ok();
  if (!x || !codes || !s1 || !s2 || !offsets || !scales)
    return fail(KVQ_ERR_NULL, "x, codes, s1, s2, offsets and scales are required");
  if ((d->hadamard != 0) != (signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "hadamard needs a signs buffer" : "signs must be NULL when hadamard == 0");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(offsets, 16) || (signs && !aligned(signs, 16)))
    return fail(KVQ_ERR_ALIGN, "x, codes, offsets and signs must be 16-byte aligned");
  if (!aligned(s1, 2) || !aligned(s2, 2) || !aligned(scales, 2))
    return fail(KVQ_ERR_ALIGN, "s1, s2 and scales must be 2-byte aligned");
  if ((s = device_ready()) != KVQ_OK) return s;
  kvq::NsnArgs a{};
  a.x = x; a.signs = signs; a.codes = codes; a.s1 = s1; a.s2 = s2; a.offsets = offsets; a.scales = scales;
  a.seqs = d->seqs; a.tokens = d->tokens_per_seq; a.heads = d->heads; a.dim = d->head_dim;
  a.block = d->block_tokens;
  a.lg_had = d->hadamard ? ilog2(d->hadamard) : 0;
  a.q = (1 << (d->bits - 1)) - 1;
  a.dtype = d->dtype == KVQ_F16 ? kvq::DT_F16 : kvq::DT_BF16;
  return launched(kvq::launch_quantize_nsn(a, static_cast<hipStream_t>(stream)), "quantize_nsn");
}

kvq_status kvq_dequantize_nsn(const kvq_desc* d, const uint8_t* codes, const uint16_t* s1, const uint16_t* s2,
                              const uint16_t* offsets, const uint16_t* scales, const int8_t* signs, void* y,
                              int32_t y_dtype, void* stream) {
  kvq_status s = check_desc(d);
  if (s != KVQ_OK) return s;
  if (!nsn_mode(d->mode)) return fail(KVQ_ERR_UNSUPPORTED, "the _nsn calls need mode KVQ_NSN_PCHAN");
  if (y_dtype != KVQ_F16 && y_dtype != KVQ_BF16 && y_dtype != KVQ_F32)
    return fail(KVQ_ERR_UNSUPPORTED, "output dtype %d not in {F16, BF16, F32}", y_dtype);
  if (empty_work(d)) return ok();
  if (!codes || !s1 || !s2 || !offsets || !scales || !y)
    return fail(KVQ_ERR_NULL, "codes, s1, s2, offsets, scales and y are required");
  if ((d->hadamard != 0) != (signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "hadamard needs a signs buffer" : "signs must be NULL when hadamard == 0");
  if (!aligned(y, 16) || !aligned(codes, 16) || !aligned(offsets, 16) || (signs && !aligned(signs, 16)))
    return fail(KVQ_ERR_ALIGN, "y, codes, offsets and signs must be 16-byte aligned");
  if (!aligned(s1, 2) || !aligned(s2, 2) || !aligned(scales, 2))
    return fail(KVQ_ERR_ALIGN, "s1, s2 and scales must be 2-byte aligned");
  if ((s = device_ready()) != KVQ_OK) return s;
  kvq::DequantArgs a{};
  a.codes = codes; a.norms = s1; a.s2 = s2; a.offsets = offsets; a.scales = scales; a.signs = signs; a.y = y;
  a.seqs = d->seqs; a.tokens = d->tokens_per_seq; a.heads = d->heads; a.dim = d->head_dim;
  a.block = d->block_tokens;
  a.lg_had = d->hadamard ? ilog2(d->hadamard) : 0;
  a.inv_sqrt_n = d->hadamard ? float(1.0 / std::sqrt(double(d->hadamard))) : 1.f;
  a.nsep = 1;
  a.per_channel = 1;
  a.out_dtype = y_dtype == KVQ_F16 ? kvq::DT_F16 : y_dtype == KVQ_BF16 ? kvq::DT_BF16 : kvq::DT_F32;
  return launched(kvq::launch_dequantize_nsn(a, static_cast<hipStream_t>(stream)), "dequantize_nsn");
}

kvq_status kvq_score_decode_nsn(const kvq_desc* d, const uint16_t* q, int64_t q_heads, const uint8_t* codes,
                                const uint16_t* s1, const uint16_t* s2, const uint16_t* offsets,
                                const uint16_t* scales, const int8_t* signs, float* scores, void* stream) {
  kvq_status s = check_desc(d);
  if (s != KVQ_OK) return s;
  if (!nsn_mode(d->mode)) return fail(KVQ_ERR_UNSUPPORTED, "the _nsn calls need mode KVQ_NSN_PCHAN");
  if (q_heads <= 0 || q_heads % d->heads != 0)
    return fail(KVQ_ERR_SHAPE, "q_heads %lld must be a positive multiple of heads %lld", (long long)q_heads,
                (long long)d->heads);
  if (q_heads / d->heads > 16) return fail(KVQ_ERR_UNSUPPORTED, "at most 16 query heads per KV head");
  if (empty_work(d)) return ok();
  if (!q || !codes || !s1 || !s2 || !offsets || !scales || !scores)
    return fail(KVQ_ERR_NULL, "q, codes, s1, s2, offsets, scales and scores are required");
  if ((d->hadamard != 0) != (signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "hadamard needs a signs buffer" : "signs must be NULL when hadamard == 0");
  if (!aligned(codes, 16)) return fail(KVQ_ERR_ALIGN, "codes must be 16-byte aligned");
  if (!aligned(q, 2) || !aligned(s1, 2) || !aligned(s2, 2) || !aligned(offsets, 2) || !aligned(scales, 2) ||
      !aligned(scores, 4))
    return fail(KVQ_ERR_ALIGN, "q, s1, s2, offsets, scales must be 2-byte and scores 4-byte aligned");
  if ((s = device_ready()) != KVQ_OK) return s;
  kvq::ScoreArgs a{};
  a.q = q; a.codes = codes; a.norms = s1; a.s2 = s2; a.offsets = offsets; a.scales = scales; a.signs = signs;
  a.scores = scores;
  a.seqs = d->seqs; a.tokens = d->tokens_per_seq; a.heads = d->heads; a.dim = d->head_dim; a.q_heads = q_heads;
  a.block = d->block_tokens;
  a.lg_had = d->hadamard ? ilog2(d->hadamard) : 0;
  a.inv_sqrt_n = d->hadamard ? float(1.0 / std::sqrt(double(d->hadamard))) : 1.f;
  a.nsep = 1;
  a.per_channel = 1;
  a.nsn = 1;
  return launched(kvq::launch_score_decode(a, static_cast<hipStream_t>(stream)), "score_decode_nsn");
}

namespace {
kvq::AttnArgs attn_args(const kvq_desc* d, int64_t q_heads) {
  kvq::AttnArgs a{};
  a.seqs = d->seqs; a.tokens = d->tokens_per_seq; a.heads = d->heads; a.dim = d->head_dim; a.q_heads = q_heads;
  a.stream_tokens = d->tokens_per_seq;
  a.block = d->block_tokens;
  a.lg_had = d->hadamard ? ilog2(d->hadamard) : 0;
  a.inv_sqrt_n = d->hadamard ? float(1.0 / std::sqrt(double(d->hadamard))) : 1.f;
  a.nsep = nsep_mode(d->mode);
  return a;
}

kvq_status check_attention(const kvq_desc* d, int64_t q_heads) {
  kvq_status s = check_desc(d);
  if (s != KVQ_OK) return s;
  if (!pchan_mode(d->mode)) return fail(KVQ_ERR_UNSUPPORTED, "fused attention needs a per-channel mode (PCHAN or NSEP_PCHAN)");
  if (d->head_dim != 128) return fail(KVQ_ERR_UNSUPPORTED, "fused attention needs head_dim 128 (got %lld)", (long long)d->head_dim);
  if (d->block_tokens != 64 && d->block_tokens != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "fused attention needs block_tokens 64 or 128 (got %d)", d->block_tokens);
  if (q_heads <= 0 || q_heads % d->heads != 0)
    return fail(KVQ_ERR_SHAPE, "q_heads %lld must be a positive multiple of heads %lld", (long long)q_heads,
                (long long)d->heads);
  if (q_heads / d->heads > 4) return fail(KVQ_ERR_UNSUPPORTED, "fused attention takes at most 4 query heads per KV head");
  if (d->seqs > 0 && d->tokens_per_seq == 0) return fail(KVQ_ERR_SHAPE, "attention over an empty cache");
  return ok();
}
}  // namespace

int64_t kvq_attention_workspace_bytes(const kvq_desc* d, int64_t q_heads) {
  if (check_attention(d, q_heads) != KVQ_OK) return -1;
  const kvq::AttnArgs a = attn_args(d, q_heads);
  return a.seqs * q_heads * kvq::attention_partials(a) * (d->head_dim + 2) * (int64_t)sizeof(float);
}

namespace {
// shared by both attention entry points: tokens_cached tokens per sequence, the whole blocks in
// the packed caches and the rest (fewer than block_tokens) in the residuals
kvq_status attention_impl(const kvq_desc* d, int64_t tokens_cached, const uint16_t* q, int64_t q_heads,
                          const uint8_t* k_codes, const uint16_t* k_norms, const uint16_t* k_scales,
                          const int8_t* k_signs, const void* k_res, const uint8_t* v_codes, const uint16_t* v_norms,
                          const uint16_t* v_scales, const int8_t* v_signs, const void* v_res, float* out,
                          void* workspace, int64_t workspace_bytes, void* stream, const char* what,
                          bool static_scratch = false) {
  kvq_status s;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !out)
    return fail(KVQ_ERR_NULL, "q, codes, scales and out are required");
  if (!static_scratch && !workspace) return fail(KVQ_ERR_NULL, "workspace is required");
  const int64_t nres = tokens_cached % d->block_tokens;
  if (nres > 0 && (!k_res || !v_res)) return fail(KVQ_ERR_NULL, "a partly filled block needs both residual buffers");
  if ((k_res && !aligned(k_res, 2)) || (v_res && !aligned(v_res, 2)))
    return fail(KVQ_ERR_ALIGN, "residuals must be 2-byte aligned");
  const bool nsep = nsep_mode(d->mode);
  if (nsep != (k_norms != nullptr) || nsep != (v_norms != nullptr))
    return fail(KVQ_ERR_NULL, nsep ? "NSEP modes need both norms buffers" : "norms must be NULL without NSEP");
  if ((d->hadamard != 0) != (k_signs != nullptr) || (d->hadamard != 0) != (v_signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "hadamard needs both signs buffers" : "signs must be NULL when hadamard == 0");
  if (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_scales, 16) || !aligned(v_scales, 16) ||
      (k_signs && !aligned(k_signs, 16)) || (v_signs && !aligned(v_signs, 16)))
    return fail(KVQ_ERR_ALIGN, "codes, scales and signs must be 16-byte aligned");
  if (!aligned(q, 2) || (k_norms && !aligned(k_norms, 2)) || (v_norms && !aligned(v_norms, 2)) || !aligned(out, 4) ||
      (!static_scratch && !aligned(workspace, 4)))
    return fail(KVQ_ERR_ALIGN, "q and norms must be 2-byte, out and workspace 4-byte aligned");
  const int64_t need = kvq_attention_workspace_bytes(d, q_heads);
  if (static_scratch) {
    if (need > kvq::ATTENTION_SCRATCH_BYTES)
      return fail(KVQ_ERR_UNSUPPORTED,
                  "%s: the partials need %lld bytes, more than the %lld-byte static scratch; use "
                  "kvq_attention_decode with a workspace", what, (long long)need, (long long)kvq::ATTENTION_SCRATCH_BYTES);
  } else if (workspace_bytes < need) {
    return fail(KVQ_ERR_SHAPE, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes, (long long)need);
  }
  if ((s = device_ready()) != KVQ_OK) return s;
  if (static_scratch) {
    float* p = nullptr;
    const hipError_t e = kvq::attention_scratch(&p);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: static scratch lookup failed: %s", what, hipGetErrorString(e));
    workspace = p;
  }

  kvq::AttnArgs a = attn_args(d, q_heads);
  a.tokens = tokens_cached - nres;
  a.q = q; a.k_codes = k_codes; a.k_norms = k_norms; a.k_scales = k_scales; a.k_signs = k_signs;
  a.v_codes = v_codes; a.v_norms = v_norms; a.v_scales = v_scales; a.v_signs = v_signs;
  a.out = out; a.ws = static_cast<float*>(workspace);
  a.k_res = k_res; a.v_res = v_res; a.nres = (int32_t)nres;
  a.res_dtype = d->dtype == KVQ_F16 ? kvq::DT_F16 : kvq::DT_BF16;
  return launched(kvq::launch_attention_decode(a, static_cast<hipStream_t>(stream)), what);
}
}  // namespace

kvq_status kvq_attention_decode(const kvq_desc* d, const uint16_t* q, int64_t q_heads, const uint8_t* k_codes,
                                const uint16_t* k_norms, const uint16_t* k_scales, const int8_t* k_signs,
                                const uint8_t* v_codes, const uint16_t* v_norms, const uint16_t* v_scales,
                                const int8_t* v_signs, float* out, void* workspace, int64_t workspace_bytes,
                                void* stream) {
  kvq_status s = check_attention(d, q_heads);
  if (s != KVQ_OK) return s;
  if (d->seqs == 0) return ok();
  return attention_impl(d, d->tokens_per_seq, q, q_heads, k_codes, k_norms, k_scales, k_signs, nullptr, v_codes,
                        v_norms, v_scales, v_signs, nullptr, out, workspace, workspace_bytes, stream, "attention_decode");
}

kvq_status kvq_attention_decode_noalloc(const kvq_desc* d, const uint16_t* q, int64_t q_heads, const uint8_t* k_codes,
                                        const uint16_t* k_norms, const uint16_t* k_scales, const int8_t* k_signs,
                                        const uint8_t* v_codes, const uint16_t* v_norms, const uint16_t* v_scales,
                                        const int8_t* v_signs, float* out, void* stream) {
  kvq_status s = check_attention(d, q_heads);
  if (s != KVQ_OK) return s;
  if (d->seqs == 0) return ok();
  return attention_impl(d, d->tokens_per_seq, q, q_heads, k_codes, k_norms, k_scales, k_signs, nullptr, v_codes,
                        v_norms, v_scales, v_signs, nullptr, out, nullptr, 0, stream, "attention_decode_noalloc", true);
}

kvq_status kvq_attention_decode_stream(const kvq_desc* d, int64_t tokens_cached, const uint16_t* q, int64_t q_heads,
                                       const uint8_t* k_codes, const uint16_t* k_norms, const uint16_t* k_scales,
                                       const int8_t* k_signs, const void* k_residual, const uint8_t* v_codes,
                                       const uint16_t* v_norms, const uint16_t* v_scales, const int8_t* v_signs,
                                       const void* v_residual, float* out, void* workspace, int64_t workspace_bytes,
                                       void* stream) {
  kvq_status s = check_attention(d, q_heads);
  if (s != KVQ_OK) return s;
  if (tokens_cached < 1 || tokens_cached > d->tokens_per_seq)
    return fail(KVQ_ERR_SHAPE, "tokens_cached %lld must be in [1, tokens_per_seq %lld]", (long long)tokens_cached,
                (long long)d->tokens_per_seq);
  if (d->seqs == 0) return ok();
  return attention_impl(d, tokens_cached, q, q_heads, k_codes, k_norms, k_scales, k_signs, k_residual, v_codes,
                        v_norms, v_scales, v_signs, v_residual, out, workspace, workspace_bytes, stream,
                        "attention_decode_stream");
}

// ----------------------------------------------------------------------------- RRS INT4 GEMM path
}  // extern "C"

namespace {

// the per-token descriptor of an [n, k] activation (or weight) matrix: one sequence of n tokens,
// one head of k channels, NAIVE mode
kvq_status rrs_desc(kvq_desc* d, int64_t n, int64_t k, int32_t dtype, int32_t hadamard, int32_t bits, const char* what) {
  if (n < 0) return fail(KVQ_ERR_SHAPE, "%s: row count %lld must be >= 0", what, (long long)n);
  if (k < 128 || k > 8192 || (k & (k - 1)) != 0)
    return fail(KVQ_ERR_UNSUPPORTED, "%s: k %lld must be a power of two in [128, 8192] (groups of 128 channels)", what,
                (long long)k);
  *d = kvq_desc{};
  d->seqs = 1; d->tokens_per_seq = n; d->heads = 1; d->head_dim = k;
  d->bits = bits; d->mode = KVQ_NAIVE; d->block_tokens = 0; d->hadamard = hadamard; d->dtype = dtype;
  return check_desc(d);
}

kvq_status rrs_inputs(const kvq_desc* d, const void* x, const int8_t* signs) {
  if (!x) return fail(KVQ_ERR_NULL, "the input matrix is required");
  if ((d->hadamard != 0) != (signs != nullptr))
    return fail(KVQ_ERR_NULL, d->hadamard ? "hadamard needs a signs buffer" : "signs must be NULL when hadamard == 0");
  if (!aligned(x, 16) || (signs && !aligned(signs, 16))) return fail(KVQ_ERR_ALIGN, "x and signs must be 16-byte aligned");
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_rrs_smooth_scales(const void* x, int64_t n_tokens, int64_t k, int32_t dtype, const int8_t* signs,
                                 int32_t hadamard, float* scales, void* stream) {
  kvq_desc d;
  kvq_status s = rrs_desc(&d, n_tokens, k, dtype, hadamard, 4, "rrs_smooth_scales");
  if (s != KVQ_OK) return s;
  if (!scales) return fail(KVQ_ERR_NULL, "scales is required");
  if (!aligned(scales, 4)) return fail(KVQ_ERR_ALIGN, "scales must be 4-byte aligned");
  if (n_tokens > 0 && (s = rrs_inputs(&d, x, signs)) != KVQ_OK) return s;
  if ((s = device_ready()) != KVQ_OK) return s;
  const kvq::QuantArgs a = quant_args(&d, x, signs, nullptr, nullptr, nullptr);
  return launched(kvq::launch_rrs_colmax(a, scales, static_cast<hipStream_t>(stream)), "rrs_smooth_scales");
}

kvq_status kvq_rrs_quantize_act(const void* x, int64_t n_tokens, int64_t k, int32_t dtype, const int8_t* signs,
                                int32_t hadamard, const float* scales, int32_t bits, uint8_t* codes,
                                uint16_t* act_scales, void* stream) {
  kvq_desc d;
  kvq_status s = rrs_desc(&d, n_tokens, k, dtype, hadamard, bits, "rrs_quantize_act");
  if (s != KVQ_OK) return s;
  if (n_tokens == 0) return ok();
  if ((s = rrs_inputs(&d, x, signs)) != KVQ_OK) return s;
  if (!scales || !codes || !act_scales) return fail(KVQ_ERR_NULL, "scales, codes and act_scales are required");
  if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(act_scales, 2))
    return fail(KVQ_ERR_ALIGN, "codes must be 16-byte, scales 4-byte and act_scales 2-byte aligned");
  if ((s = device_ready()) != KVQ_OK) return s;
  kvq::QuantArgs a = quant_args(&d, x, signs, codes, nullptr, act_scales);
  a.seg_div = scales;
  return launched(kvq::launch_quantize_ptok(a, static_cast<hipStream_t>(stream)), "rrs_quantize_act");
}

kvq_status kvq_rrs_quantize_weights(const void* w, int64_t m, int64_t k, int32_t dtype, const int8_t* signs,
                                    int32_t hadamard, int32_t bits, uint8_t* codes, uint16_t* w_scales, void* stream) {
  kvq_desc d;
  kvq_status s = rrs_desc(&d, m, k, dtype, hadamard, bits, "rrs_quantize_weights");
  if (s != KVQ_OK) return s;
  if (m == 0) return ok();
  if ((s = rrs_inputs(&d, w, signs)) != KVQ_OK) return s;
  if (!codes || !w_scales) return fail(KVQ_ERR_NULL, "codes and w_scales are required");
  if (!aligned(codes, 16) || !aligned(w_scales, 2)) return fail(KVQ_ERR_ALIGN, "codes must be 16-byte and w_scales 2-byte aligned");
  if ((s = device_ready()) != KVQ_OK) return s;
  const kvq::QuantArgs a = quant_args(&d, w, signs, codes, nullptr, w_scales);
  return launched(kvq::launch_quantize_ptok(a, static_cast<hipStream_t>(stream)), "rrs_quantize_weights");
}

kvq_status kvq_rrs_gemm(const uint8_t* x_codes, const uint16_t* act_scales, int64_t n_tokens, const uint8_t* w_codes,
                        const uint16_t* w_scales, int64_t m, int64_t k, const float* scales, float* y, void* stream) {
  if (n_tokens < 0 || m < 0) return fail(KVQ_ERR_SHAPE, "n_tokens %lld and m %lld must be >= 0", (long long)n_tokens, (long long)m);
  if (k < 128 || k % 128 != 0 || k > (int64_t(1) << 20))
    return fail(KVQ_ERR_UNSUPPORTED, "k %lld must be a multiple of 128 in [128, 2^20]", (long long)k);
  if (n_tokens == 0 || m == 0) return ok();
  if ((n_tokens + 127) / 128 * ((m + 127) / 128) >= (int64_t(1) << 31)) return fail(KVQ_ERR_UNSUPPORTED, "too many output tiles");
  if (!x_codes || !act_scales || !w_codes || !w_scales || !scales || !y)
    return fail(KVQ_ERR_NULL, "x_codes, act_scales, w_codes, w_scales, scales and y are required");
  if (!aligned(x_codes, 16) || !aligned(w_codes, 16) || !aligned(act_scales, 2) || !aligned(w_scales, 2) ||
      !aligned(scales, 4) || !aligned(y, 4))
    return fail(KVQ_ERR_ALIGN, "codes must be 16-byte, scales and y 4-byte, act_scales and w_scales 2-byte aligned");
  kvq_status s;
  if ((s = device_ready()) != KVQ_OK) return s;
  kvq::RrsGemmArgs a{};
  a.x_codes = x_codes; a.x_scales = act_scales; a.w_codes = w_codes; a.w_scales = w_scales;
  a.s = scales; a.y = y; a.n = n_tokens; a.m = m; a.k = k;
  return launched(kvq::launch_rrs_gemm(a, static_cast<hipStream_t>(stream)), "rrs_gemm");
}

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_NULL: return "KVQ_ERR_NULL: missing or forbidden pointer";
    case KVQ_ERR_ALIGN: return "KVQ_ERR_ALIGN: misaligned buffer";
    case KVQ_ERR_SHAPE: return "KVQ_ERR_SHAPE: inconsistent sizes";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED: parameters outside the built kernels";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP: HIP runtime error";
  }
  return "unknown kvq_status";
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

int32_t kvq_version(void) { return 10500; }

}  // extern "C"
