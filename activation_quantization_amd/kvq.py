"""Thin ctypes binding of libkvq (argument marshalling only; every step runs in HIP kernels).

The names mirror the C ABI in include/kvq.h: quantize / dequantize / score_decode.  Tensors
are torch tensors on the current HIP device (torch is used for device memory and streams);
outputs are allocated with torch when not supplied.  There is no CPU fallback: if libkvq.so
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

OK, ERR_NULL, ERR_ALIGN, ERR_SHAPE, ERR_UNSUPPORTED, ERR_HIP = range(6)
MODES = {"naive": 0, "nsep": 1, "pchan": 2, "nsep_pchan": 3, "nsn_pchan": 4}
DTYPES = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2}
DTYPE_NAMES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


class KvqDesc(ctypes.Structure):
    _fields_ = [("seqs", ctypes.c_int64), ("tokens_per_seq", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32), ("hadamard", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_SIGNATURES = {
    "kvq_validate": (ctypes.c_int, [ctypes.POINTER(KvqDesc)]),
    "kvq_codes_bytes": (ctypes.c_int64, [ctypes.POINTER(KvqDesc)]),
    "kvq_norms_count": (ctypes.c_int64, [ctypes.POINTER(KvqDesc)]),
    "kvq_scales_count": (ctypes.c_int64, [ctypes.POINTER(KvqDesc)]),
    "kvq_quantize": (ctypes.c_int, [ctypes.POINTER(KvqDesc), _P, _P, _P, _P, _P, _P]),
    "kvq_dequantize": (ctypes.c_int, [ctypes.POINTER(KvqDesc), _P, _P, _P, _P, _P, ctypes.c_int32, _P]),
    "kvq_score_decode": (ctypes.c_int, [ctypes.POINTER(KvqDesc), _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P]),
    "kvq_attention_workspace_bytes": (ctypes.c_int64, [ctypes.POINTER(KvqDesc), ctypes.c_int64]),
    "kvq_attention_decode": (ctypes.c_int, [ctypes.POINTER(KvqDesc), _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P, _P, ctypes.c_int64, _P]),
    "kvq_attention_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(KvqDesc), _P, ctypes.c_int64, _P, _P, _P, _P, _P,
                                                    _P, _P, _P, _P, _P]),
    "kvq_append": (ctypes.c_int, [ctypes.POINTER(KvqDesc), ctypes.c_int64, _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P]),
    "kvq_append_kv": (ctypes.c_int, [ctypes.POINTER(KvqDesc), ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _P, _P, _P,
                                     _P, _P, _P, _P, _P, _P, _P]),
    "kvq_attention_decode_stream": (ctypes.c_int, [ctypes.POINTER(KvqDesc), ctypes.c_int64, _P, ctypes.c_int64,
                                                   _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                   ctypes.c_int64, _P]),
    "kvq_quantize_nsn": (ctypes.c_int, [ctypes.POINTER(KvqDesc), _P, _P, _P, _P, _P, _P, _P, _P]),
    "kvq_dequantize_nsn": (ctypes.c_int, [ctypes.POINTER(KvqDesc), _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P]),
    "kvq_score_decode_nsn": (ctypes.c_int, [ctypes.POINTER(KvqDesc), _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P,
                                            _P]),
    "kvq_rrs_smooth_scales": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _P, ctypes.c_int32,
                                             _P, _P]),
    "kvq_rrs_quantize_act": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _P, ctypes.c_int32,
                                            _P, ctypes.c_int32, _P, _P, _P]),
    "kvq_rrs_quantize_weights": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _P,
                                                ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "kvq_rrs_gemm": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P, _P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P]),
    "kvq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "kvq_last_error": (ctypes.c_char_p, []),
    "kvq_version": (ctypes.c_int32, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so (built in-tree by activation_quantization_amd.build_lib)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m activation_quantization_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        L = lib()
        super().__init__(f"{what}: {L.kvq_status_str(status).decode()} -- {L.kvq_last_error().decode()}")
        self.status = status


@dataclasses.dataclass(frozen=True)
class Desc:
    """Python mirror of kvq_desc; x is [seqs * tokens_per_seq, heads, head_dim]."""
    seqs: int
    tokens_per_seq: int
    heads: int
    head_dim: int
    bits: int = 4
    mode: str = "nsep_pchan"
    block_tokens: int = 128
    hadamard: int = 0
    dtype: torch.dtype = torch.float16

    def c(self) -> KvqDesc:
        return KvqDesc(self.seqs, self.tokens_per_seq, self.heads, self.head_dim, self.bits,
                       MODES[self.mode], self.block_tokens if "pchan" in self.mode else 0,
                       self.hadamard, DTYPES[self.dtype], 0)

    @property
    def nsep(self) -> bool:
        return self.mode in ("nsep", "nsep_pchan")

    @property
    def per_channel(self) -> bool:
        return self.mode in ("pchan", "nsep_pchan", "nsn_pchan")

    @property
    def nsn(self) -> bool:
        return self.mode == "nsn_pchan"

    @property
    def rows(self) -> int:
        return self.seqs * self.tokens_per_seq

    def validate(self) -> int:
        return lib().kvq_validate(ctypes.byref(self.c()))

    def codes_bytes(self) -> int:
        return lib().kvq_codes_bytes(ctypes.byref(self.c()))

    def norms_count(self) -> int:
        return lib().kvq_norms_count(ctypes.byref(self.c()))

    def scales_count(self) -> int:
        return lib().kvq_scales_count(ctypes.byref(self.c()))

    # outputs are head-major: [seqs, heads, tokens, ...] (see include/kvq.h)
    def codes_shape(self):
        return (self.seqs, self.heads, self.tokens_per_seq, self.head_dim // 2)

    def norms_shape(self):
        return (self.seqs, self.heads, self.tokens_per_seq)

    def scales_shape(self):
        if self.per_channel:
            return (self.seqs, self.heads, self.tokens_per_seq // self.block_tokens, self.head_dim)
        return (self.seqs, self.heads, self.tokens_per_seq)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != OK:
        raise KvqError(status, what)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the HIP device")


def alloc_outputs(d: Desc, device):
    codes = torch.empty(d.codes_shape(), dtype=torch.uint8, device=device)
    norms = torch.empty(d.norms_shape(), dtype=torch.float16, device=device) if d.nsep else None
    scales = torch.empty(d.scales_shape(), dtype=torch.float16, device=device)
    return codes, norms, scales


def quantize(d: Desc, x: torch.Tensor, signs: torch.Tensor | None = None,
             out=None, stream=None):
    """kvq_quantize.  Returns (codes uint8, norms fp16 or None, scales fp16)."""
    codes, norms, scales = out if out is not None else alloc_outputs(d, x.device)
    _need_cuda(x, signs, codes, norms, scales)
    st = lib().kvq_quantize(ctypes.byref(d.c()), _ptr(x), _ptr(signs), _ptr(codes), _ptr(norms),
                            _ptr(scales), _stream(stream))
    _check(st, "kvq_quantize")
    return codes, norms, scales


def dequantize(d: Desc, codes, norms, scales, signs=None, out_dtype=torch.float16,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_dequantize.  Returns y [rows, heads, head_dim] in out_dtype."""
    if out is None:
        out = torch.empty((d.rows, d.heads, d.head_dim), dtype=out_dtype, device=codes.device)
    _need_cuda(codes, norms, scales, signs, out)
    st = lib().kvq_dequantize(ctypes.byref(d.c()), _ptr(codes), _ptr(norms), _ptr(scales), _ptr(signs),
                              _ptr(out), DTYPES[out.dtype], _stream(stream))
    _check(st, "kvq_dequantize")
    return out


def score_decode(d: Desc, q: torch.Tensor, codes, norms, scales, signs=None,
                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_score_decode.  q fp16 [seqs, q_heads, head_dim] -> scores fp32 [seqs, q_heads, tokens]."""
    if q.dtype != torch.float16:
        raise ValueError("q must be fp16")
    q_heads = q.shape[1]
    if out is None:
        out = torch.empty((d.seqs, q_heads, d.tokens_per_seq), dtype=torch.float32, device=codes.device)
    _need_cuda(q, codes, norms, scales, signs, out)
    st = lib().kvq_score_decode(ctypes.byref(d.c()), _ptr(q), q_heads, _ptr(codes), _ptr(norms),
                                _ptr(scales), _ptr(signs), _ptr(out), _stream(stream))
    _check(st, "kvq_score_decode")
    return out


def attention_workspace_bytes(d: Desc, q_heads: int) -> int:
    return lib().kvq_attention_workspace_bytes(ctypes.byref(d.c()), q_heads)


def attention_decode(d: Desc, q: torch.Tensor, k_cache, v_cache, k_signs=None, v_signs=None,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """kvq_attention_decode.  k_cache / v_cache: (codes, norms, scales) as kvq_quantize returns
    them.  q fp16 [seqs, q_heads, head_dim] -> out fp32 [seqs, q_heads, head_dim].  The workspace
    (caller-owned device memory) is allocated here with torch when not supplied."""
    if q.dtype != torch.float16:
        raise ValueError("q must be fp16")
    q_heads = q.shape[1]
    kc, kn, ks = k_cache
    vc, vn, vs = v_cache
    if out is None:
        out = torch.empty((d.seqs, q_heads, d.head_dim), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = attention_workspace_bytes(d, q_heads)
        if nbytes < 0:
            _check(lib().kvq_validate(ctypes.byref(d.c())) or ERR_UNSUPPORTED, "kvq_attention_workspace_bytes")
        workspace = torch.empty(max(nbytes, 4) // 4, dtype=torch.float32, device=q.device)
    _need_cuda(q, kc, kn, ks, vc, vn, vs, k_signs, v_signs, out, workspace)
    st = lib().kvq_attention_decode(ctypes.byref(d.c()), _ptr(q), q_heads, _ptr(kc), _ptr(kn), _ptr(ks), _ptr(k_signs),
                                    _ptr(vc), _ptr(vn), _ptr(vs), _ptr(v_signs), _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "kvq_attention_decode")
    return out


def attention_decode_noalloc(d: Desc, q: torch.Tensor, k_cache, v_cache, k_signs=None, v_signs=None,
                             out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_attention_decode_noalloc: kvq_attention_decode with the partials in the library's static
    per-GPU scratch instead of a caller workspace (the C call allocates nothing; `out` is allocated
    here with torch when not supplied)."""
    if q.dtype != torch.float16:
        raise ValueError("q must be fp16")
    q_heads = q.shape[1]
    kc, kn, ks = k_cache
    vc, vn, vs = v_cache
    if out is None:
        out = torch.empty((d.seqs, q_heads, d.head_dim), dtype=torch.float32, device=q.device)
    _need_cuda(q, kc, kn, ks, vc, vn, vs, k_signs, v_signs, out)
    st = lib().kvq_attention_decode_noalloc(ctypes.byref(d.c()), _ptr(q), q_heads, _ptr(kc), _ptr(kn), _ptr(ks),
                                            _ptr(k_signs), _ptr(vc), _ptr(vn), _ptr(vs), _ptr(v_signs), _ptr(out),
                                            _stream(stream))
    _check(st, "kvq_attention_decode_noalloc")
    return out


def alloc_nsn(d: Desc, device):
    """Outputs of kvq_quantize_nsn: codes, s1, s2 (fp16 per token), offsets, scales (fp16 per block
    and channel), all head-major."""
    codes = torch.empty(d.codes_shape(), dtype=torch.uint8, device=device)
    s1 = torch.empty(d.norms_shape(), dtype=torch.float16, device=device)
    s2 = torch.empty(d.norms_shape(), dtype=torch.float16, device=device)
    offsets = torch.empty(d.scales_shape(), dtype=torch.float16, device=device)
    scales = torch.empty(d.scales_shape(), dtype=torch.float16, device=device)
    return codes, s1, s2, offsets, scales


def quantize_nsn(d: Desc, x: torch.Tensor, signs: torch.Tensor | None = None, out=None, stream=None):
    """kvq_quantize_nsn.  Returns (codes, s1, s2, offsets, scales)."""
    codes, s1, s2, offsets, scales = out if out is not None else alloc_nsn(d, x.device)
    _need_cuda(x, signs, codes, s1, s2, offsets, scales)
    st = lib().kvq_quantize_nsn(ctypes.byref(d.c()), _ptr(x), _ptr(signs), _ptr(codes), _ptr(s1), _ptr(s2),
                                _ptr(offsets), _ptr(scales), _stream(stream))
    _check(st, "kvq_quantize_nsn")
    return codes, s1, s2, offsets, scales


def dequantize_nsn(d: Desc, codes, s1, s2, offsets, scales, signs=None, out_dtype=torch.float16,
                   out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_dequantize_nsn: x^ = s1 (s2 R^T (c scale) + offset), [rows, heads, head_dim]."""
    if out is None:
        out = torch.empty((d.rows, d.heads, d.head_dim), dtype=out_dtype, device=codes.device)
    _need_cuda(codes, s1, s2, offsets, scales, signs, out)
    st = lib().kvq_dequantize_nsn(ctypes.byref(d.c()), _ptr(codes), _ptr(s1), _ptr(s2), _ptr(offsets), _ptr(scales),
                                  _ptr(signs), _ptr(out), DTYPES[out.dtype], _stream(stream))
    _check(st, "kvq_dequantize_nsn")
    return out


def score_decode_nsn(d: Desc, q: torch.Tensor, codes, s1, s2, offsets, scales, signs=None,
                     out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_score_decode_nsn: scores fp32 [seqs, q_heads, tokens] from an NSN cache."""
    if q.dtype != torch.float16:
        raise ValueError("q must be fp16")
    q_heads = q.shape[1]
    if out is None:
        out = torch.empty((d.seqs, q_heads, d.tokens_per_seq), dtype=torch.float32, device=codes.device)
    _need_cuda(q, codes, s1, s2, offsets, scales, signs, out)
    st = lib().kvq_score_decode_nsn(ctypes.byref(d.c()), _ptr(q), q_heads, _ptr(codes), _ptr(s1), _ptr(s2),
                                    _ptr(offsets), _ptr(scales), _ptr(signs), _ptr(out), _stream(stream))
    _check(st, "kvq_score_decode_nsn")
    return out


def alloc_residual(d: Desc, device):
    """The full-precision residual of a streamed cache: [seqs, block_tokens, heads, head_dim]."""
    return torch.empty((d.seqs, d.block_tokens, d.heads, d.head_dim), dtype=d.dtype, device=device)


def append(d: Desc, tokens_cached: int, x_new: torch.Tensor, residual: torch.Tensor, cache, signs=None,
           stream=None) -> int:
    """kvq_append: append x_new [seqs, n_new, heads, head_dim] to every sequence of the cache
    (codes, norms, scales with d.tokens_per_seq the capacity) and its residual.  Returns the new
    token count tokens_cached + n_new."""
    codes, norms, scales = cache
    _need_cuda(x_new, residual, signs, codes, norms, scales)
    n_new = x_new.shape[1] if x_new.dim() == 4 else 0
    st = lib().kvq_append(ctypes.byref(d.c()), tokens_cached, _ptr(x_new), n_new, _ptr(residual), _ptr(signs),
                          _ptr(codes), _ptr(norms), _ptr(scales), _stream(stream))
    _check(st, "kvq_append")
    return tokens_cached + n_new


def append_kv(d: Desc, tokens_cached: int, k_new: torch.Tensor, v_new: torch.Tensor, k_residual: torch.Tensor,
              v_residual: torch.Tensor, k_cache, v_cache, k_signs=None, v_signs=None, stream=None) -> int:
    """kvq_append_kv: append k_new and v_new [seqs, n_new, heads, head_dim] to the K and V caches
    and their residuals in one call (the same results as append on each).  Returns tokens_cached +
    n_new."""
    kc, kn, ks = k_cache
    vc, vn, vs = v_cache
    _need_cuda(k_new, v_new, k_residual, v_residual, k_signs, v_signs, kc, kn, ks, vc, vn, vs)
    n_new = k_new.shape[1] if k_new.dim() == 4 else 0
    if tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError(f"k_new {tuple(k_new.shape)} and v_new {tuple(v_new.shape)} differ")
    st = lib().kvq_append_kv(ctypes.byref(d.c()), tokens_cached, n_new, _ptr(k_new), _ptr(k_residual), _ptr(k_signs),
                             _ptr(kc), _ptr(kn), _ptr(ks), _ptr(v_new), _ptr(v_residual), _ptr(v_signs), _ptr(vc),
                             _ptr(vn), _ptr(vs), _stream(stream))
    _check(st, "kvq_append_kv")
    return tokens_cached + n_new


def attention_decode_stream(d: Desc, tokens_cached: int, q: torch.Tensor, k_cache, k_residual, v_cache, v_residual,
                            k_signs=None, v_signs=None, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_attention_decode_stream: attention over the first tokens_cached tokens of a streamed
    cache (whole blocks packed, the rest in the residuals).  Same conventions as attention_decode."""
    if q.dtype != torch.float16:
        raise ValueError("q must be fp16")
    q_heads = q.shape[1]
    kc, kn, ks = k_cache
    vc, vn, vs = v_cache
    if out is None:
        out = torch.empty((d.seqs, q_heads, d.head_dim), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = attention_workspace_bytes(d, q_heads)
        if nbytes < 0:
            _check(lib().kvq_validate(ctypes.byref(d.c())) or ERR_UNSUPPORTED, "kvq_attention_workspace_bytes")
        workspace = torch.empty(max(nbytes, 4) // 4, dtype=torch.float32, device=q.device)
    _need_cuda(q, kc, kn, ks, vc, vn, vs, k_signs, v_signs, k_residual, v_residual, out, workspace)
    st = lib().kvq_attention_decode_stream(ctypes.byref(d.c()), tokens_cached, _ptr(q), q_heads, _ptr(kc), _ptr(kn),
                                           _ptr(ks), _ptr(k_signs), _ptr(k_residual), _ptr(vc), _ptr(vn), _ptr(vs),
                                           _ptr(v_signs), _ptr(v_residual), _ptr(out), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "kvq_attention_decode_stream")
    return out


# ----------------------------------------------------------------------------- RRS INT4 GEMM path
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x and w must be float16 or bfloat16")
    return DTYPES[t.dtype]


def rrs_smooth_scales(x: torch.Tensor, signs: torch.Tensor | None, hadamard: int, out=None, stream=None):
    """kvq_rrs_smooth_scales: fp32 [k/128], the group maxima of |x R| over all rows of x [n, k]."""
    n, k = x.shape
    s = out if out is not None else torch.empty(k // 128, dtype=torch.float32, device=x.device)
    _need_cuda(x, signs, s)
    _check(lib().kvq_rrs_smooth_scales(_ptr(x), n, k, _dtype_code(x), _ptr(signs), hadamard, _ptr(s), _stream(stream)),
           "kvq_rrs_smooth_scales")
    return s


def rrs_quantize_act(x: torch.Tensor, signs: torch.Tensor | None, hadamard: int, scales: torch.Tensor, bits: int = 4,
                     out=None, stream=None):
    """kvq_rrs_quantize_act: (codes uint8 [n, k/2], act_scales fp16 [n])."""
    n, k = x.shape
    codes, a = out if out is not None else (torch.empty((n, k // 2), dtype=torch.uint8, device=x.device),
                                            torch.empty(n, dtype=torch.float16, device=x.device))
    _need_cuda(x, signs, scales, codes, a)
    _check(lib().kvq_rrs_quantize_act(_ptr(x), n, k, _dtype_code(x), _ptr(signs), hadamard, _ptr(scales), bits,
                                      _ptr(codes), _ptr(a), _stream(stream)), "kvq_rrs_quantize_act")
    return codes, a


def rrs_quantize_weights(w: torch.Tensor, signs: torch.Tensor | None, hadamard: int, bits: int = 4, out=None,
                         stream=None):
    """kvq_rrs_quantize_weights: (codes uint8 [m, k/2], w_scales fp16 [m])."""
    m, k = w.shape
    codes, b = out if out is not None else (torch.empty((m, k // 2), dtype=torch.uint8, device=w.device),
                                            torch.empty(m, dtype=torch.float16, device=w.device))
    _need_cuda(w, signs, codes, b)
    _check(lib().kvq_rrs_quantize_weights(_ptr(w), m, k, _dtype_code(w), _ptr(signs), hadamard, bits, _ptr(codes),
                                          _ptr(b), _stream(stream)), "kvq_rrs_quantize_weights")
    return codes, b


def rrs_gemm(x_codes, act_scales, w_codes, w_scales, scales, out=None, stream=None) -> torch.Tensor:
    """kvq_rrs_gemm: y fp32 [n, m] = a_t b_m sum_g s_g (integer product of group g)."""
    n, m, k = x_codes.shape[0], w_codes.shape[0], 2 * x_codes.shape[1]
    y = out if out is not None else torch.empty((n, m), dtype=torch.float32, device=x_codes.device)
    _need_cuda(x_codes, act_scales, w_codes, w_scales, scales, y)
    _check(lib().kvq_rrs_gemm(_ptr(x_codes), _ptr(act_scales), n, _ptr(w_codes), _ptr(w_scales), m, k, _ptr(scales),
                              _ptr(y), _stream(stream)), "kvq_rrs_gemm")
    return y


def token_major(d: Desc, codes=None, norms=None, scales=None):
    """Views of kvq_quantize's head-major outputs in x's token-major order (new contiguous
    tensors): codes [rows, heads, head_dim/2], norms [rows, heads], scales [rows, heads] or
    [rows/B, heads, head_dim].  Pure data movement; None passes through."""
    S, H, T, D, D2 = d.seqs, d.heads, d.tokens_per_seq, d.head_dim, d.head_dim // 2
    c = None if codes is None else codes.reshape(S, H, T, D2).transpose(1, 2).reshape(S * T, H, D2).contiguous()
    n = None if norms is None else norms.reshape(S, H, T).transpose(1, 2).reshape(S * T, H).contiguous()
    sc = None
    if scales is not None:
        if d.per_channel:
            nb = T // d.block_tokens
            sc = scales.reshape(S, H, nb, D).transpose(1, 2).reshape(S * nb, H, D).contiguous()
        else:
            sc = scales.reshape(S, H, T).transpose(1, 2).reshape(S * T, H).contiguous()
    return c, n, sc


def head_major(d: Desc, codes=None, norms=None, scales=None):
    """Inverse of token_major: token-major codes / norms / scales -> the head-major layout the
    kernels read (new contiguous tensors)."""
    S, H, T, D, D2 = d.seqs, d.heads, d.tokens_per_seq, d.head_dim, d.head_dim // 2
    c = None if codes is None else codes.reshape(S, T, H, D2).transpose(1, 2).contiguous()
    n = None if norms is None else norms.reshape(S, T, H).transpose(1, 2).contiguous()
    sc = None
    if scales is not None:
        if d.per_channel:
            nb = T // d.block_tokens
            sc = scales.reshape(S, nb, H, D).transpose(1, 2).contiguous()
        else:
            sc = scales.reshape(S, T, H).transpose(1, 2).contiguous()
    return c, n, sc
