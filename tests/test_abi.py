"""CPU-side checks of the C ABI: the library loads, exports every declared symbol, lays out
kvq_desc as the header says, and refuses bad arguments before touching any device."""
import ctypes
import os
import re

import pytest

from activation_quantization_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = kvq.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"libkvq.so does not export {n}"
    assert set(names) == set(kvq._SIGNATURES), "binding and header disagree"


def test_desc_layout_matches_header():
    assert "56 bytes" in open(HEADER).read()
    assert ctypes.sizeof(kvq.KvqDesc) == 56
    offs = [getattr(kvq.KvqDesc, f[0]).offset for f in kvq.KvqDesc._fields_]
    assert offs == [0, 8, 16, 24, 32, 36, 40, 44, 48, 52]


def test_version_and_status_strings():
    L = kvq.lib()
    assert L.kvq_version() >= 10000
    for s in range(6):
        assert L.kvq_status_str(s).startswith(b"KVQ_")


GOOD = dict(seqs=2, tokens_per_seq=256, heads=4, head_dim=128, bits=4, mode="nsep_pchan",
            block_tokens=128, hadamard=128)


@pytest.mark.parametrize("change,want", [
    ({}, kvq.OK),
    ({"tokens_per_seq": 250}, kvq.ERR_SHAPE),             # block does not divide the sequence
    ({"head_dim": 127, "mode": "naive"}, kvq.ERR_SHAPE),  # odd
    ({"heads": 0}, kvq.ERR_SHAPE),
    ({"seqs": -1}, kvq.ERR_SHAPE),
    ({"hadamard": 48}, kvq.ERR_SHAPE),                    # not a power of two
    ({"hadamard": 256, "mode": "naive", "head_dim": 512}, kvq.ERR_UNSUPPORTED),
    ({"hadamard": 8}, kvq.ERR_UNSUPPORTED),
    ({"bits": 5}, kvq.ERR_UNSUPPORTED),
    ({"bits": 1}, kvq.ERR_UNSUPPORTED),
    ({"head_dim": 256}, kvq.ERR_UNSUPPORTED),             # per-channel needs 64 / 128
    ({"head_dim": 96, "mode": "naive", "hadamard": 0}, kvq.ERR_UNSUPPORTED),
    ({"block_tokens": 32, "tokens_per_seq": 256}, kvq.ERR_UNSUPPORTED),
    ({"block_tokens": 256}, kvq.ERR_UNSUPPORTED),         # 256 only with head_dim 64
    ({"head_dim": 64, "block_tokens": 256, "hadamard": 64}, kvq.OK),
    ({"head_dim": 4096, "mode": "naive", "block_tokens": 0}, kvq.OK),
    ({"head_dim": 16384, "mode": "naive", "block_tokens": 0}, kvq.ERR_UNSUPPORTED),
    ({"seqs": 0}, kvq.OK),                                # empty input is valid
])
def test_validation_matrix(change, want):
    p = dict(GOOD)
    p.update(change)
    d = kvq.Desc(**p)
    got = d.validate()
    assert got == want, kvq.lib().kvq_last_error()
    if want != kvq.OK:
        assert kvq.lib().kvq_last_error()


def test_size_queries():
    d = kvq.Desc(**GOOD)
    assert d.codes_bytes() == 2 * 256 * 4 * 64
    assert d.norms_count() == 2 * 256 * 4
    assert d.scales_count() == 2 * 2 * 4 * 128
    n = kvq.Desc(1, 8192, 1, 4096, 4, "naive", 0, 128, kvq.torch.bfloat16)
    assert n.codes_bytes() == 8192 * 2048 and n.norms_count() == 0 and n.scales_count() == 8192
    assert kvq.Desc(**{**GOOD, "bits": 7}).codes_bytes() == -1


FAKE = 1 << 20   # an aligned address that is never dereferenced: validation fails first


def _q(d, x=FAKE, signs=FAKE, codes=FAKE, norms=FAKE, scales=FAKE):
    return kvq.lib().kvq_quantize(ctypes.byref(d.c()), x, signs, codes, norms, scales, None)


def test_pointer_checks_before_any_device_call():
    d = kvq.Desc(**GOOD)
    assert _q(d, x=None) == kvq.ERR_NULL
    assert _q(d, norms=None) == kvq.ERR_NULL
    assert _q(d, signs=None) == kvq.ERR_NULL
    assert _q(kvq.Desc(**{**GOOD, "mode": "pchan"})) == kvq.ERR_NULL      # norms must be NULL
    assert _q(kvq.Desc(**{**GOOD, "hadamard": 0})) == kvq.ERR_NULL        # signs must be NULL
    assert _q(d, x=FAKE + 2) == kvq.ERR_ALIGN
    assert _q(d, codes=FAKE + 8) == kvq.ERR_ALIGN
    assert _q(d, scales=FAKE + 1) == kvq.ERR_ALIGN
    L = kvq.lib()
    assert L.kvq_dequantize(ctypes.byref(d.c()), FAKE, FAKE, FAKE, FAKE, FAKE, 7, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_score_decode(ctypes.byref(d.c()), FAKE, 6, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_SHAPE
    assert L.kvq_score_decode(ctypes.byref(d.c()), FAKE, 4 * 17, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present")
def test_no_device_maps_to_err_hip():
    d = kvq.Desc(**GOOD)
    assert _q(d) == kvq.ERR_HIP
    assert b"no HIP device" in kvq.lib().kvq_last_error()


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(kvq, "_lib", None)
    monkeypatch.setattr(kvq, "LIB_PATH", "/nonexistent/libkvq.so")
    with pytest.raises(ImportError):
        kvq.lib()


def _att(d, q_heads=16, ws_bytes=1 << 30, **ptr):
    p = dict(q=FAKE, kc=FAKE, kn=FAKE, ks=FAKE, ksg=FAKE, vc=FAKE, vn=FAKE, vs=FAKE, vsg=FAKE, out=FAKE, ws=FAKE)
    p.update(ptr)
    return kvq.lib().kvq_attention_decode(ctypes.byref(d.c()), p["q"], q_heads, p["kc"], p["kn"], p["ks"], p["ksg"],
                                          p["vc"], p["vn"], p["vs"], p["vsg"], p["out"], p["ws"], ws_bytes, None)


def test_attention_workspace_size():
    d = kvq.Desc(**GOOD)                                   # 2 seqs x 256 tokens: 2 blocks -> 1 chunk -> 1 partial
    assert kvq.attention_workspace_bytes(d, 16) == 2 * 16 * 1 * (128 + 2) * 4
    long = kvq.Desc(64, 32768, 8, 128, 4, "nsep_pchan", 128, 128)
    assert kvq.attention_workspace_bytes(long, 32) == 64 * 32 * (256 // 16) * 130 * 4
    assert kvq.attention_workspace_bytes(kvq.Desc(**{**GOOD, "mode": "nsep"}), 16) == -1
    assert kvq.attention_workspace_bytes(d, 20) == -1     # 5 query heads per KV head


def test_attention_validation_before_any_device_call():
    d = kvq.Desc(**GOOD)
    assert _att(kvq.Desc(**{**GOOD, "mode": "nsep", "block_tokens": 0})) == kvq.ERR_UNSUPPORTED   # per-token scales
    assert _att(kvq.Desc(**{**GOOD, "head_dim": 64, "hadamard": 64})) == kvq.ERR_UNSUPPORTED
    assert _att(d, q_heads=20) == kvq.ERR_UNSUPPORTED     # G = 5
    assert _att(d, q_heads=6) == kvq.ERR_SHAPE            # not a multiple of heads
    assert _att(kvq.Desc(**{**GOOD, "tokens_per_seq": 0})) == kvq.ERR_SHAPE
    assert _att(kvq.Desc(**{**GOOD, "seqs": 0})) == kvq.OK   # nothing to do
    assert _att(d, ws=None) == kvq.ERR_NULL
    assert _att(d, vn=None) == kvq.ERR_NULL               # NSEP needs both norms
    assert _att(d, ksg=None) == kvq.ERR_NULL              # Hadamard needs both signs
    assert _att(d, vs=FAKE + 2) == kvq.ERR_ALIGN          # scales are read as 16-byte vectors
    assert _att(d, out=FAKE + 2) == kvq.ERR_ALIGN
    assert _att(d, ws_bytes=100) == kvq.ERR_SHAPE


def _app(d, tokens_cached=0, n_new=8, **ptr):
    p = dict(x=FAKE, res=FAKE, sg=FAKE, c=FAKE, n=FAKE, s=FAKE)
    p.update(ptr)
    return kvq.lib().kvq_append(ctypes.byref(d.c()), tokens_cached, p["x"], n_new, p["res"], p["sg"], p["c"], p["n"],
                                p["s"], None)


def test_append_validation_before_any_device_call():
    d = kvq.Desc(**GOOD)                                  # capacity 256 tokens, B = 128, NSEP + Hadamard
    assert _app(kvq.Desc(**{**GOOD, "mode": "nsep", "block_tokens": 0})) == kvq.ERR_UNSUPPORTED   # per-token codes
    assert _app(d, tokens_cached=250, n_new=7) == kvq.ERR_SHAPE          # past the capacity
    assert _app(d, tokens_cached=-1) == kvq.ERR_SHAPE
    assert _app(d, n_new=-1) == kvq.ERR_SHAPE
    assert _app(d, tokens_cached=250, n_new=6, res=None) == kvq.ERR_NULL  # exactly full passes the size check
    assert _app(d, n_new=0) == kvq.OK                                    # nothing to append
    assert _app(d, res=None) == kvq.ERR_NULL
    assert _app(d, n=None) == kvq.ERR_NULL                               # NSEP needs norms
    assert _app(d, sg=None) == kvq.ERR_NULL                              # Hadamard needs signs
    assert _app(d, res=FAKE + 8) == kvq.ERR_ALIGN
    assert _app(d, x=FAKE + 2) == kvq.ERR_ALIGN


def _appkv(d, tokens_cached=0, n_new=8, **ptr):
    p = dict(kx=FAKE, kr=FAKE, ksg=FAKE, kc=FAKE, kn=FAKE, ks=FAKE, vx=FAKE, vr=FAKE, vsg=FAKE, vc=FAKE, vn=FAKE, vs=FAKE)
    p.update(ptr)
    return kvq.lib().kvq_append_kv(ctypes.byref(d.c()), tokens_cached, n_new, p["kx"], p["kr"], p["ksg"], p["kc"],
                                   p["kn"], p["ks"], p["vx"], p["vr"], p["vsg"], p["vc"], p["vn"], p["vs"], None)


def test_append_kv_validation_before_any_device_call():
    # every case fails (or returns OK for an empty append) before any device is touched
    d = kvq.Desc(**GOOD)
    assert _appkv(kvq.Desc(**{**GOOD, "mode": "nsep", "block_tokens": 0})) == kvq.ERR_UNSUPPORTED
    assert _appkv(d, tokens_cached=250, n_new=7) == kvq.ERR_SHAPE
    assert _appkv(d, n_new=0) == kvq.OK
    for side, name in (("k", b"K side"), ("v", b"V side")):
        for change, want in ((dict(r=None), kvq.ERR_NULL), (dict(c=None), kvq.ERR_NULL), (dict(n=None), kvq.ERR_NULL),
                             (dict(sg=None), kvq.ERR_NULL), (dict(x=FAKE + 2), kvq.ERR_ALIGN),
                             (dict(s=FAKE + 1), kvq.ERR_ALIGN)):
            assert _appkv(d, **{side + k: v for k, v in change.items()}) == want
            assert kvq.lib().kvq_last_error().startswith(name)


def _atts(d, tokens_cached, q_heads=16, ws_bytes=1 << 30, **ptr):
    p = dict(q=FAKE, kc=FAKE, kn=FAKE, ks=FAKE, ksg=FAKE, kr=FAKE, vc=FAKE, vn=FAKE, vs=FAKE, vsg=FAKE, vr=FAKE,
             out=FAKE, ws=FAKE)
    p.update(ptr)
    return kvq.lib().kvq_attention_decode_stream(ctypes.byref(d.c()), tokens_cached, p["q"], q_heads, p["kc"], p["kn"],
                                                 p["ks"], p["ksg"], p["kr"], p["vc"], p["vn"], p["vs"], p["vsg"],
                                                 p["vr"], p["out"], p["ws"], ws_bytes, None)


def test_stream_attention_validation_before_any_device_call():
    d = kvq.Desc(**GOOD)
    assert _atts(d, 0) == kvq.ERR_SHAPE                                  # nothing cached
    assert _atts(d, 257) == kvq.ERR_SHAPE                                # past the capacity
    assert _atts(d, 130, kr=None) == kvq.ERR_NULL                        # 2 tokens wait in the residual
    assert _atts(d, 130, vr=FAKE + 1) == kvq.ERR_ALIGN
    # whole blocks only: no residual needed (validation goes on to the workspace size)
    assert _atts(d, 128, kr=None, vr=None, ws_bytes=100) == kvq.ERR_SHAPE
    assert _atts(d, 130, kr=None, ws_bytes=100) == kvq.ERR_NULL
    assert _atts(kvq.Desc(**{**GOOD, "mode": "naive", "block_tokens": 0}), 10) == kvq.ERR_UNSUPPORTED


NSN = dict(GOOD, mode="nsn_pchan")


def test_nsn_sizes_and_mode_checks():
    d = kvq.Desc(**NSN)
    assert d.validate() == kvq.OK
    rows = d.seqs * d.tokens_per_seq
    assert d.norms_count() == rows * d.heads                             # each of s1 and s2
    assert d.scales_count() == rows // d.block_tokens * d.heads * d.head_dim   # also the offsets
    L = kvq.lib()
    c = ctypes.byref(d.c())
    # the plain calls refuse the NSN mode, the _nsn calls refuse the others
    assert L.kvq_quantize(c, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_dequantize(c, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_score_decode(c, FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    g = ctypes.byref(kvq.Desc(**GOOD).c())
    assert L.kvq_quantize_nsn(g, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_dequantize_nsn(g, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_score_decode_nsn(g, FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    # missing byproducts, signs, alignment
    assert L.kvq_quantize_nsn(c, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == kvq.ERR_NULL
    assert L.kvq_quantize_nsn(c, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_NULL   # Hadamard on
    assert L.kvq_quantize_nsn(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, None) == kvq.ERR_ALIGN
    assert L.kvq_dequantize_nsn(c, FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE, FAKE, 0, None) == kvq.ERR_ALIGN
    assert L.kvq_dequantize_nsn(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 7, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_score_decode_nsn(c, FAKE, 6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_SHAPE
    assert L.kvq_score_decode_nsn(c, FAKE, 16, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == kvq.ERR_NULL
    # attention and the streaming append do not take the NSN mode
    assert _att(d) == kvq.ERR_UNSUPPORTED
    assert _app(d) == kvq.ERR_UNSUPPORTED


def test_rrs_validation_before_any_device_call():
    L = kvq.lib()
    F16, BF16 = 0, 1
    # shapes: k a power of two in [128, 8192] for the quantizers, a multiple of 128 for the GEMM
    assert L.kvq_rrs_smooth_scales(FAKE, 16, 384, F16, FAKE, 128, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_rrs_smooth_scales(FAKE, 16, 64, F16, FAKE, 64, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_rrs_smooth_scales(FAKE, -1, 256, F16, FAKE, 128, FAKE, None) == kvq.ERR_SHAPE
    assert L.kvq_rrs_quantize_act(FAKE, 16, 16384, BF16, FAKE, 128, FAKE, 4, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_rrs_quantize_weights(FAKE, 8, 200, F16, FAKE, 128, 4, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_rrs_gemm(FAKE, FAKE, 16, FAKE, FAKE, 8, 200, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_rrs_gemm(FAKE, FAKE, -1, FAKE, FAKE, 8, 256, FAKE, FAKE, None) == kvq.ERR_SHAPE
    # bits, dtype, Hadamard size
    assert L.kvq_rrs_quantize_act(FAKE, 16, 256, F16, FAKE, 128, FAKE, 5, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_rrs_quantize_weights(FAKE, 8, 256, 2, FAKE, 128, 4, FAKE, FAKE, None) == kvq.ERR_UNSUPPORTED
    assert L.kvq_rrs_smooth_scales(FAKE, 16, 256, F16, FAKE, 256, FAKE, None) == kvq.ERR_UNSUPPORTED
    # pointers: required buffers, signs iff Hadamard
    assert L.kvq_rrs_smooth_scales(FAKE, 16, 256, F16, FAKE, 128, None, None) == kvq.ERR_NULL
    assert L.kvq_rrs_smooth_scales(None, 16, 256, F16, FAKE, 128, FAKE, None) == kvq.ERR_NULL
    assert L.kvq_rrs_smooth_scales(FAKE, 16, 256, F16, None, 128, FAKE, None) == kvq.ERR_NULL
    assert L.kvq_rrs_quantize_act(FAKE, 16, 256, F16, FAKE, 0, FAKE, 4, FAKE, FAKE, None) == kvq.ERR_NULL
    assert L.kvq_rrs_quantize_act(FAKE, 16, 256, F16, FAKE, 128, None, 4, FAKE, FAKE, None) == kvq.ERR_NULL
    assert L.kvq_rrs_quantize_weights(FAKE, 8, 256, F16, FAKE, 128, 4, FAKE, None, None) == kvq.ERR_NULL
    assert L.kvq_rrs_gemm(FAKE, FAKE, 16, None, FAKE, 8, 256, FAKE, FAKE, None) == kvq.ERR_NULL
    # alignment
    assert L.kvq_rrs_smooth_scales(FAKE + 8, 16, 256, F16, FAKE, 128, FAKE, None) == kvq.ERR_ALIGN
    assert L.kvq_rrs_smooth_scales(FAKE, 16, 256, F16, FAKE, 128, FAKE + 2, None) == kvq.ERR_ALIGN
    assert L.kvq_rrs_quantize_act(FAKE, 16, 256, F16, FAKE, 128, FAKE, 4, FAKE + 4, FAKE, None) == kvq.ERR_ALIGN
    assert L.kvq_rrs_quantize_weights(FAKE, 8, 256, F16, FAKE, 128, 4, FAKE, FAKE + 1, None) == kvq.ERR_ALIGN
    assert L.kvq_rrs_gemm(FAKE, FAKE, 16, FAKE + 8, FAKE, 8, 256, FAKE, FAKE, None) == kvq.ERR_ALIGN
    assert L.kvq_rrs_gemm(FAKE, FAKE, 16, FAKE, FAKE, 8, 256, FAKE, FAKE + 2, None) == kvq.ERR_ALIGN
    # empty work enqueues nothing (the quantizers and the GEMM return before any pointer is used)
    assert L.kvq_rrs_quantize_act(None, 0, 256, F16, None, 0, None, 4, None, None, None) == kvq.OK
    assert L.kvq_rrs_gemm(None, None, 0, None, None, 8, 256, None, None, None) == kvq.OK
