"""GPU parity of the streaming append (kvq_append) and of attention over a streamed cache
(kvq_attention_decode_stream).

The append must leave exactly the state the oracle defines (oracle.stream_state): whole blocks
quantized bit for bit as kvq_quantize quantizes them, the trailing tokens in the residual
unchanged, whatever the sizes of the appends.  Attention over the streamed cache is compared with
the oracle's softmax over the GPU's own dequantized blocks followed by the residual tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from activation_quantization_amd import kvq
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _history(seed, S, n, H, D, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((S, n, H, D)).astype(np.float32)
    x[..., 5] *= 30.0                                               # an outlier channel
    x *= rng.uniform(0.3, 3.0, size=(S, n, 1, 1)).astype(np.float32)
    signs = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, D)))
    return torch.from_numpy(x).to(dtype), signs


def _append_all(d, x_hist, chunks, signs):
    """Append x_hist [S, n, H, D] chunk by chunk to a fresh cache of capacity d.tokens_per_seq;
    the buffers start poisoned so that anything left unwritten shows."""
    cache = kvq.alloc_outputs(d, DEV)
    for t in cache:
        if t is not None:
            t.view(torch.uint8).fill_(0xAB)
    res = kvq.alloc_residual(d, DEV)
    res.view(torch.uint8).fill_(0xAB)
    xd = x_hist.to(DEV)
    n = 0
    for c in chunks:
        n = kvq.append(d, n, xd[:, n:n + c].contiguous(), res, cache, signs)
    torch.cuda.synchronize()
    assert n == x_hist.shape[1]
    return cache, res


def _cached_part(d, cache, whole):
    """The first `whole` tokens of every stream of a capacity-d cache, with their descriptor."""
    S, H, C, D = d.seqs, d.heads, d.tokens_per_seq, d.head_dim
    dq = kvq.Desc(S, whole, H, D, d.bits, d.mode, d.block_tokens, d.hadamard, d.dtype)
    codes, norms, scales = cache
    c = codes.view(S, H, C, D // 2)[:, :, :whole].contiguous()
    n = None if norms is None else norms.view(S, H, C)[:, :, :whole].contiguous()
    s = scales.view(S, H, C // d.block_tokens, D)[:, :, :whole // d.block_tokens].contiguous()
    return dq, (c, n, s)


CASES = [
    # S, H, D, B, mode, had, dtype, chunks
    (2, 2, 128, 64, "nsep_pchan", 128, torch.float16, [1] * 70 + [67, 5, 129, 7]),
    (3, 1, 64, 128, "pchan", 0, torch.bfloat16, [200, 1, 55, 130]),
    (1, 4, 128, 128, "nsep_pchan", 64, torch.float16, [127, 1, 1, 256, 3]),
    (2, 3, 64, 64, "nsep_pchan", 16, torch.bfloat16, [64, 64, 1, 63, 64]),
]


@pytest.mark.parametrize("S,H,D,B,mode,had,dtype,chunks", CASES)
def test_append_matches_quantize_and_oracle(S, H, D, B, mode, had, dtype, chunks):
    n = sum(chunks)
    cap = (n // B + 1) * B
    x_hist, signs = _history(n + D, S, n, H, D, dtype)
    sg = signs.to(DEV) if had else None
    d = kvq.Desc(S, cap, H, D, 4, mode, B, had, dtype)
    cache, res = _append_all(d, x_hist, chunks, sg)
    whole = n // B * B
    r = n - whole

    # the residual is the exact tail, in its first r slots
    assert torch.equal(res[:, :r].cpu().view(torch.int16), x_hist[:, whole:].contiguous().view(torch.int16))

    # the blocks are bit for bit what kvq_quantize writes for the same tokens
    dq, part = _cached_part(d, cache, whole)
    ref = kvq.quantize(dq, x_hist[:, :whole].reshape(S * whole, H, D).to(DEV), sg)
    torch.cuda.synchronize()
    for got, want in zip(part, ref):
        if want is not None:
            assert torch.equal(got.cpu(), want.cpu())

    # and they match the oracle's streamed state
    sp = oracle.Spec(S, 0, H, D, 4, mode, B, had)
    st = oracle.stream_state(x_hist.double().numpy(), sp, signs.numpy() if had else None)
    c, nn, sc = (None if t is None else t.cpu().numpy() for t in kvq.token_major(dq, *part))
    parity.check_codes(c, st.quantized, 4)
    if dq.nsep:
        parity.check_rel_f16(nn, st.quantized.nu, "norms")
    parity.check_rel_f16(sc, st.quantized.scale, "scales")
    np.testing.assert_array_equal(res[:, :r].cpu().double().numpy(), st.residual)


def test_append_leaves_later_blocks_untouched():
    # only the blocks that filled are written: the rest of the capacity keeps its contents (the
    # residual's slots past the tail are scratch: a top-up that fills it writes all of them)
    S, H, D, B = 2, 2, 128, 64
    x_hist, signs = _history(7, S, 2 * B + 9, H, D, torch.float16)
    d = kvq.Desc(S, 4 * B, H, D, 4, "nsep_pchan", B, 128, torch.float16)
    cache, res = _append_all(d, x_hist, [B + 3, B + 6], signs.to(DEV))
    codes, norms, scales = (t.cpu() for t in cache)
    assert bool((codes.view(S, H, 4 * B, D // 2)[:, :, 2 * B:] == 0xAB).all())
    assert bool((norms.view(S, H, 4 * B)[:, :, 2 * B:].view(torch.uint8) == 0xAB).all())
    assert bool((scales.view(S, H, 4, D)[:, :, 2:].view(torch.uint8) == 0xAB).all())
    assert not bool((codes.view(S, H, 4 * B, D // 2)[:, :, :2 * B] == 0xAB).all())


def _oracle_stream_attention(d, n, q, k_cache, k_res, v_cache, v_res, sk, sv):
    whole = n // d.block_tokens * d.block_tokens
    S, H, D = d.seqs, d.heads, d.head_dim
    k_hat = v_hat = None
    if whole:
        dq, kp = _cached_part(d, k_cache, whole)
        _, vp = _cached_part(d, v_cache, whole)
        sp = oracle.Spec(S, whole, H, D, d.bits, d.mode, d.block_tokens, d.hadamard)
        kt = [None if t is None else t.cpu().numpy() for t in kvq.token_major(dq, *kp)]
        vt = [None if t is None else t.cpu().numpy() for t in kvq.token_major(dq, *vp)]
        k_hat = oracle.dequantize(*kt, sp, None if sk is None else sk.cpu().numpy())
        v_hat = oracle.dequantize(*vt, sp, None if sv is None else sv.cpu().numpy())
    r = n - whole
    spec = oracle.Spec(S, 0, H, D, d.bits, d.mode, d.block_tokens, d.hadamard)
    return oracle.attention_decode_stream(q.double().numpy(), k_hat, v_hat, k_res[:, :r].cpu().double().numpy(),
                                          v_res[:, :r].cpu().double().numpy(), spec)


@pytest.mark.parametrize("S,H,G,B,had,mode,dtype,n", [
    (2, 2, 4, 64, 128, "nsep_pchan", torch.float16, 3 * 64 + 17),   # blocks and a residual
    (2, 2, 4, 64, 128, "nsep_pchan", torch.float16, 3 * 64),        # whole blocks only
    (3, 1, 2, 128, 0, "pchan", torch.bfloat16, 90),                 # residual only
    (1, 4, 1, 128, 32, "nsep_pchan", torch.float16, 2 * 128 + 127), # the largest residual
    (2, 2, 3, 128, 64, "pchan", torch.bfloat16, 5 * 128 + 1),
])
def test_stream_attention(S, H, G, B, had, mode, dtype, n):
    D = 128
    cap = (n // B + 2) * B
    xk, sk = _history(n, S, n, H, D, dtype)
    xv, sv = _history(n + 1, S, n, H, D, dtype)
    sk = sk.to(DEV) if had else None
    sv = sv.to(DEV) if had else None
    d = kvq.Desc(S, cap, H, D, 4, mode, B, had, dtype)
    chunks = [n // 3, 1, n - n // 3 - 1]
    kc, kr = _append_all(d, xk, chunks, sk)
    vc, vr = _append_all(d, xv, chunks, sv)
    q = torch.from_numpy(np.random.default_rng(n + 2).standard_normal((S, G * H, D)).astype(np.float32) * 0.3).half()
    out = kvq.attention_decode_stream(d, n, q.to(DEV), kc, kr, vc, vr, sk, sv)
    torch.cuda.synchronize()
    ref = _oracle_stream_attention(d, n, q, kc, kr, vc, vr, sk, sv)
    print("worst error / tolerance", parity.check_attention(out.cpu().numpy(), ref))


def test_stream_attention_equals_cache_attention_on_whole_blocks():
    # with no residual the streamed call over a larger capacity equals kvq_attention_decode over
    # a cache of exactly the cached tokens (the same kernels, the same sums)
    S, H, G, B, D, n = 2, 2, 4, 128, 128, 3 * 128
    xk, sk = _history(11, S, n, H, D, torch.float16)
    xv, sv = _history(12, S, n, H, D, torch.float16)
    sk, sv = sk.to(DEV), sv.to(DEV)
    d = kvq.Desc(S, 5 * B, H, D, 4, "nsep_pchan", B, 128, torch.float16)
    kc, kr = _append_all(d, xk, [n], sk)
    vc, vr = _append_all(d, xv, [n], sv)
    q = torch.from_numpy(np.random.default_rng(13).standard_normal((S, G * H, D)).astype(np.float32)).half().to(DEV)
    got = kvq.attention_decode_stream(d, n, q, kc, None, vc, None, sk, sv)
    dn = kvq.Desc(S, n, H, D, 4, "nsep_pchan", B, 128, torch.float16)
    want = kvq.attention_decode(dn, q, kvq.quantize(dn, xk.reshape(S * n, H, D).to(DEV), sk),
                                kvq.quantize(dn, xv.reshape(S * n, H, D).to(DEV), sv), sk, sv)
    torch.cuda.synchronize()
    np.testing.assert_allclose(got.cpu().numpy(), want.cpu().numpy(), rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("S,H,D,B,mode,had,dtype,chunks", CASES)
def test_append_kv_equals_two_appends(S, H, D, B, mode, had, dtype, chunks):
    # kvq_append_kv must leave both caches and residuals byte for byte as kvq_append on K and then V
    n_tot = sum(chunks)
    C = ((n_tot + B - 1) // B + 1) * B
    d = kvq.Desc(S, C, H, D, 4, mode, B, had, dtype)
    xk, sk = _history(S + n_tot, S, n_tot, H, D, dtype)
    xv, sv = _history(S + n_tot + 1, S, n_tot, H, D, dtype)
    sgk = sk.to(DEV) if had else None
    sgv = sv.to(DEV) if had else None
    ref_k, ref_rk = _append_all(d, xk, chunks, sgk)
    ref_v, ref_rv = _append_all(d, xv, chunks, sgv)

    caches = []
    for _ in range(2):
        cache = kvq.alloc_outputs(d, DEV)
        for t in cache:
            if t is not None:
                t.view(torch.uint8).fill_(0xAB)
        caches.append(cache)
    rk, rv = kvq.alloc_residual(d, DEV), kvq.alloc_residual(d, DEV)
    rk.view(torch.uint8).fill_(0xAB)
    rv.view(torch.uint8).fill_(0xAB)
    xkd, xvd = xk.to(DEV), xv.to(DEV)
    n = 0
    for c in chunks:
        n = kvq.append_kv(d, n, xkd[:, n:n + c].contiguous(), xvd[:, n:n + c].contiguous(), rk, rv, caches[0],
                          caches[1], sgk, sgv)
    torch.cuda.synchronize()
    assert n == n_tot
    for got, want in ((caches[0], ref_k), (caches[1], ref_v)):
        for g, w in zip(got, want):
            if w is None:
                assert g is None
            else:
                assert torch.equal(g.view(torch.uint8), w.view(torch.uint8))
    assert torch.equal(rk.view(torch.uint8), ref_rk.view(torch.uint8))
    assert torch.equal(rv.view(torch.uint8), ref_rv.view(torch.uint8))
