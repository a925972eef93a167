"""The no-alloc decode attention entry point (kvq_attention_decode_noalloc, partials in the
library's static per-GPU scratch) against kvq_attention_decode with a caller workspace, through the
C ABI: outputs must be identical, on two calls in a row (the second on a smaller cache, so the
scratch holds the first call's partials when it starts), and the oracle agrees with both."""
import numpy as np
import pytest
import torch

import oracle
from activation_quantization_amd import kvq
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _caches(seed, S, T, H, G, B, had):
    rng = np.random.default_rng(seed)
    D = 128
    xk = torch.from_numpy(rng.standard_normal((S * T, H, D)).astype(np.float32) * 2).half()
    xk[:, :, 9] *= 25                                   # an outlier channel
    xv = torch.from_numpy(rng.standard_normal((S * T, H, D)).astype(np.float32)).half()
    q = torch.from_numpy(rng.standard_normal((S, H * G, D)).astype(np.float32)).half().to(DEV)
    sk = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, D))).to(DEV) if had else None
    sv = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, D))).to(DEV) if had else None
    d = kvq.Desc(S, T, H, D, 4, "nsep_pchan", B, had, torch.float16)
    kc = kvq.quantize(d, xk.to(DEV), sk)
    vc = kvq.quantize(d, xv.to(DEV), sv)
    return d, q, kc, vc, sk, sv


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 4 sequences x 8192 tokens, 4 KV heads, GQA 4 (133 kB of partials); second call: a
    # smaller cache (2 x 1024 tokens, 2 KV heads, GQA 2, B = 64, no rotation)
    for seed, (S, T, H, G, B, had) in ((1, (4, 8192, 4, 4, 128, 128)), (2, (2, 1024, 2, 2, 64, 0))):
        d, q, kc, vc, sk, sv = _caches(seed, S, T, H, G, B, had)
        assert 0 < kvq.attention_workspace_bytes(d, q.shape[1]) <= 32 << 20
        want = kvq.attention_decode(d, q, kc, vc, sk, sv)
        got = torch.full_like(want, float("nan"))
        kvq.attention_decode_noalloc(d, q, kc, vc, sk, sv, out=got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"seed {seed}: no-alloc output differs from the workspace entry point"
        # and both agree with the oracle on one (sequence, KV head) pair
        tc, tn, ts = (t.cpu().numpy() for t in kvq.token_major(d, *kc))
        vtc, vtn, vts = (t.cpu().numpy() for t in kvq.token_major(d, *vc))
        sp = oracle.Spec(d.seqs, d.tokens_per_seq, d.heads, d.head_dim, d.bits, d.mode, d.block_tokens, d.hadamard)
        k_hat = oracle.dequantize(tc, tn, ts, sp, None if sk is None else sk.cpu().numpy())
        v_hat = oracle.dequantize(vtc, vtn, vts, sp, None if sv is None else sv.cpu().numpy())
        ref = oracle.attention_decode(q.cpu().double().numpy(), k_hat, v_hat, sp)
        parity.check_attention(got.cpu().numpy(), ref)


def test_noalloc_refuses_partials_beyond_the_scratch():
    # 512 sequences x 32768 tokens, 8 KV heads, 32 query heads: 136 MB of partials > 32 MiB
    d = kvq.Desc(512, 32768, 8, 128, 4, "nsep_pchan", 128, 128, torch.float16)
    assert kvq.attention_workspace_bytes(d, 32) > 32 << 20
    q = torch.zeros((1, 32, 128), dtype=torch.float16, device=DEV)   # never read: refused before any launch
    t = torch.zeros(16, dtype=torch.float16, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.attention_decode_noalloc(d, q, (t, t, t), (t, t, t), t, t, out=torch.zeros(4, device=DEV))
    assert e.value.status == kvq.ERR_UNSUPPORTED and "static scratch" in str(e.value)
