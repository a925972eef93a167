"""Host logic: the head-major output layout and its token-major views (no GPU needed)."""
import itertools

import torch

from activation_quantization_amd import kvq


def _desc(mode, S=2, T=8, H=3, D=4, B=4):
    return kvq.Desc(S, T, H, D, 4, mode, B if "pchan" in mode else 0, 0, torch.float16)


def test_token_major_matches_index_formula():
    # entry (s, h, t) of a head-major stream is row s*T + t, head h of x's order
    for mode in ("nsep", "nsep_pchan"):
        d = _desc(mode)
        S, T, H, D, B = d.seqs, d.tokens_per_seq, d.heads, d.head_dim, d.block_tokens
        codes = torch.arange(S * H * T * (D // 2), dtype=torch.int32).reshape(d.codes_shape())
        norms = torch.arange(S * H * T, dtype=torch.int32).reshape(d.norms_shape())
        scales = torch.arange(int(torch.tensor(d.scales_shape()).prod()), dtype=torch.int32).reshape(d.scales_shape())
        c, n, sc = kvq.token_major(d, codes, norms, scales)
        for s, t, h in itertools.product(range(S), range(T), range(H)):
            assert torch.equal(c[s * T + t, h], codes[s, h, t])
            assert n[s * T + t, h] == norms[s, h, t]
        if d.per_channel:
            for s, b, h in itertools.product(range(S), range(T // B), range(H)):
                assert torch.equal(sc[s * (T // B) + b, h], scales[s, h, b])
        else:
            for s, t, h in itertools.product(range(S), range(T), range(H)):
                assert sc[s * T + t, h] == scales[s, h, t]


def test_head_major_inverts_token_major():
    for mode in ("naive", "pchan", "nsep", "nsep_pchan"):
        d = _desc(mode)
        codes = torch.randint(0, 255, d.codes_shape(), dtype=torch.uint8)
        norms = torch.randn(d.norms_shape()).half() if d.nsep else None
        scales = torch.randn(d.scales_shape()).half()
        back = kvq.head_major(d, *kvq.token_major(d, codes, norms, scales))
        assert torch.equal(back[0], codes) and torch.equal(back[2], scales)
        assert (back[1] is None) == (norms is None) and (norms is None or torch.equal(back[1], norms))


def test_shapes_hold_the_counts_the_abi_reports():
    d = _desc("nsep_pchan", S=3, T=256, H=2, D=128, B=128)
    assert d.codes_shape() == (3, 2, 256, 64)
    assert d.norms_shape() == (3, 2, 256)
    assert d.scales_shape() == (3, 2, 2, 128)
