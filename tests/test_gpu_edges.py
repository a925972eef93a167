"""GPU edge cases: empty and ragged inputs, zero vectors, wide rows, determinism, and
outputs left untouched when a call is refused."""
import numpy as np
import pytest
import torch

import oracle
from activation_quantization_amd import kvq, synth
from tests import grid, parity
from tests.test_gpu_parity import DEV, run_full

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", oracle.MODES)
def test_empty_input_is_a_no_op(mode):
    d = kvq.Desc(0, 128, 2, 128, 4, mode, 128 if "pchan" in mode else 0, 0)
    x = torch.empty((0, 2, 128), dtype=torch.float16, device=DEV)
    codes, norms, scales = kvq.quantize(d, x)
    y = kvq.dequantize(d, codes, norms, scales)
    assert codes.numel() == 0 and y.numel() == 0


@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("had", [0, 128])
def test_zero_vectors_and_zero_blocks(mode, had):
    rng = np.random.default_rng(1)
    S, T, H, D = 1, 256, 2, 128
    x = torch.from_numpy(rng.standard_normal((S * T, H, D)).astype(np.float32)).half()
    x[5] = 0                      # zero vectors (every head of token 5)
    x[128:256, 1] = 0             # a whole per-channel block of head 1
    x[200, 0, 7] = 0.5            # a lone value inside that region of head 0
    signs = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, D))) if had else None
    d = kvq.Desc(S, T, H, D, 4, mode, 128 if "pchan" in mode else 0, had)
    run_full(d, x, signs)
    codes, norms, scales = kvq.quantize(d, x.to(DEV), None if signs is None else signs.to(DEV))
    tc, tn, ts = kvq.token_major(d, codes, norms, scales)
    c = oracle.unpack_nibbles(tc.cpu().numpy())
    assert np.all(c[5] == 0) and np.all(c[128:256, 1] == 0)
    if d.nsep:
        assert np.all(tn.cpu().numpy()[5] == 0)
    if d.per_channel:
        assert np.all(ts.cpu().numpy()[1, 1] == 0)


@pytest.mark.parametrize("rows,heads,dim,had,mode", [
    (37, 3, 128, 0, "naive"), (37, 3, 128, 128, "nsep"), (9, 5, 64, 16, "naive"),
    (13, 1, 256, 128, "nsep"), (11, 1, 8192, 128, "nsep"), (7, 2, 1024, 32, "naive"),
])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_per_token_ragged_and_wide(rows, heads, dim, had, mode, dtype):
    rng = np.random.default_rng(rows * dim)
    x = torch.from_numpy(rng.standard_normal((rows, heads, dim)).astype(np.float32) *
                         rng.uniform(0.2, 4.0, size=(rows, 1, 1)).astype(np.float32)).to(dtype)
    signs = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(heads, dim))) if had else None
    d = kvq.Desc(1, rows, heads, dim, 4, mode, 0, had, dtype)
    run_full(d, x, signs)


@pytest.mark.parametrize("seqs,rows,heads,dim,had,mode", [
    (2, 128, 3, 64, 16, "naive"), (2, 64, 3, 128, 128, "nsep"), (3, 128, 2, 512, 64, "nsep"),
    (1, 192, 1, 8192, 128, "naive"), (2, 64, 5, 1024, 0, "nsep"),
])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_per_token_whole_chunks(seqs, rows, heads, dim, had, mode, dtype):
    # tokens per sequence a multiple of 64: per-token dequantize runs on the matrix cores, a
    # vector of more than 128 channels walked as 128-channel segments
    rng = np.random.default_rng(seqs * rows * dim + heads)
    x = torch.from_numpy(rng.standard_normal((seqs * rows, heads, dim)).astype(np.float32) *
                         rng.uniform(0.2, 4.0, size=(seqs * rows, 1, 1)).astype(np.float32)).to(dtype)
    signs = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(heads, dim))) if had else None
    d = kvq.Desc(seqs, rows, heads, dim, 4, mode, 0, had, dtype)
    run_full(d, x, signs)


def test_block_256_d64():
    w = synth.scaled("single_head_d64", tokens=1024, heads=3)
    d = kvq.Desc(1, 1024, 3, 64, 3, "nsep_pchan", 256, 64, torch.float16)
    run_full(d, synth.make_x(w), synth.make_signs(w))


def test_deterministic_bytes():
    w = synth.WORKLOADS["qwen_kv_layer"]
    d = kvq.Desc(1, 4096, 4, 128, 4, "nsep_pchan", 128, 128, torch.bfloat16)
    x, sg = synth.make_x(w).to(DEV), synth.make_signs(w).to(DEV)
    a = [t.clone() for t in kvq.quantize(d, x, sg)]
    b = kvq.quantize(d, x, sg)
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))
    q = torch.randn(1, 16, 128, generator=torch.Generator().manual_seed(0)).half().to(DEV)
    s1 = kvq.score_decode(d, q, *a, sg)
    s2 = kvq.score_decode(d, q, *a, sg)
    assert torch.equal(s1, s2)


def test_outputs_untouched_on_refusal():
    d = kvq.Desc(1, 256, 2, 128, 4, "nsep_pchan", 128, 0)
    x = torch.randn(256 * 2 * 128 + 8, device=DEV).half()
    codes, norms, scales = kvq.alloc_outputs(d, DEV)
    for t in (codes, norms, scales):
        t.view(torch.uint8).fill_(0xAB)
    bad_x = x[1:1 + 256 * 2 * 128].view(256, 2, 128)          # 2-byte offset: misaligned
    with pytest.raises(kvq.KvqError) as e:
        kvq.quantize(d, bad_x, None, out=(codes, norms, scales))
    assert e.value.status == kvq.ERR_ALIGN
    bad_d = kvq.Desc(1, 250, 2, 128, 4, "nsep_pchan", 128, 0)
    with pytest.raises(kvq.KvqError) as e:
        kvq.quantize(bad_d, x[:250 * 256].view(250, 2, 128), None, out=(codes, norms, scales))
    assert e.value.status == kvq.ERR_SHAPE
    torch.cuda.synchronize()
    for t in (codes, norms, scales):
        assert bool((t.view(torch.uint8) == 0xAB).all())


def test_f16_subnormal_scales_and_large_norms():
    # tiny vectors give subnormal fp16 scales; norms up to ~6e4 stay finite
    rng = np.random.default_rng(4)
    x = rng.standard_normal((128, 1, 128)).astype(np.float32)
    x[:64] *= 1e-6
    x[64:] *= 3000.0
    xt = torch.from_numpy(x).half()
    for mode in ("naive", "nsep"):
        d = kvq.Desc(1, 128, 1, 128, 4, mode, 0, 0)
        stats, (codes, norms, scales) = run_full(d, xt, None)
        assert np.all(np.isfinite(scales.cpu().numpy().astype(np.float32)))


def test_tie_flip_rate_report():
    # the rate of rounding-tie flips on the largest element-wise workload, for the record
    w = synth.scaled("batched_hadamard", seqs=4)
    d = kvq.Desc(w.seqs, w.tokens, w.heads, w.head_dim, 4, "nsep_pchan", 128, 128, torch.float16)
    stats, _ = run_full(d, synth.make_x(w), synth.make_signs(w), deq=False)
    print("tie flips", stats, "rate", stats["tie_flips"] / stats["codes"])
    assert stats["tie_flips"] <= parity.tie_budget(stats["codes"])


@pytest.mark.parametrize("had", [0, 16])
@pytest.mark.parametrize("mode", oracle.MODES)
def test_exact_ties_are_rounded_half_even(mode, had):
    x64, signs, want = grid.all_ties(had)
    d = kvq.Desc(1, 128, 2, 64, 4, mode, 64 if "pchan" in mode else 0, had, torch.float16)
    sg = None if signs is None else torch.from_numpy(signs).to(DEV)
    codes, norms, scales = kvq.quantize(d, torch.from_numpy(x64).half().to(DEV), sg)
    torch.cuda.synchronize()
    got = oracle.unpack_nibbles(kvq.token_major(d, codes)[0].cpu().numpy())
    np.testing.assert_array_equal(got, want)
    # and the oracle agrees (rne of the exact quotient)
    sp = oracle.Spec(1, 128, 2, 64, 4, mode, d.block_tokens if "pchan" in mode else 0, had)
    np.testing.assert_array_equal(oracle.quantize(x64, sp, signs).codes, want)


@pytest.mark.parametrize("dim,had,extra_max", [(256, 0, 0), (512, 64, 0), (1024, 16, 0), (512, 64, 3), (128, 64, 2)])
@pytest.mark.parametrize("mode", ["naive", "nsep"])
def test_exact_ties_wide_per_token(mode, dim, had, extra_max):
    # a vector spans several 128-channel row segments: every code is a tie and the exact max
    # (the 7s) sits in one segment, or in several, so the re-decision needs the max from other
    # lanes
    x64, signs, want = grid.all_ties(had, seed=dim, T=96, H=2, D=dim, extra_max=extra_max)
    d = kvq.Desc(1, 96, 2, dim, 4, mode, 0, had, torch.float16)
    sg = None if signs is None else torch.from_numpy(signs).to(DEV)
    codes, norms, scales = kvq.quantize(d, torch.from_numpy(x64).half().to(DEV), sg)
    torch.cuda.synchronize()
    got = oracle.unpack_nibbles(kvq.token_major(d, codes)[0].cpu().numpy())
    np.testing.assert_array_equal(got, want)
    sp = oracle.Spec(1, 96, 2, dim, 4, mode, 0, had)
    np.testing.assert_array_equal(oracle.quantize(x64, sp, signs).codes, want)


@pytest.mark.parametrize("had,extra_max", [(0, 0), (64, 0), (64, 3), (0, 5)])
@pytest.mark.parametrize("mode", ["pchan", "nsep_pchan"])
def test_exact_ties_per_channel_d128(mode, had, extra_max):
    # head_dim 128 and 128-token blocks: every code is a tie, in both 64-channel halves of each
    # wave's channels, every value of every wave is re-decided exactly, and with extra_max > 0 a
    # channel's max sits in several tokens at once
    x64, signs, want = grid.all_ties(had, seed=7 + extra_max, T=128, H=2, D=128, extra_max=extra_max)
    d = kvq.Desc(1, 128, 2, 128, 4, mode, 128, had, torch.float16)
    sg = None if signs is None else torch.from_numpy(signs).to(DEV)
    codes, norms, scales = kvq.quantize(d, torch.from_numpy(x64).half().to(DEV), sg)
    torch.cuda.synchronize()
    got = oracle.unpack_nibbles(kvq.token_major(d, codes)[0].cpu().numpy())
    np.testing.assert_array_equal(got, want)
    sp = oracle.Spec(1, 128, 2, 128, 4, mode, 128, had)
    np.testing.assert_array_equal(oracle.quantize(x64, sp, signs).codes, want)


@pytest.mark.parametrize("dim", [64, 128])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("mode", oracle.MODES)
def test_near_ties_follow_the_exact_quotient(mode, bits, dtype, dim):
    # quotients a hair (~2^-26) above and below a tie that half-to-even rounds down: the codes are
    # the rounding of the exact quotient (rational arithmetic, tests/grid.py), with no tie band;
    # a decision on the fp32 quotient would give the tie's even neighbour for both.  With head_dim
    # 128 the flagged channels 0..15 fall in both 4-channel halves of the first wave's slots.
    per_channel = "pchan" in mode
    x64, signs, want = grid.near_ties(bits, per_channel, D=dim, B=dim)
    d = kvq.Desc(1, dim, 1, dim, bits, mode, dim if per_channel else 0, 16, dtype)
    codes, norms, scales = kvq.quantize(d, torch.from_numpy(x64).to(dtype).to(DEV), torch.from_numpy(signs).to(DEV))
    torch.cuda.synchronize()
    got = oracle.unpack_nibbles(kvq.token_major(d, codes)[0].cpu().numpy())
    np.testing.assert_array_equal(got, want)
