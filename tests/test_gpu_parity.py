"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same inputs.

Run on an MI355X.  Inputs are the seeded synthetic workloads (activation_quantization_amd.
synth) or grid inputs with closed-form results (tests/grid.py).
"""
import numpy as np
import pytest
import torch

import oracle
from activation_quantization_amd import kvq, synth
from tests import grid, parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def spec_of(d: kvq.Desc) -> oracle.Spec:
    return oracle.Spec(d.seqs, d.tokens_per_seq, d.heads, d.head_dim, d.bits, d.mode,
                       d.block_tokens if d.per_channel else 0, d.hadamard)


def np16(t):
    return None if t is None else t.cpu().numpy()


def desc_for(w: synth.Workload, bits=None, mode=None, hadamard=None, **kw) -> kvq.Desc:
    mode = mode or w.mode
    return kvq.Desc(w.seqs, w.tokens, w.heads, w.head_dim, bits or w.bits[0], mode,
                    w.block_tokens if "pchan" in mode else 0,
                    w.hadamard if hadamard is None else hadamard, synth.torch_dtype(w), **kw)


def run_full(d: kvq.Desc, x_cpu: torch.Tensor, signs_cpu, lowp_out=True, deq=True):
    """Quantize on the GPU, compare every output with the oracle; then dequantize."""
    x = x_cpu.to(DEV)
    sg = signs_cpu.to(DEV) if signs_cpu is not None else None
    codes, norms, scales = kvq.quantize(d, x, sg)
    torch.cuda.synchronize()
    sp = spec_of(d)
    sg_np = None if signs_cpu is None else signs_cpu.numpy()
    ref = oracle.quantize(x_cpu.double().numpy(), sp, sg_np)
    tc, tn, ts = kvq.token_major(d, codes, norms, scales)     # the oracle's [rows, heads, ...] order
    gc, gn, gs = tc.cpu().numpy(), np16(tn), np16(ts)
    stats = parity.check_codes(gc, ref, d.bits)
    if d.nsep:
        parity.check_rel_f16(gn, ref.nu, "norms")
    parity.check_rel_f16(gs, ref.scale, "scales")
    if deq:
        ref_dq = oracle.dequantize(gc, gn, gs, sp, sg_np)
        y = kvq.dequantize(d, codes, norms, scales, sg, torch.float32)
        torch.cuda.synchronize()
        parity.check_dequant(y.cpu().numpy(), ref_dq)
        if lowp_out:
            y2 = kvq.dequantize(d, codes, norms, scales, sg, d.dtype)
            torch.cuda.synchronize()
            parity.check_dequant_lowp(y2.cpu(), ref_dq, "f16" if d.dtype == torch.float16 else "bf16")
    return stats, (codes, norms, scales)


# ----------------------------------------------------------------------------- grid: bit exact
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("had", [0, 16, 64])
@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_grid_bit_exact(bits, mode, had, dtype):
    sp, x64, signs, k = grid.make(bits, mode, had, head_dim=64, seed=bits * 7 + had)
    d = kvq.Desc(sp.seqs, sp.tokens, sp.heads, sp.head_dim, bits, mode, sp.block_tokens, had, dtype)
    x = torch.from_numpy(x64).to(dtype)
    assert torch.equal(x.double(), torch.from_numpy(x64))
    sg = None if signs is None else torch.from_numpy(signs).to(DEV)
    codes, norms, scales = kvq.quantize(d, x.to(DEV), sg)
    y = kvq.dequantize(d, codes, norms, scales, sg, torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(oracle.unpack_nibbles(kvq.token_major(d, codes)[0].cpu().numpy()), k)
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), x64)


@pytest.mark.parametrize("mode", oracle.MODES)
def test_grid_bit_exact_d128(mode):
    sp, x64, signs, k = grid.make(4, mode, 64, head_dim=128, seed=11)
    d = kvq.Desc(sp.seqs, sp.tokens, sp.heads, 128, 4, mode, sp.block_tokens, 64, torch.float16)
    sg = torch.from_numpy(signs).to(DEV)
    codes, norms, scales = kvq.quantize(d, torch.from_numpy(x64).half().to(DEV), sg)
    y = kvq.dequantize(d, codes, norms, scales, sg, torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(oracle.unpack_nibbles(kvq.token_major(d, codes)[0].cpu().numpy()), k)
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), x64)


# ----------------------------------------------------------------------------- workloads
@pytest.mark.parametrize("mode", oracle.MODES)
@pytest.mark.parametrize("bits", [4, 3])
def test_single_head_d64(mode, bits):
    w = synth.WORKLOADS["single_head_d64"]
    d = desc_for(w, bits=bits, mode=mode)
    run_full(d, synth.make_x(w), None)


@pytest.mark.parametrize("tensor_id", [0, 1])        # K and V
@pytest.mark.parametrize("bits", [4, 3])
def test_qwen_kv_layer(tensor_id, bits):
    w = synth.WORKLOADS["qwen_kv_layer"]
    d = desc_for(w, bits=bits)
    stats, _ = run_full(d, synth.make_x(w, tensor_id=tensor_id), None)
    print(stats)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_batched_hadamard_two_seqs(bits):
    w = synth.scaled("batched_hadamard", seqs=2)
    d = desc_for(w, bits=bits)
    stats, _ = run_full(d, synth.make_x(w), synth.make_signs(w))
    print(stats)


def test_activation_4096_full():
    w = synth.WORKLOADS["activation_4096"]
    d = desc_for(w)
    stats, _ = run_full(d, synth.make_x(w), synth.make_signs(w))
    print(stats)


def _sampled_tiles(d: kvq.Desc, x_cpu, signs_cpu, codes, norms, scales, n_tiles, seed, y=None):
    """Oracle on chosen (seq, block, head) tiles of a full-size GPU run: the first and the last
    tile (the highest element offsets) and n_tiles random ones.  y: the GPU's dequantized output
    of the whole tensor (x's layout and dtype), compared on the same tiles with the oracle's
    dequantization of the GPU's own codes, norms and scales."""
    rng = np.random.default_rng(seed)
    B, nb = d.block_tokens, d.tokens_per_seq // d.block_tokens
    gc, gn, gs = (None if t is None else t.cpu() for t in kvq.token_major(d, codes, norms, scales))
    flips, checked = 0, 0
    tiles = [(0, 0, 0), (d.seqs - 1, nb - 1, d.heads - 1)]
    tiles += [(int(rng.integers(d.seqs)), int(rng.integers(nb)), int(rng.integers(d.heads))) for _ in range(n_tiles)]
    for s, b, h in tiles:
        r0 = s * d.tokens_per_seq + b * B
        xt = x_cpu[r0:r0 + B, h:h + 1].double().numpy()
        sp = oracle.Spec(1, B, 1, d.head_dim, d.bits, d.mode, B, d.hadamard)
        sg = None if signs_cpu is None else signs_cpu[h:h + 1].numpy()
        ref = oracle.quantize(xt, sp, sg)
        c = gc[r0:r0 + B, h:h + 1].numpy()
        st = parity.check_codes(c, ref, d.bits, sampled_from=d.rows * d.heads * d.head_dim)
        flips += st["tie_flips"]
        checked += st["codes"]
        if gn is not None:
            parity.check_rel_f16(gn[r0:r0 + B, h:h + 1].numpy(), ref.nu, "norms")
        parity.check_rel_f16(gs[s * nb + b, h:h + 1].numpy()[None], ref.scale, "scales")
        if y is not None:
            nt = None if gn is None else gn[r0:r0 + B, h:h + 1].numpy()
            dq = oracle.dequantize(c, nt, gs[s * nb + b, h:h + 1].numpy()[None], sp, sg)
            yt = y[r0:r0 + B, h:h + 1].cpu()
            if yt.dtype == torch.float32:
                parity.check_dequant(yt.numpy(), dq)
            else:
                parity.check_dequant_lowp(yt, dq, "f16" if yt.dtype == torch.float16 else "bf16")
    assert flips <= parity.tie_budget(checked, d.rows * d.heads * d.head_dim)
    return checked, flips


def test_batched_hadamard_full_sampled():
    w = synth.WORKLOADS["batched_hadamard"]
    d = desc_for(w)
    x_cpu, signs = synth.make_x(w), synth.make_signs(w)
    sg = signs.to(DEV)
    codes, norms, scales = kvq.quantize(d, x_cpu.to(DEV), sg)
    y16 = kvq.dequantize(d, codes, norms, scales, sg, torch.float16)
    y32 = kvq.dequantize(d, codes, norms, scales, sg, torch.float32)
    torch.cuda.synchronize()
    print(_sampled_tiles(d, x_cpu, signs, codes, norms, scales, 48, seed=3, y=y16))
    print(_sampled_tiles(d, x_cpu, signs, codes, norms, scales, 16, seed=4, y=y32))


# Caches of a few thousand tiles with head counts that are not powers of two and every block size:
# every scale row must be written (they start as NaN), and sampled tiles match the oracle.
@pytest.mark.parametrize("S,T,H,D,B,mode,had,dt", [(5, 1024, 67, 128, 128, "nsep_pchan", 128, torch.float16),
                                                   (5, 1024, 67, 128, 64, "pchan", 32, torch.bfloat16),
                                                   (3, 2048, 100, 64, 256, "nsep_pchan", 64, torch.float16)])
def test_quantize_every_tile_written(S, T, H, D, B, mode, had, dt):
    rng = np.random.default_rng(S * T + H + D + B)
    x = torch.from_numpy(rng.standard_normal((S * T, H, D)).astype(np.float32))
    x[:, :, 3] *= 25
    x = x.to(dt)
    signs = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, D)))
    d = kvq.Desc(S, T, H, D, 4, mode, B, had, dt)
    codes, norms, scales = kvq.alloc_outputs(d, DEV)
    scales.fill_(float("nan"))
    kvq.quantize(d, x.to(DEV), signs.to(DEV), out=(codes, norms, scales))
    torch.cuda.synchronize()
    assert not torch.isnan(scales.float()).any(), "a tile was not written"
    print(_sampled_tiles(d, x, signs, codes, norms, scales, 24, seed=11))


# ----------------------------------------------------------------------------- decode score
def _score_check(d: kvq.Desc, q_cpu, codes, norms, scales, signs_cpu, scores, pairs):
    """Oracle scores for the given (seq, kv head) pairs from the GPU's own cache."""
    G = q_cpu.shape[1] // d.heads
    T, nb = d.tokens_per_seq, (d.tokens_per_seq // d.block_tokens if d.per_channel else 0)
    worst = 0.0
    tc, tn, ts = kvq.token_major(d, codes, norms, scales)
    gc, gn, gs, gsc = tc.cpu(), None if tn is None else tn.cpu(), ts.cpu(), scores.cpu()
    for s, h in pairs:
        rows = slice(s * T, (s + 1) * T)
        sp = oracle.Spec(1, T, 1, d.head_dim, d.bits, d.mode, d.block_tokens if d.per_channel else 0, d.hadamard)
        n16 = None if gn is None else gn[rows, h:h + 1].numpy()
        s16 = gs[s * nb:(s + 1) * nb, h:h + 1].numpy() if d.per_channel else gs[rows, h:h + 1].numpy()
        sg = None if signs_cpu is None else signs_cpu[h:h + 1].numpy()
        k_hat = oracle.dequantize(gc[rows, h:h + 1].numpy(), n16, s16, sp, sg)
        qq = q_cpu[s:s + 1, h * G:(h + 1) * G].double().numpy()
        sp1 = oracle.Spec(1, T, 1, d.head_dim, d.bits, d.mode, sp.block_tokens, d.hadamard)
        ref = np.stack([oracle.score_decode(qq[:, g:g + 1], k_hat, sp1)[0, 0] for g in range(G)])[None]
        got = gsc[s:s + 1, h * G:(h + 1) * G].numpy()
        worst = max(worst, parity.check_scores(got, ref, qq, k_hat, sp1))
    return worst


def test_long_context_decode_scaled():
    w = synth.scaled("long_context_decode", seqs=2, tokens=4096)
    d = desc_for(w)
    x_cpu, signs, q_cpu = synth.make_x(w), synth.make_signs(w), synth.make_q(w)
    _, (codes, norms, scales) = run_full(d, x_cpu, signs, lowp_out=False)
    sc = kvq.score_decode(d, q_cpu.to(DEV), codes, norms, scales, signs.to(DEV))
    torch.cuda.synchronize()
    worst = _score_check(d, q_cpu, codes, norms, scales, signs, sc,
                         [(s, h) for s in range(w.seqs) for h in range(w.heads)])
    print("worst score error / tolerance", worst)


def test_long_context_decode_full_sampled():
    w = synth.WORKLOADS["long_context_decode"]
    d = desc_for(w)
    x_cpu = synth.make_x(w, pin=True)
    signs, q_cpu = synth.make_signs(w), synth.make_q(w)
    x = x_cpu.to(DEV, non_blocking=True)
    sg = signs.to(DEV)
    codes, norms, scales = kvq.quantize(d, x, sg)
    sc = kvq.score_decode(d, q_cpu.to(DEV), codes, norms, scales, sg)
    torch.cuda.synchronize()
    del x
    # the dequantized cache in fp16, as the step writes it (2^31 elements: 64-bit offsets)
    y = kvq.dequantize(d, codes, norms, scales, sg, torch.float16)
    torch.cuda.synchronize()
    print(_sampled_tiles(d, x_cpu, signs, codes, norms, scales, 64, seed=5, y=y))
    del y
    rng = np.random.default_rng(9)
    pairs = [(int(rng.integers(w.seqs)), int(rng.integers(w.heads))) for _ in range(3)] + [(w.seqs - 1, w.heads - 1)]
    print("worst score error / tolerance", _score_check(d, q_cpu, codes, norms, scales, signs, sc, pairs))


@pytest.mark.parametrize("mode", oracle.MODES)
# G = 3 on whole units: the lanes past the pass's last head rewrite that head's row; T = 201: the
# score rows take 4-byte stores and the last unit is partial
@pytest.mark.parametrize("dim,G,T,had", [(128, 4, 512, 128), (64, 1, 256, 0), (128, 16, 384, 32), (64, 8, 200, 64),
                                         (128, 3, 256, 128), (64, 2, 201, 0)])
def test_score_shapes_and_modes(mode, dim, G, T, had):
    if "pchan" in mode and T % 64:
        pytest.skip("per-channel blocks must divide the sequence")
    rng = np.random.default_rng(dim + G + T)
    S, H = 2, 2
    x = torch.from_numpy(rng.standard_normal((S * T, H, dim)).astype(np.float32) * 3).half()
    x[:, :, 5] *= 30
    signs = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, dim))) if had else None
    q = torch.from_numpy(rng.standard_normal((S, H * G, dim)).astype(np.float32)).half()
    d = kvq.Desc(S, T, H, dim, 4, mode, 64 if "pchan" in mode else 0, had, torch.float16)
    sg = None if signs is None else signs.to(DEV)
    codes, norms, scales = kvq.quantize(d, x.to(DEV), sg)
    sc = kvq.score_decode(d, q.to(DEV), codes, norms, scales, sg)
    torch.cuda.synchronize()
    _score_check(d, q, codes, norms, scales, signs, sc, [(s, h) for s in range(S) for h in range(H)])
