"""The register-butterfly per-token kernels (selected with KVQ_ROTATION=butterfly, the variant the
matrix-core rotation is measured against) keep parity with the oracle: per-token quantize and
dequantize on the activation workload and on a KV cache with several heads, and the RRS activation
quantizer."""
import numpy as np
import pytest
import torch

import oracle
from activation_quantization_amd import kvq, synth
from tests import parity
from tests.test_gpu_parity import DEV, desc_for, run_full

pytestmark = pytest.mark.gpu


@pytest.fixture
def butterfly(monkeypatch):
    monkeypatch.setenv("KVQ_ROTATION", "butterfly")


def test_activation_4096_butterfly(butterfly):
    w = synth.WORKLOADS["activation_4096"]
    stats, _ = run_full(desc_for(w), synth.make_x(w), synth.make_signs(w))
    print(stats)


@pytest.mark.parametrize("mode", ["naive", "nsep"])
def test_kv_heads_butterfly(butterfly, mode):
    rng = np.random.default_rng(3)
    S, T, H, D = 2, 192, 3, 128
    x = torch.from_numpy(rng.standard_normal((S * T, H, D)).astype(np.float32) * 2).half()
    x[:, :, 11] *= 25
    signs = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=(H, D)))
    run_full(kvq.Desc(S, T, H, D, 4, mode, 0, 128, torch.float16), x, signs)


def test_butterfly_and_matrix_core_codes_agree(monkeypatch):
    # both kernels decide every code as the oracle does, so they agree code for code (away from
    # ties, which both re-decide exactly)
    w = synth.WORKLOADS["activation_4096"]
    d = desc_for(w)
    x, sg = synth.make_x(w).to(DEV), synth.make_signs(w).to(DEV)
    a = kvq.quantize(d, x, sg)
    monkeypatch.setenv("KVQ_ROTATION", "butterfly")
    b = kvq.quantize(d, x, sg)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])
    parity.check_rel_f16(b[2].cpu().numpy(), a[2].cpu().numpy().astype(np.float64), "scales")


def test_rrs_act_butterfly(butterfly):
    n, k = 300, 4096
    rng = np.random.default_rng(8)
    x = torch.from_numpy(rng.standard_normal((n, k)).astype(np.float32)).to(torch.bfloat16)
    sg = torch.from_numpy(rng.choice(np.array([-1, 1], np.int8), size=k))
    s = kvq.rrs_smooth_scales(x.to(DEV), sg.to(DEV), 128)
    xc, xa = kvq.rrs_quantize_act(x.to(DEV), sg.to(DEV), 128, s, 4)
    torch.cuda.synchronize()
    act = oracle.rrs_quantize_act(x.double().numpy(), sg.numpy(), 128, s.double().cpu().numpy(), 4)
    parity.check_codes(xc.cpu().numpy(), act, 4)
    parity.check_rel_f16(xa.cpu().numpy(), act.scale, "activation scales")
