"""The synthetic inputs reproduce the statistics the pages print (tests/golden/page_figures.json)."""
import hashlib
import json
import os

import numpy as np

from activation_quantization_amd import synth

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_regenerates_byte_identically():
    import torch
    a = synth.make_x("qwen_kv_layer", tensor_id=1).view(torch.int16).numpy().tobytes()
    b = synth.make_x("qwen_kv_layer", tensor_id=1).view(torch.int16).numpy().tobytes()
    assert hashlib.sha256(a).hexdigest() == hashlib.sha256(b).hexdigest()


def test_sequences_are_independent_chunks():
    w = synth.scaled("batched_hadamard", seqs=3, heads=4)
    full = synth.make_x(w)
    part = synth.make_x(w, seq_range=(1, 3))
    assert np.array_equal(full[w.tokens:].float().numpy(), part.float().numpy())


def test_qwen_like_outliers_match_page_figures():
    w = synth.WORKLOADS["qwen_kv_layer"]
    x = synth.make_x(w).float().numpy()
    lay = synth.outlier_layout(w)
    n_out = FIG["outlier_channels_per_head"]["value"]
    amax = FIG["outlier_absmax"]["value"]
    lo, hi = FIG["norm_swing"]["value"]
    for h in range(w.heads):
        ch_max = np.abs(x[:, h, :]).max(axis=0)
        top = np.argsort(ch_max)[-n_out:]
        assert set(top) == set(lay["channels"][h])
        assert amax * 0.95 <= ch_max[top].max() <= amax * 1.001
        others = np.delete(np.arange(w.head_dim), top)
        ratio = np.abs(x[:, h, top]).mean() / np.abs(x[:, h, others]).mean()
        assert ratio > FIG["outlier_factor_vs_mean"]["value"][0]
        nrm = np.linalg.norm(x[:, h, :], axis=-1)
        assert lo <= nrm.max() / nrm.min() <= hi


def test_spike_rate():
    w = synth.scaled("batched_hadamard", seqs=1, heads=8)
    x = synth.make_x(w).float().numpy()
    lay = synth.outlier_layout(w)
    big = np.abs(x) > 20.0
    for h in range(8):
        big[:, h, lay["channels"][h]] = False
    rate = big.mean()
    assert 0.5e-3 < rate < 1.5e-3


def test_activation_outliers():
    w = synth.WORKLOADS["activation_4096"]
    part = synth.scaled(w, tokens=512)
    x = synth.make_x(part).float().numpy()[:, 0, :]
    lay = synth.outlier_layout(w)
    top = np.argsort(np.abs(x).mean(axis=0))[-16:]
    assert set(top) == set(lay["channels"][0])
