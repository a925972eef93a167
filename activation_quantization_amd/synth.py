"""Seeded synthetic KV-cache / activation tensors with the statistics the pages describe.

This module only draws random numbers and casts them to the storage dtype; it holds
none of the quantizer's arithmetic.  Both the fp64 oracle (via the tests) and the HIP
path read the very same host bytes produced here.

Statistics (source pages):
  * per-token norm swing of 2-5x in Pre-LN models  -- norm-separation post, "root cause"
  * persistent outlier channels 8-100x the mean; Qwen2-7B layer 0 has 8 channels with
    absmax 167                                      -- same post, "root cause"
  * isolated spike outliers                         -- Rotated Runtime Smooth analysis,
                                                       "problem definition" (channel-wise vs spike)

Recipe (identical for every config unless stated):
  * base values z ~ N(0, 1)
  * token factor f_t = exp(0.25 g_t), g_t ~ N(0, 1), clipped to [e^-0.6, e^0.6] and
    divided by its maximum within the sequence (span <= 3.32, max 1); it multiplies the
    whole token, outlier channels included.
  * "qwen" outliers: per head, 8 distinct channels, a fixed random sign per channel,
    magnitude U(100, 167) drawn per element, times f_t (they replace the base value).
  * spikes (batched-cache config only): each element independently with p = 1e-3 is
    replaced by +-50 f_t (uniform sign).
  * RNG: numpy PCG64 seeded by SeedSequence([seed, cfg_id, tensor_id, chunk]); chunk is the
    sequence index.  Outlier channels/signs come from chunk 10**6, Hadamard signs from
    10**6 + 1, decode queries from 10**6 + 2, so they are fixed per head across sequences.
  * cast to fp16 / bf16 with round-to-nearest-even (torch CPU cast).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np
import torch

OUTLIER_STREAM = 10**6
SIGN_STREAM = 10**6 + 1
QUERY_STREAM = 10**6 + 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: tensor x is [seqs * tokens, heads, head_dim]."""
    name: str
    cfg_id: int
    seqs: int
    tokens: int          # tokens per sequence
    heads: int           # KV heads (1 for the activation workload)
    head_dim: int
    dtype: str           # "f16" | "bf16"
    mode: str            # main mode: "naive" | "nsep" | "pchan" | "nsep_pchan"
    bits: tuple          # bit widths exercised
    block_tokens: int    # per-channel token block (0 for per-token modes)
    hadamard: int        # 0 = no rotation, else Hadamard block size
    outliers: str        # "ch3_17" | "qwen" | "act16"
    spikes: float = 0.0  # probability of a spike per element
    q_heads: int = 0     # decode query heads (0 = no decode step)
    tensors: int = 1     # 2 for a K/V pair

    @property
    def rows(self) -> int:
        return self.seqs * self.tokens

    @property
    def numel(self) -> int:
        return self.rows * self.heads * self.head_dim


WORKLOADS = {
    # one KV head, 256 tokens x 64 channels, fp16; channels 3 and 17 x20
    "single_head_d64": Workload("single_head_d64", 1, 1, 256, 1, 64, "f16", "nsep_pchan",
                                (4,), 64, 0, "ch3_17"),
    # Qwen2-7B-like layer KV: K and V each [4096, 4, 128] bf16
    "qwen_kv_layer": Workload("qwen_kv_layer", 2, 1, 4096, 4, 128, "bf16", "nsep_pchan",
                              (4, 3), 128, 0, "qwen", tensors=2),
    # batched cache with randomized Hadamard: [16 x 2048, 32, 128] fp16 + 0.1% spikes
    "batched_hadamard": Workload("batched_hadamard", 3, 16, 2048, 32, 128, "f16", "nsep_pchan",
                                 (4, 3, 2), 128, 128, "qwen", spikes=1e-3),
    # activations [8192, 4096] bf16, block Hadamard 128, per-token INT4
    "activation_4096": Workload("activation_4096", 4, 1, 8192, 1, 4096, "bf16", "naive",
                                (4,), 0, 128, "act16"),
    # long-context decode: K cache [64 x 32768, 8, 128] fp16, GQA 4 (32 query heads)
    "long_context_decode": Workload("long_context_decode", 5, 64, 32768, 8, 128, "f16",
                                    "nsep_pchan", (4,), 128, 128, "qwen", q_heads=32),
}


def _rng(seed: int, cfg_id: int, tensor_id: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, tensor_id, chunk])))


def _token_factor(rng: np.random.Generator, tokens: int, lognormal_sigma: float | None) -> np.ndarray:
    g = rng.standard_normal(tokens)
    if lognormal_sigma is None:
        f = np.exp(np.clip(0.25 * g, -0.6, 0.6))
        return f / f.max()
    return np.exp(lognormal_sigma * g)   # activation workload: lognormal(0, 0.5), unclipped


def outlier_layout(w: Workload, seed: int = 0, tensor_id: int = 0):
    """Fixed outlier channels (per head) and their signs / multipliers."""
    rng = _rng(seed, w.cfg_id, tensor_id, OUTLIER_STREAM)
    if w.outliers == "ch3_17":
        return {"channels": np.array([[3, 17]] * w.heads), "scale": 20.0}
    if w.outliers == "qwen":
        ch = np.stack([rng.choice(w.head_dim, size=8, replace=False) for _ in range(w.heads)])
        sign = rng.choice(np.array([-1.0, 1.0]), size=ch.shape)
        return {"channels": ch, "sign": sign}
    if w.outliers == "act16":
        ch = rng.choice(w.head_dim, size=16, replace=False)[None, :]
        mult = rng.uniform(30.0, 100.0, size=ch.shape)
        return {"channels": ch, "mult": mult}
    raise ValueError(w.outliers)


def _sequence_f32(w: Workload, seed: int, tensor_id: int, s: int, lay) -> np.ndarray:
    rng = _rng(seed, w.cfg_id, tensor_id, s)
    z = rng.standard_normal((w.tokens, w.heads, w.head_dim), dtype=np.float32)
    if w.outliers == "act16":
        f = _token_factor(rng, w.tokens, 0.5).astype(np.float32)
        ch = lay["channels"][0]
        z[:, 0, ch] *= lay["mult"][0].astype(np.float32)
        z *= f[:, None, None]
        return z
    f = _token_factor(rng, w.tokens, None).astype(np.float32)
    if w.outliers == "ch3_17":
        z *= f[:, None, None]
        z[:, :, lay["channels"][0]] *= np.float32(lay["scale"])
        return z
    # qwen-like: outlier channels replaced by sign * U(100, 167), then everything times f_t
    for h in range(w.heads):
        ch = lay["channels"][h]
        mag = rng.uniform(100.0, 167.0, size=(w.tokens, ch.size)).astype(np.float32)
        z[:, h, ch] = mag * lay["sign"][h].astype(np.float32)
    if w.spikes > 0.0:
        hit = rng.random(z.shape, dtype=np.float32) < np.float32(w.spikes)
        sgn = np.where(rng.random(z.shape, dtype=np.float32) < 0.5, -50.0, 50.0).astype(np.float32)
        z = np.where(hit, sgn, z)
    z *= f[:, None, None]
    return z


def torch_dtype(w_or_name) -> torch.dtype:
    name = w_or_name.dtype if isinstance(w_or_name, Workload) else w_or_name
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[name]


def make_x(w: Workload | str, seed: int = 0, tensor_id: int = 0, seq_range=None,
           pin: bool = False, threads: int | None = None) -> torch.Tensor:
    """x for sequences [a, b) as a CPU tensor [(b-a) * tokens, heads, head_dim] in w.dtype."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    a, b = seq_range if seq_range is not None else (0, w.seqs)
    lay = outlier_layout(w, seed, tensor_id)
    out = torch.empty(((b - a) * w.tokens, w.heads, w.head_dim), dtype=torch_dtype(w), pin_memory=pin)

    def one(s):
        blk = _sequence_f32(w, seed, tensor_id, s, lay)
        out[(s - a) * w.tokens:(s - a + 1) * w.tokens].copy_(torch.from_numpy(blk))

    n = threads or min(16, os.cpu_count() or 1)
    if b - a <= 1 or n <= 1:
        for s in range(a, b):
            one(s)
    else:
        with _cf.ThreadPoolExecutor(n) as ex:
            list(ex.map(one, range(a, b)))
    return out


def make_signs(w: Workload | str, seed: int = 0, tensor_id: int = 0) -> torch.Tensor:
    """Random +-1 signs, int8 [heads, head_dim] (one vector per head, shared by all tokens)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = _rng(seed, w.cfg_id, tensor_id, SIGN_STREAM)
    s = rng.choice(np.array([-1, 1], dtype=np.int8), size=(w.heads, w.head_dim))
    return torch.from_numpy(s)


def make_q(w: Workload | str, seed: int = 0, seq_range=None) -> torch.Tensor:
    """Decode queries, fp16 [seqs, q_heads, head_dim], N(0, 1)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = _rng(seed, w.cfg_id, 0, QUERY_STREAM)
    q = rng.standard_normal((w.seqs, w.q_heads, w.head_dim), dtype=np.float32)
    if seq_range is not None:
        q = q[seq_range[0]:seq_range[1]]
    return torch.from_numpy(np.ascontiguousarray(q)).to(torch.float16)


WEIGHT_STREAM = 1 << 20     # chunk id of the synthetic weight stream (disjoint from the sequences)


def make_weights(m: int, k: int, seed: int = 0, dtype: str = "bf16", std: float = 0.02) -> torch.Tensor:
    """Synthetic linear-layer weights [m, k] (no trained weights are available): N(0, std^2),
    with every 64th output row scaled x8 (a few large rows, as in trained layers), in dtype."""
    rng = _rng(seed, 99, 7, WEIGHT_STREAM)
    wt = rng.standard_normal((m, k), dtype=np.float32) * np.float32(std)
    wt[::64] *= np.float32(8.0)
    return torch.from_numpy(wt).to(torch_dtype(dtype))


def scaled(w: Workload | str, **changes) -> Workload:
    """The same statistics at another size (e.g. fewer sequences for CPU-sized parity)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return dataclasses.replace(w, **changes)
