"""Seeded synthetic workloads shaped like the pages' serving scenarios.

This module only draws random numbers and holds shapes; it contains none of the
quantization or attention arithmetic, so both the HIP path's tests and the CPU
oracle can consume what it produces.

Shapes and value models follow the scenarios the pages discuss: a Llama-2-7B
layer and a 70B model at 128K context [P3, section on HBM being the ceiling;
P4, section "Le problème"], GQA models [P2, family three], and the outlier
structure that motivates KIVI: a few key channels carry much larger values and
a few value tokens are large across all channels [P4, section "KIVI (2024)"
and the section on naive INT8/INT4 quantization].

  [P2] zubnet.ai survey of KV-cache compression techniques.
  [P3] encorp.ai, "La compression du cache KV est une décision d'infrastructure ...".
  [P4] patricehuetz.fr, "Quantification du KV-Cache : TurboQuant et l'état de l'art en 2026".

Values are drawn in fp32 with torch generators and rounded (nearest-even) to the
workload's input dtype. Everything is reproducible from (workload, seed, layer).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int                 # tokens per sequence (ragged: the cap)
    dtype: str                   # "f16" | "bf16"
    k_bits: int
    v_bits: int
    k_group: int                 # G
    v_group: int                 # G_V
    residual: int                # R
    value_model: str             # "outlier" | "lognormal"
    layers: int = 1
    paged: bool = False
    ragged: bool = False         # lengths lognormal(median 8192, sigma 1) clipped
    ragged_min: int = 1024
    fixed_hot_channels: tuple = ()
    hot_channels: int = 4        # per (sequence, kv head), x20
    hot_token_frac: float = 0.02  # of V tokens, x15 (outlier model)
    description: str = ""

    @property
    def n_g(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, 1, 1, 64, 512, "f16", 2, 2, 32, 32, 32, "outlier",
        fixed_hot_channels=(3, 17, 40, 61),
        description="1 seq, 1 head, d=64, S=512, fp16, INT2 K/V, G=G_V=32, R=32"),
    "llama2-7b-layer": Workload(
        "llama2-7b-layer", 8, 32, 32, 128, 4096, "f16", 2, 2, 32, 32, 128, "outlier",
        description="Llama-2-7B-shaped layer: MHA 32 heads, d=128, batch 8, S=4096, "
                    "fp16, INT2 K/V, G=32, R=128"),
    "llama3-8b-gqa-int4": Workload(
        "llama3-8b-gqa-int4", 32, 32, 8, 128, 32768, "bf16", 4, 4, 32, 32, 128, "lognormal",
        description="Llama-3-8B-shaped GQA layer 32/8, d=128, batch 32, S=32768, bf16, INT4, G=32, R=128"),
    "llama3-8b-gqa-int2": Workload(
        "llama3-8b-gqa-int2", 32, 32, 8, 128, 32768, "bf16", 2, 2, 32, 32, 128, "lognormal",
        description="Llama-3-8B-shaped GQA layer 32/8, d=128, batch 32, S=32768, bf16, INT2, G=32, R=128"),
    "llama-70b-128k-80layer": Workload(
        "llama-70b-128k-80layer", 4, 64, 8, 128, 131072, "bf16", 2, 2, 64, 64, 128, "lognormal",
        layers=80,
        description="70B-shaped 80-layer decode step: GQA 64/8, d=128, batch 4, S=131072, "
                    "bf16, INT2 K/V, G=G_V=64, R=128"),
    "ragged-paged": Workload(
        "ragged-paged", 64, 48, 8, 128, 65536, "bf16", 4, 2, 16, 32, 64, "lognormal",
        paged=True, ragged=True,
        description="64 ragged sequences (lognormal median 8K, clipped [1K, 64K]), GQA 48/8, "
                    "d=128, 16-token pages, K INT4 / V INT2, G=16, G_V=32, R=64, bf16"),
}


def _seed(*parts) -> int:
    h = 1469598103934665603
    for p in parts:
        for ch in str(p).encode():
            h = ((h ^ ch) * 1099511628211) & ((1 << 63) - 1)
        h = ((h ^ 0xFF) * 1099511628211) & ((1 << 63) - 1)
    return h


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def sequence_lengths(w: Workload, seed: int = 0) -> list[int]:
    """Per-sequence token counts. Ragged: 8192*exp(N(0,1)), rounded, clipped to
    [ragged_min, seq_len], with the normal draws taken from numpy's
    default_rng(seed). For the 64-sequence paged workload at seed 0 that is
    840,699 tokens in all (shortest 1,024, median 8,769, longest 58,173)."""
    if not w.ragged:
        return [w.seq_len] * w.batch
    z = np.random.default_rng(seed).standard_normal(w.batch)
    lens = np.clip(np.round(8192.0 * np.exp(z)), w.ragged_min, w.seq_len)
    return [int(x) for x in lens]


@dataclass
class LayerInputs:
    k: torch.Tensor          # [B][H_kv][S_max][d] input dtype
    v: torch.Tensor          # [B][H_kv][S_max][d]
    q: torch.Tensor          # [B][H_q][d]
    lengths: list            # S_b
    k_channel_scale: torch.Tensor  # [B][H_kv][d] fp32 multiplier used for keys
    v_hot_prob: float


def channel_scales(w: Workload, device, layer: int = 0, seed: int = 0) -> torch.Tensor:
    """Key multiplier [B][H_kv][d]: e^Z with Z ~ N(0,1) per (kv head, channel),
    shared by the sequences (lognormal model), times 20 on the hot channels,
    drawn per (sequence, kv head) (or fixed)."""
    B, H, d = w.batch, w.num_kv_heads, w.head_dim
    g = _gen(device, w.name, seed, layer, "kscale")
    scale = torch.ones(B, H, d, device=device, dtype=torch.float32)
    if w.value_model == "lognormal":
        z = torch.randn(H, d, generator=g, device=device, dtype=torch.float32)
        scale = scale * torch.exp(z)[None, :, :]
    if w.fixed_hot_channels:
        idx = torch.tensor(w.fixed_hot_channels, device=device, dtype=torch.long)
        scale[:, :, idx] *= 20.0
    elif w.hot_channels:
        r = torch.rand(B, H, d, generator=g, device=device)
        hot = torch.argsort(r, dim=-1)[..., :w.hot_channels]
        mult = torch.ones(B, H, d, device=device, dtype=torch.float32)
        mult.scatter_(-1, hot, 20.0)
        scale = scale * mult
    return scale


def make_layer(w: Workload, device="cpu", layer: int = 0, seed: int = 0,
               lengths: list | None = None) -> LayerInputs:
    """Draw one layer's K, V (all S_max tokens) and the decode query q."""
    B, H, Hq, d = w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim
    lengths = lengths if lengths is not None else sequence_lengths(w, seed)
    S = max(lengths)
    dt = w.torch_dtype
    g = _gen(device, w.name, seed, layer, "kv")
    cs = channel_scales(w, device, layer, seed)
    k = torch.randn(B, H, S, d, generator=g, device=device, dtype=torch.float32)
    k.mul_(cs[:, :, None, :])
    k = k.to(dt)
    v = torch.randn(B, H, S, d, generator=g, device=device, dtype=torch.float32)
    hot_p = 0.0
    if w.value_model == "outlier":
        n_hot = int(round(w.hot_token_frac * S))
        r = torch.rand(B, H, S, generator=g, device=device)
        hot = torch.argsort(r, dim=-1)[..., :n_hot]
        mult = torch.ones(B, H, S, device=device, dtype=torch.float32)
        mult.scatter_(-1, hot, 15.0)
        v.mul_(mult[..., None])
        hot_p = w.hot_token_frac
    v = v.to(dt)
    q = torch.randn(B, Hq, d, generator=g, device=device, dtype=torch.float32).to(dt)
    return LayerInputs(k, v, q, list(lengths), cs, hot_p)


def new_tokens(w: Workload, inp: LayerInputs, n: int, device="cpu", seed: int = 0, step: int = 0):
    """n further decode tokens per sequence from the same value model:
    k_new, v_new [B][H_kv][n][d] in the input dtype, and a fresh query."""
    B, H, Hq, d = w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim
    g = _gen(device, w.name, seed, step, "step")
    k = torch.randn(B, H, n, d, generator=g, device=device, dtype=torch.float32)
    k.mul_(inp.k_channel_scale.to(device)[:, :, None, :])
    v = torch.randn(B, H, n, d, generator=g, device=device, dtype=torch.float32)
    if inp.v_hot_prob > 0:
        hot = torch.rand(B, H, n, generator=g, device=device) < inp.v_hot_prob
        v = torch.where(hot[..., None], v * 15.0, v)
    q = torch.randn(B, Hq, d, generator=g, device=device, dtype=torch.float32)
    dt = w.torch_dtype
    return k.to(dt), v.to(dt), q.to(dt)


def random_page_table(w: Workload, lengths: list, extra_tokens: int = 0, seed: int = 0):
    """A random permutation of physical pages for the blocks of every sequence.

    Every sequence gets pages for ceil((S_b + extra_tokens)/G) blocks, so it can
    grow by extra_tokens decode steps. Returns (table [B][max_blocks] int32 with
    -1 for unused entries, num_pages). One page holds one G-token block of every
    kv head.
    """
    G = w.k_group
    counts = [math.ceil((s + extra_tokens) / G) for s in lengths]
    max_blocks = max(counts)
    num_pages = sum(counts)
    g = _gen("cpu", w.name, seed, "pages")
    perm = torch.randperm(num_pages, generator=g)
    table = torch.full((w.batch, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b, nb in enumerate(counts):
        table[b, :nb] = perm[off:off + nb].to(torch.int32)
        off += nb
    return table, num_pages
