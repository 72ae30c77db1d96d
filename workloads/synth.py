"""Workload definitions and seeded generators.

Shapes follow the DMuon pages' models:
* "Quick Start", model.py: TinyMLP with gate/up ``nn.Linear(d, ff)`` (weight
  ff x d) and down ``nn.Linear(ff, d)`` (weight d x ff), 4 layers.
* "Tensor Parallelism", the Llama-style q/k/v/o and gate/up/down projection
  names; sizes are the usual 8B (d=4096, kv=1024, ff=14336) and 70B MLP
  (d=8192, ff=28672) shapes.

Recipes (the second argument of N(.,.) is a standard deviation):
* ``gauss``       iid N(0, 1)
* ``gauss_lognormal``  iid N(0, 1) times one exp(N(0, 1)) factor per matrix
* ``lowrank``     L + E: L = U diag(s) V^T of rank 64 with Haar U, V and
                  s_k proportional to 1/k, scaled so L has unit-rms entries;
                  E iid N(0, 1e-2).  Fresh every step.
* ``powerlaw_t3`` L + E: full-rank L = U diag(k^-1.5) V^T with Haar U, V drawn
                  once per matrix, scaled to unit-rms entries; E is
                  Student-t(3) scaled to std 1e-2, fresh every step.
* params          iid N(0, 0.02)

numpy generators (``*_np``) are portable (PCG64 via SeedSequence) and are the
ones parity tests use; the torch generators (``*_torch``) follow the same
recipes on the GPU for full-size benchmark inputs whose fp64 reference would
be too slow to build on the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Seed streams: one SeedSequence per (config, step, matrix, stream).
STREAM_GRAD = 0
STREAM_BASIS = 1
STREAM_PARAM = 2
STREAM_SHAPES = 3


def seed_words(cfg_id: int, step: int, idx: int, stream: int):
    return [int(cfg_id), int(step), int(idx), int(stream)]


@dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    shapes: tuple
    grad_dtype: str          # "f32" | "bf16"
    param_dtype: str         # "f32" | "bf16"
    ns_prec: str             # "f32" | "bf16" | "bf16_split" | "auto"
    steps: int
    grad_kind: str
    momentum: float = 0.95
    lr: float = 0.02
    weight_decay: float = 0.0
    ns_steps: int = 5
    nesterov: bool = False
    ns_only: bool = False
    notes: str = field(default="", compare=False)

    @property
    def numel(self) -> int:
        return sum(m * n for m, n in self.shapes)


def _tinymlp(d, ff, layers):
    out = []
    for _ in range(layers):
        out += [(ff, d), (ff, d), (d, ff)]
    return tuple(out)


def _llama8b(layers):
    out = []
    for _ in range(layers):
        out += [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),
                (14336, 4096), (14336, 4096), (4096, 14336)]
    return tuple(out)


def c4_shapes(count: int = 512, cfg_id: int = 4):
    """Sides drawn independently, log-uniform on [32, 1024], rounded to a
    multiple of 32 and clipped to [32, 1024]."""
    rng = np.random.default_rng(seed_words(cfg_id, 0, 0, STREAM_SHAPES))
    lo, hi = math.log(32.0), math.log(1024.0)
    out = []
    for _ in range(count):
        m, n = np.exp(rng.uniform(lo, hi, size=2))
        m = 32 * int(np.clip(np.rint(m / 32.0), 1, 32))
        n = 32 * int(np.clip(np.rint(n / 32.0), 1, 32))
        out.append((m, n))
    return tuple(out)


CONFIGS = {
    1: Config(1, "tinymlp_d256_ff1024_fp32", _tinymlp(256, 1024, 1),
              "f32", "f32", "f32", 1, "gauss"),
    2: Config(2, "tinymlp_d512_ff2048_x4", _tinymlp(512, 2048, 4),
              "f32", "f32", "auto", 20, "gauss"),
    3: Config(3, "llama8b_proj_x4", _llama8b(4),
              "bf16", "bf16", "auto", 10, "lowrank"),
    4: Config(4, "packed_small_512", c4_shapes(),
              "bf16", "bf16", "auto", 1, "gauss_lognormal", ns_only=True),
    5: Config(5, "llama70b_mlp", ((28672, 8192),) * 4 + ((8192, 28672),) * 2,
              "bf16", "bf16", "auto", 3, "powerlaw_t3", nesterov=True),
}


# ---------------------------------------------------------------- numpy ---

def _haar_np(rng, rows, cols):
    q, r = np.linalg.qr(rng.standard_normal((rows, cols)))
    return q * np.sign(np.diag(r))


def _unit_rms(L):
    return L * (math.sqrt(L.size) / np.linalg.norm(L))


def powerlaw_basis_np(m: int, n: int, cfg_id: int, idx: int):
    """Unit-rms full-rank L with a k^-1.5 spectrum for matrix ``idx``: the
    part of every step's power-law gradient that does not change."""
    brng = np.random.default_rng(seed_words(cfg_id, 0, idx, STREAM_BASIS))
    k = min(m, n)
    U = _haar_np(brng, m, k)
    V = _haar_np(brng, n, k)
    s = np.arange(1, k + 1, dtype=np.float64) ** -1.5
    return _unit_rms((U * s) @ V.T)


def grad_np(kind: str, m: int, n: int, cfg_id: int, step: int, idx: int, basis=None):
    """float32 gradient for matrix ``idx`` of config ``cfg_id`` at ``step``.
    ``basis``: :func:`powerlaw_basis_np` of the same matrix, if the caller
    keeps it across steps (power-law kind only; recomputed when omitted)."""
    rng = np.random.default_rng(seed_words(cfg_id, step, idx, STREAM_GRAD))
    if kind == "gauss":
        g = rng.standard_normal((m, n))
    elif kind == "gauss_lognormal":
        scale = math.exp(rng.standard_normal())
        g = rng.standard_normal((m, n)) * scale
    elif kind == "lowrank":
        r = min(64, m, n)
        U = _haar_np(rng, m, r)
        V = _haar_np(rng, n, r)
        s = 1.0 / np.arange(1, r + 1)
        L = _unit_rms((U * s) @ V.T)
        g = L + 1e-2 * rng.standard_normal((m, n))
    elif kind == "powerlaw_t3":
        L = powerlaw_basis_np(m, n, cfg_id, idx) if basis is None else basis
        g = L + (1e-2 / math.sqrt(3.0)) * rng.standard_t(3, size=(m, n))
    else:
        raise ValueError(f"unknown gradient kind {kind!r}")
    return g.astype(np.float32)


def param_np(m: int, n: int, cfg_id: int, idx: int):
    rng = np.random.default_rng(seed_words(cfg_id, 0, idx, STREAM_PARAM))
    return (0.02 * rng.standard_normal((m, n))).astype(np.float32)


# ---------------------------------------------------------------- torch ---

def _torch_gen(device, words):
    import torch
    seed = int(np.random.SeedSequence(words).generate_state(1, np.uint64)[0]
               & np.uint64(0x7FFFFFFFFFFFFFFF))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _haar_torch(gen, rows, cols, device):
    import torch
    a = torch.randn(rows, cols, generator=gen, device=device,
                    dtype=torch.float32)
    q, r = torch.linalg.qr(a)
    return q * torch.sign(torch.diagonal(r)).unsqueeze(0)


def powerlaw_basis_torch(m, n, cfg_id, idx, device):
    """Unit-rms full-rank L with a k^-1.5 spectrum (computed once per
    matrix and reused by every step)."""
    import torch
    gen = _torch_gen(device, seed_words(cfg_id, 0, idx, STREAM_BASIS))
    k = min(m, n)
    U = _haar_torch(gen, m, k, device)
    V = _haar_torch(gen, n, k, device)
    s = torch.arange(1, k + 1, device=device, dtype=torch.float32) ** -1.5
    L = (U * s) @ V.T.contiguous()
    return L * (math.sqrt(L.numel()) / torch.linalg.norm(L))


def grad_torch(kind, m, n, cfg_id, step, idx, device, dtype, basis=None):
    """Same recipes as :func:`grad_np` drawn with torch's generator on
    ``device`` (different random stream, same distribution)."""
    import torch
    gen = _torch_gen(device, seed_words(cfg_id, step, idx, STREAM_GRAD))
    f32 = torch.float32
    if kind == "gauss":
        g = torch.randn(m, n, generator=gen, device=device, dtype=f32)
    elif kind == "gauss_lognormal":
        scale = torch.exp(torch.randn(1, generator=gen, device=device,
                                      dtype=f32))
        g = torch.randn(m, n, generator=gen, device=device, dtype=f32) * scale
    elif kind == "lowrank":
        r = min(64, m, n)
        U = _haar_torch(gen, m, r, device)
        V = _haar_torch(gen, n, r, device)
        s = 1.0 / torch.arange(1, r + 1, device=device, dtype=f32)
        L = (U * s) @ V.T.contiguous()
        L = L * (math.sqrt(L.numel()) / torch.linalg.norm(L))
        g = L + 1e-2 * torch.randn(m, n, generator=gen, device=device,
                                   dtype=f32)
    elif kind == "powerlaw_t3":
        if basis is None:
            basis = powerlaw_basis_torch(m, n, cfg_id, idx, device)
        # Student-t(3) = N(0,1) / sqrt(chi2_3 / 3)
        z = torch.randn(m, n, generator=gen, device=device, dtype=f32)
        chi = torch.zeros(m, n, device=device, dtype=f32)
        for _ in range(3):
            chi += torch.randn(m, n, generator=gen, device=device,
                               dtype=f32) ** 2
        t3 = z / torch.sqrt(chi / 3.0)
        g = basis + (1e-2 / math.sqrt(3.0)) * t3
    else:
        raise ValueError(f"unknown gradient kind {kind!r}")
    return g.to(dtype)


def param_torch(m, n, cfg_id, idx, device, dtype):
    import torch
    gen = _torch_gen(device, seed_words(cfg_id, 0, idx, STREAM_PARAM))
    return (0.02 * torch.randn(m, n, generator=gen, device=device,
                               dtype=torch.float32)).to(dtype)


# ------------------------------------------------ element-wise companions --

@dataclass(frozen=True)
class OpConfig:
    """Workload of an element-wise companion of the Muon step."""
    name: str
    shapes: tuple            # tensor shapes
    dtype: str               # param / gradient dtype
    buckets: tuple = ()      # clipping: bucket of each tensor
    max_norm: float = 0.0    # clipping: chosen below the gradients' norm
    transposed: tuple = ()   # Gram NS on shards: the full matrix's orientation
    notes: str = field(default="", compare=False)


# The workloads by name.
BY_NAME = {c.name: c for c in CONFIGS.values()}


OP_CONFIGS = {
    # the 28 projection gradients of the Llama-8B batch, one bucket per layer
    # (bench.py lowers max_norm from call to call so that every call clips)
    "clip": OpConfig("llama8b_proj_grads_4_buckets", _llama8b(4), "bf16",
                     buckets=tuple(i // 7 for i in range(28)), max_norm=100.0),
    # AdamW's share of a Llama-8B: token embedding and LM head (vocab 128256)
    "adamw": OpConfig("llama8b_embed_lmhead", ((128256, 4096),) * 2, "bf16"),
    # One rank's blocks of a Llama-8B tensor-parallel group of 8, for the
    # matrices whose Megatron shard is a column block of the oriented matrix:
    # o (4096 x 4096, split along its input side), down (4096 x 14336, same),
    # gate and up (14336 x 4096, split along their output side, transposed).
    "gram_local": OpConfig("llama8b_o_mlp_tp8_rank_blocks",
                           ((4096, 512), (4096, 1792), (1792, 4096), (1792, 4096)) * 4,
                           "bf16", transposed=(0, 0, 1, 1) * 4),
}
