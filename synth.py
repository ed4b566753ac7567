"""Seeded synthetic workloads shared by the tests, the oracle timing and bench.py.

This module draws random inputs and nothing else: it holds none of the
encoding, attention or search arithmetic.  Every tensor it returns is a
deterministic function of its arguments (torch Philox/mt19937 generators
seeded explicitly), so the CPU oracle and the GPU library see the same values.

Workload recipes (sizes are the defaults; tests pass smaller ones):

* tiny:    1 head, d=128, 512 keys and 512 values, fp32 N(0,1); 8 fp32 N(0,1)
           queries; a 128x128 N(0,1) QJL projection.  Seed 0, draw order
           K, V, Q, S.
* kv_block (the "Qwen2.5-7B-shaped" key/value recipe): keys N(0,1) in which
           round(0.06*d) channels per head (a seeded permutation, fixed per
           head) are scaled by 30, then every key is multiplied by one global
           factor so that E||k||^2 = 170^2; values N(0, 0.25), i.e. sigma 0.5.
           Real-model statistics (key norm ~172, value norm ~3, 4-6% outlier
           channels in middle layers) are described on the TurboQuant PyTorch
           write-up (idea.jsleekr.com, "핵심 발견 2" and "핵심 발견 4"); no
           model or dataset is available, so this recipe stands in for them.
* decode:  batch 16 sequences, 4 kv heads x 32768 tokens each drawn with
           kv_block (seed 1000+b), queries fp16 N(0,1) [16][28][128].
* search:  2^20 unit-norm Gaussian directions at d=256, 1024 unit queries,
           a 256x256 N(0,1) projection.
* long:    8 kv heads x 2^20 tokens, bf16, kv_block recipe, generated in
           4096-token chunks (seed 5000+chunk); queries bf16 N(0,1) [64][128].
"""
from __future__ import annotations

import math

import torch

# Seeds of the workloads (one place, so tests and bench agree).
SEED_TINY = 0
SEED_ENCODE = 1
SEED_DECODE_BASE = 1000
SEED_DECODE_Q = 2000
SEED_SEARCH = 3000
SEED_LONG_BASE = 5000
SEED_LONG_Q = 6000
SEED_QJL_S = 7000


def _gen(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, device="cpu", dtype=torch.float32, std: float = 1.0):
    """i.i.d. N(0, std^2) drawn in fp32 and cast to ``dtype``."""
    g = _gen(seed, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def qjl_projection(m: int, d: int, seed: int = SEED_QJL_S, device="cpu"):
    """Gaussian projection S [m][d], i.i.d. N(0,1) fp32 (the QJL sketch matrix)."""
    return normal((m, d), seed, device)


def outlier_channels(heads: int, d: int, seed: int, frac: float = 0.06):
    """Per-head outlier channel ids: the first round(frac*d) of a seeded permutation."""
    n_out = int(round(frac * d))
    g = _gen(seed, "cpu")
    return torch.stack([torch.randperm(d, generator=g)[:n_out] for _ in range(heads)])


def kv_block(heads: int, tokens: int, d: int, seed: int, device="cpu",
             dtype=torch.float16, outlier_seed: int | None = None,
             outlier_scale: float = 30.0, key_norm: float = 170.0,
             v_sigma: float = 0.5):
    """Keys and values [heads][tokens][d] with the outlier-channel key recipe.

    ``outlier_seed`` fixes which channels are outliers (defaults to ``seed``);
    chunks of one long sequence pass the same ``outlier_seed`` so the channels
    stay fixed per head across chunks.
    """
    oseed = seed if outlier_seed is None else outlier_seed
    chans = outlier_channels(heads, d, oseed)
    n_out = chans.shape[1]
    alpha = key_norm / math.sqrt((d - n_out) + n_out * outlier_scale ** 2)
    g = _gen(seed, device)
    k = torch.randn(heads, tokens, d, generator=g, device=device, dtype=torch.float32)
    scale = torch.ones(heads, d, dtype=torch.float32)
    for h in range(heads):
        scale[h, chans[h]] = outlier_scale
    k.mul_((scale * alpha).to(device)[:, None, :])
    v = torch.randn(heads, tokens, d, generator=g, device=device, dtype=torch.float32)
    v.mul_(v_sigma)
    return k.to(dtype), v.to(dtype)


def tiny(seed: int = SEED_TINY, n: int = 512, d: int = 128, n_q: int = 8, m: int = 128):
    """The tiny reference workload: K, V [n][d], Q [n_q][d] fp32 N(0,1), S [m][d]."""
    g = _gen(seed, "cpu")
    k = torch.randn(n, d, generator=g)
    v = torch.randn(n, d, generator=g)
    q = torch.randn(n_q, d, generator=g)
    s = torch.randn(m, d, generator=g)
    return k, v, q, s


def decode_cache_inputs(batch: int = 16, kv_heads: int = 4, ctx: int = 32768,
                        d: int = 128, device="cpu", dtype=torch.float16,
                        seed_base: int = SEED_DECODE_BASE):
    """Per-sequence K/V [batch][kv_heads][ctx][d]; sequence b uses seed seed_base+b."""
    ks, vs = [], []
    for b in range(batch):
        k, v = kv_block(kv_heads, ctx, d, seed_base + b, device=device, dtype=dtype)
        ks.append(k)
        vs.append(v)
    return torch.stack(ks), torch.stack(vs)


def decode_queries(batch: int = 16, q_heads: int = 28, d: int = 128, device="cpu",
                   dtype=torch.float16, seed: int = SEED_DECODE_Q):
    return normal((batch, q_heads, d), seed, device, dtype)


def unit_rows(n: int, d: int, seed: int, device="cpu"):
    """n unit-norm Gaussian directions [n][d] fp32."""
    x = normal((n, d), seed, device)
    return x / x.norm(dim=1, keepdim=True)


def search_inputs(n_db: int = 1 << 20, n_q: int = 1024, d: int = 256, m: int = 256,
                  device="cpu", seed: int = SEED_SEARCH):
    db = unit_rows(n_db, d, seed, device)
    q = unit_rows(n_q, d, seed + 1, device)
    s = qjl_projection(m, d, seed + 2, device)
    return db, q, s


def long_chunk(chunk: int, kv_heads: int = 8, tokens: int = 4096, d: int = 128,
               device="cpu", dtype=torch.bfloat16, seed_base: int = SEED_LONG_BASE):
    """Chunk ``chunk`` of the long-context sequence: K/V [kv_heads][tokens][d]."""
    return kv_block(kv_heads, tokens, d, seed_base + chunk, device=device, dtype=dtype,
                    outlier_seed=seed_base)


def long_queries(q_heads: int = 64, d: int = 128, device="cpu", dtype=torch.bfloat16,
                 seed: int = SEED_LONG_Q):
    return normal((q_heads, d), seed, device, dtype)
