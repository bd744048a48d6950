"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module holds no arithmetic of the quantized-linear method: it only draws random
numbers and rounds activations to their storage dtype.  Every array is drawn from
``numpy.random.default_rng(seed)`` (PCG64), so a seed fully determines a workload.

Workload shapes stand in for the layer shapes the pages quote (real weights and
datasets are not used):

* ``QWEN3_0_6B_DECODE``: the Qwen3-0.6B projection set (hidden 1024, intermediate 3072,
  28 layers, vocabulary 151936) that the tinygpt PRD quantizes to 4-bit and 8-bit.
* ``PREFILL_9B_LAYER``: one layer of a 9B-class model (hidden 4096, intermediate 12288).
* ``EXPERTS_32x5760x2880``: a 32-expert stack of 5760x2880 weights with top-4 routing.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng",
    "weights_f32",
    "acts_bits",
    "mxfp4_codes_scales",
    "q8_0_random_blocks",
    "kquant_random_blocks",
    "topk_ids",
    "seed_for",
    "QWEN3_0_6B_LAYER",
    "QWEN3_0_6B_DECODE",
    "PREFILL_9B_LAYER",
    "EXPERTS_32x5760x2880",
]

# (name, k inputs, n outputs) of one Qwen3-0.6B decoder layer.
QWEN3_0_6B_LAYER = [
    ("q", 1024, 2048),
    ("k", 1024, 1024),
    ("v", 1024, 1024),
    ("o", 2048, 1024),
    ("gate", 1024, 3072),
    ("up", 1024, 3072),
    ("down", 3072, 1024),
]
# 28 layers then the lm_head: 197 projections.
QWEN3_0_6B_DECODE = [(f"l{li}.{nm}", k, n) for li in range(28) for (nm, k, n) in QWEN3_0_6B_LAYER] + [
    ("lm_head", 1024, 151936)
]
# One 9B-class layer at prefill: (name, k, n); tokens M = 2048.
PREFILL_9B_LAYER = [
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 12288),
    ("up", 4096, 12288),
    ("down", 12288, 4096),
]
# Routed experts: e experts of [n, k], tokens x top.
EXPERTS_32x5760x2880 = dict(e=32, n=5760, k=2880, tokens=512, top=4)


def seed_for(cfg: int, layer: int = 0, proj: int = 0, part: int = 0) -> int:
    """Seed recipe: 1_000_000*cfg + 1000*layer + 10*proj + part (0: W, 1: x, 2..: other)."""
    return 1_000_000 * cfg + 1000 * layer + 10 * proj + part


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def weights_f32(seed: int, n: int, k: int, std: float = 0.02) -> np.ndarray:
    """fp32 weights [n, k] ~ N(0, std^2)."""
    return (rng(seed).standard_normal((n, k), dtype=np.float32) * np.float32(std)).astype(np.float32)


def acts_bits(seed: int, m: int, k: int, dtype: str, std: float = 1.0) -> np.ndarray:
    """Activations [m, k] ~ N(0, std^2) drawn in fp32 and stored as fp16/bf16 bit patterns (uint16).

    The fp32 -> 16-bit storage rounding is torch's CPU conversion (round to nearest even).
    """
    import torch

    a = rng(seed).standard_normal((m, k), dtype=np.float32) * np.float32(std)
    t = torch.from_numpy(a)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f16":
        t = t.to(torch.float16)
    else:
        raise ValueError(dtype)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def mxfp4_codes_scales(seed: int, e: int, n: int, k: int, smin: int = 118, smax: int = 130):
    """MXFP4 parts with scales apart: uniform code bytes [e, n, k/2] and uniform E8M0 scale
    bytes in [smin, smax] of shape [e, n, k/32]."""
    g = rng(seed)
    codes = g.integers(0, 256, size=(e, n, k // 2), dtype=np.uint8)
    scales = g.integers(smin, smax + 1, size=(e, n, k // 32), dtype=np.uint8)
    return codes, scales


def q8_0_random_blocks(seed: int, e: int, n: int, k: int) -> np.ndarray:
    """Structurally valid Q8_0 blocks [e, n, k/32*34] with random contents: a little-endian
    fp16 scale d drawn log-uniform in [2^-14, 2^-9] (the range amax/127 takes for N(0, 0.02)
    weights) followed by 32 int8 quants uniform in [-127, 127]."""
    g = rng(seed)
    nb = k // 32
    d = np.exp2(g.uniform(-14.0, -9.0, size=(e, n, nb))).astype(np.float16)
    q = g.integers(-127, 128, size=(e, n, nb, 32), dtype=np.int8)
    blocks = np.empty((e, n, nb, 34), dtype=np.uint8)
    blocks[..., 0:2] = d.view(np.uint8).reshape(e, n, nb, 2)
    blocks[..., 2:] = q.view(np.uint8)
    return blocks.reshape(e, n, nb * 34)


def kquant_random_blocks(seed: int, rows: int, k: int, fmt: str) -> np.ndarray:
    """Structurally valid Q4_K ('q4_k', 144 bytes) or Q6_K ('q6_k', 210 bytes) blocks [rows,
    k/256*bytes] with random contents: every byte uniform, then the fp16 fields set to finite
    values: Q4_K's d and dmin (bytes 0..3) log-uniform in [2^-16, 2^-11] (with 6-bit scales and
    4-bit quants that spans the +-0.05 of N(0, 0.02) weights), Q6_K's d (bytes 208..209)
    log-uniform in [2^-17, 2^-12] (int8 scales, quants - 32 in [-32, 31])."""
    g = rng(seed)
    nbytes = 144 if fmt == "q4_k" else 210
    nb = k // 256
    blocks = g.integers(0, 256, size=(rows, nb, nbytes), dtype=np.uint8)
    if fmt == "q4_k":
        dd = np.exp2(g.uniform(-16.0, -11.0, size=(rows, nb, 2))).astype(np.float16)
        blocks[..., 0:4] = dd.view(np.uint8).reshape(rows, nb, 4)
    else:
        d = np.exp2(g.uniform(-17.0, -12.0, size=(rows, nb))).astype(np.float16)
        blocks[..., 208:210] = d.view(np.uint8).reshape(rows, nb, 2)
    return blocks.reshape(rows, nb * nbytes)


def topk_ids(seed: int, tokens: int, top: int, e: int) -> np.ndarray:
    """int64 ids [tokens, top]: `top` distinct experts per token, uniform without replacement."""
    g = rng(seed)
    keys = g.random((tokens, e))
    return np.argsort(keys, axis=1)[:, :top].astype(np.int64)
