"""Seeded synthetic inputs for the block-scaled FP8 linear-layer path.

This module draws tensors only; it holds none of the method's arithmetic
(no scaling, rounding into FP8, or GEMM).  Both the HIP path and the CPU
oracle are fed from the same arrays, so they read identical bits.

Recipe (numpy ``Generator(PCG64(seed))``, draws in the order listed):

* fp32 values are ``standard_normal * std``; the second parameter of every
  N(mean, std) below is the standard deviation.
* "1% outlier channels x50": ``round(0.01*C)`` channels chosen with
  ``rng.choice(C, k, replace=False)`` and multiplied by 50 in fp32, the
  same channels for every token.
* bf16 tensors are the fp32 draws rounded to nearest-even on the host and
  stored as raw uint16 bits.
* MoE routing: each token picks 8 distinct experts uniformly without
  replacement; routed rows are ordered stably by (expert, token) and
  ``offsets[e]`` is the first routed row of expert e.

Workloads (Qwen3-family linear-layer shapes):

* tiny      X fp32 [256, 512] ~ N(0,1); W fp32 [384, 512] ~ N(0, 0.02);
            dY fp32 [256, 384] ~ N(0, 1e-3)
* decode    X bf16 [64, 4096] ~ N(0,1) with 41 outlier channels;
            W bf16 [24576, 4096] ~ N(0, 0.02) (fused gate+up, 2 x 12288)
* train     X bf16 [8192, 12288] ~ N(0,1) with 123 outlier channels;
            W bf16 [4096, 12288] ~ N(0, 0.02); dY bf16 [8192, 4096] ~ N(0, 1e-3)
* mx        decode's X and W from the same seed, then dY bf16 [64, 24576]
            ~ N(0, 1e-3)
* moe       4096 tokens, hidden 2048, 128 experts, intermediate 768, top-8;
            X_tok bf16 [4096, 2048] ~ N(0,1); W_gu bf16 [128, 1536, 2048]
            ~ N(0, 0.02); W_d bf16 [128, 2048, 768] ~ N(0, 0.02); down-proj
            input A bf16 [32768, 768] ~ N(0,1); dH bf16 [32768, 1536] and
            dY_d bf16 [32768, 2048] ~ N(0, 1e-3)
"""
from __future__ import annotations

import numpy as np


def rng_for(seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits.
    Inputs are finite by construction."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(rng: np.random.Generator, shape, std: float, chunk_rows: int = 1024) -> np.ndarray:
    """fp32 N(0, std) draws, generated in row chunks to bound peak memory;
    the stream of draws is the same as one call for the whole shape."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = rng.standard_normal(size=(r1 - r0, flat.shape[1]), dtype=np.float32)
    if std != 1.0:
        np.multiply(out, np.float32(std), out=out)
    return out


def add_outlier_channels(rng: np.random.Generator, x: np.ndarray, frac: float = 0.01,
                         factor: float = 50.0) -> np.ndarray:
    C = x.shape[1]
    k = int(round(frac * C))
    ch = rng.choice(C, k, replace=False)
    x[:, ch] *= np.float32(factor)
    return ch


def normal_bf16(rng, shape, std):
    return f32_to_bf16_bits(normal(rng, shape, std))


# ------------------------------------------------------------ workloads
def tiny(seed: int = 0) -> dict:
    rng = rng_for(seed)
    X = normal(rng, (256, 512), 1.0)
    W = normal(rng, (384, 512), 0.02)
    dY = normal(rng, (256, 384), 1e-3)
    return {"name": "tiny", "X": X, "W": W, "dY": dY, "N": 256, "C": 512, "D": 384,
            "dtype": "f32"}


def decode(seed: int = 0) -> dict:
    rng = rng_for(seed)
    X = normal(rng, (64, 4096), 1.0)
    ch = add_outlier_channels(rng, X)
    W = normal(rng, (24576, 4096), 0.02)
    return {"name": "decode", "X": f32_to_bf16_bits(X), "W": f32_to_bf16_bits(W),
            "outlier_channels": ch, "N": 64, "C": 4096, "D": 24576, "dtype": "bf16"}


def train(seed: int = 0, rows: int | None = None) -> dict:
    """Training-step down_proj shapes.  ``rows`` draws a smaller token count
    with the same recipe (its own stream, not a slice of the full one)."""
    rng = rng_for(seed)
    N = 8192 if rows is None else rows
    X = normal(rng, (N, 12288), 1.0)
    ch = add_outlier_channels(rng, X)
    Xb = f32_to_bf16_bits(X)
    del X
    W = normal_bf16(rng, (4096, 12288), 0.02)
    dY = normal_bf16(rng, (N, 4096), 1e-3)
    return {"name": "train", "X": Xb, "W": W, "dY": dY, "outlier_channels": ch,
            "N": N, "C": 12288, "D": 4096, "dtype": "bf16"}


def mx(seed: int = 0) -> dict:
    w = decode(seed)
    rng = rng_for(seed)
    # re-draw the decode stream to reach the same generator state, then dY
    Xr = normal(rng, (64, 4096), 1.0)
    add_outlier_channels(rng, Xr)
    normal(rng, (24576, 4096), 0.02)
    dY = normal_bf16(rng, (64, 24576), 1e-3)
    w.update({"name": "mx", "dY": dY})
    return w


def moe_routing(rng: np.random.Generator, tokens: int, experts: int, topk: int):
    """Each token draws `topk` distinct experts uniformly.  Returns
    (expert_of_row, token_of_row, offsets) for rows ordered by (expert, token)."""
    choice = np.empty((tokens, topk), dtype=np.int64)
    for t in range(tokens):
        choice[t] = rng.choice(experts, topk, replace=False)
    expert = choice.reshape(-1)
    token = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    order = np.lexsort((token, expert))
    expert_sorted = expert[order]
    counts = np.bincount(expert_sorted, minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return expert_sorted, token[order], offsets


def moe(seed: int = 0, tokens: int = 4096, hidden: int = 2048, experts: int = 128,
        inter: int = 768, topk: int = 8) -> dict:
    rng = rng_for(seed)
    expert_of_row, token_of_row, offsets = moe_routing(rng, tokens, experts, topk)
    X_tok = normal(rng, (tokens, hidden), 1.0)
    X_perm = f32_to_bf16_bits(X_tok)[token_of_row]
    W_gu = normal_bf16(rng, (experts * 2 * inter, hidden), 0.02).reshape(experts, 2 * inter, hidden)
    W_d = normal_bf16(rng, (experts * hidden, inter), 0.02).reshape(experts, hidden, inter)
    R = tokens * topk
    A = normal_bf16(rng, (R, inter), 1.0)
    dH = normal_bf16(rng, (R, 2 * inter), 1e-3)
    dYd = normal_bf16(rng, (R, hidden), 1e-3)
    return {"name": "moe", "X_perm": X_perm, "W_gu": W_gu, "W_d": W_d, "A": A, "dH": dH,
            "dY_d": dYd, "offsets": offsets, "expert_of_row": expert_of_row,
            "token_of_row": token_of_row, "tokens": tokens, "hidden": hidden,
            "experts": experts, "inter": inter, "topk": topk, "dtype": "bf16"}
