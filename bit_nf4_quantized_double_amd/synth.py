"""Seeded synthetic inputs and the layer shapes they are drawn for.

This module holds random draws and shapes only -- none of the method's
arithmetic -- so both the CPU oracle (in tests) and the HIP path consume the
very same bits.

Distributions: W ~ N(0, 0.02^2) fp32 (roughly normal pretrained weights,
which is what NF4 is built for); X, dY ~ N(0, 1); A ~ N(0, 1/K);
B ~ N(0, 0.01^2).  X, A, B, dY are rounded to bf16 (round to nearest even,
by torch's CPU conversion) and returned as uint16 bit patterns.

Seeds: the 256x256 single-linear case uses ``default_rng(0)``; every other
linear ``i`` of workload ``w`` uses ``default_rng([WORKLOAD_ID[w], i])``.
Draw order is always W, X, A, B, dY.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Linear:
    name: str
    k_in: int
    n_out: int


# Decoder-layer linears of the model sizes the pages discuss (3B with a
# 3,072 width, 8 KV heads and an 8,192 MLP; a 6.74e9-parameter 7B; an 8B;
# 70B bandwidth-bound shapes).
LAYERS = {
    "cfg1": [Linear("w", 256, 256)],
    "3b": [Linear("q", 3072, 3072), Linear("k", 3072, 1024), Linear("v", 3072, 1024),
           Linear("o", 3072, 3072), Linear("gate", 3072, 8192), Linear("up", 3072, 8192),
           Linear("down", 8192, 3072)],
    "7b": [Linear("q", 4096, 4096), Linear("k", 4096, 4096), Linear("v", 4096, 4096),
           Linear("o", 4096, 4096), Linear("gate", 4096, 11008), Linear("up", 4096, 11008),
           Linear("down", 11008, 4096)],
    "8b": [Linear("q", 4096, 4096), Linear("k", 4096, 1024), Linear("v", 4096, 1024),
           Linear("o", 4096, 4096), Linear("gate", 4096, 14336), Linear("up", 4096, 14336),
           Linear("down", 14336, 4096)],
    "70b": [Linear("gate", 8192, 28672), Linear("down", 28672, 8192)],
}
TOKENS = {"cfg1": 16, "3b": 2048, "7b": 2048, "8b": 8192, "70b": 16}
RANK = {"cfg1": 8, "3b": 16, "7b": 16, "8b": 16, "70b": 16}
ALPHA = {"cfg1": 16.0, "3b": 32.0, "7b": 32.0, "8b": 32.0, "70b": 32.0}
WORKLOAD_ID = {"cfg1": 0, "3b": 1, "7b": 2, "8b": 3, "70b": 4}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (RNE, torch CPU) as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 (RNE, torch CPU) as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rng_for(workload: str, linear_index: int) -> np.random.Generator:
    if workload == "cfg1":
        return np.random.default_rng(0)
    return np.random.default_rng([WORKLOAD_ID[workload], linear_index])


def draw(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def linear_inputs(n_out: int, k_in: int, m: int, r: int, rng: np.random.Generator,
                  with_grad: bool = True, dtype: str = "bf16") -> dict:
    """One linear's inputs: W fp32 [N, K]; X [M, K], A [r, K], B [N, r],
    dY [M, N] as bf16 bits (dtype="f16": fp16 bits, same draws)."""
    to16 = to_f16_bits if dtype == "f16" else to_bf16_bits
    W = draw(rng, (n_out, k_in), 0.02)
    X = to16(draw(rng, (m, k_in), 1.0))
    A = to16(draw(rng, (r, k_in), float(1.0 / np.sqrt(k_in))))
    B = to16(draw(rng, (n_out, r), 0.01))
    out = {"W": W, "X": X, "A": A, "B": B}
    if with_grad:
        out["dY"] = to16(draw(rng, (m, n_out), 1.0))
    return out


def workload_linear(workload: str, index: int, m: int | None = None,
                    with_grad: bool = True, dtype: str = "bf16") -> dict:
    lin = LAYERS[workload][index]
    mm = TOKENS[workload] if m is None else m
    d = linear_inputs(lin.n_out, lin.k_in, mm, RANK[workload], rng_for(workload, index),
                      with_grad=with_grad, dtype=dtype)
    d.update(name=lin.name, n_out=lin.n_out, k_in=lin.k_in, m=mm,
             r=RANK[workload], alpha=ALPHA[workload])
    return d

