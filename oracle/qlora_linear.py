"""Forward and backward of the QLoRA linear -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

The layer keeps a frozen weight W, dequantized to bf16, and adds a rank-r
adapter scaled by alpha / r:  y = W x + (alpha / r) B A x  ([P1] "The
mechanism in brief").  In row-major batch form with X [M, K], W [N, K],
A [r, K], B [N, r]:

    U  = X A^T                          (M x r)
    Y  = X W^T + s U B^T,  s = alpha / r

Backward returns gradients for the activations and for A and B but never for
W, which is frozen ([P1] "The mechanism in brief"; [P4] "The idea in one
line"):

    V  = dY B                           (M x r)
    dX = dY W + s V A
    dA = s V^T X
    dB = s dY^T U

This is the plain definition: dense fp64 products on exact upcasts of the
bf16 inputs and of the bf16 dequantized weight.  s is rounded to fp32 first
(the kernels' scalar type).  No dropout, no bias (the pages' adapters use
``bias="none"``; [P5] "Walking through the tooling").

Pinned by: B = 0 reduces Y to the plain product X W^T (checked against
exactly-rounded per-element sums); Y equals X times the merged weight
W + s B A ([P5] "Walking through the tooling" gives the merge); doubling alpha
doubles the adapter term; central finite differences of <dY, Y> give dX, dA
and dB.
"""

from __future__ import annotations

import numpy as np

from .nf4_dq import f64_from_bf16_bits


def lora_scale(alpha: float, r: int) -> float:
    """s = fp32(alpha / r) as a Python float.

    Rank 0 means there is no adapter at all, so its (empty) term contributes
    nothing; s is then 0 rather than alpha / 0.
    """
    if r == 0:
        return 0.0
    return float(np.float32(alpha) / np.float32(r))


def _f64(bits_or_float):
    a = np.asarray(bits_or_float)
    if a.dtype == np.uint16:
        return f64_from_bf16_bits(a)
    return a.astype(np.float64)


def linear_fwd(W_bf, X, A, B, alpha: float, r: int):
    """Returns (Y fp64 [M, N], U fp64 [M, r]).

    W_bf, X, A, B are bf16 bit arrays (uint16) or float arrays.
    """
    W = _f64(W_bf)
    Xf, Af, Bf = _f64(X), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    U = Xf @ Af.T
    Y = Xf @ W.T + s * (U @ Bf.T)
    return Y, U


def adapter_grads(X, dY, A, B, alpha: float, r: int):
    """The adapter's gradients alone: (dA fp64 [r, K], dB fp64 [N, r]).

    dA = s V^T X and dB = s dY^T U with V = dY B and U = X A^T; they need no
    weight, so a test can take them over every token of a large layer
    without forming dX.  ``linear_bwd`` returns exactly these.
    """
    Xf, dYf, Af, Bf = _f64(X), _f64(dY), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    U = Xf @ Af.T
    V = dYf @ Bf
    dA = s * (V.T @ Xf)
    dB = s * (dYf.T @ U)
    return dA, dB


def linear_bwd(W_bf, X, dY, A, B, alpha: float, r: int):
    """Returns (dX fp64 [M, K], dA fp64 [r, K], dB fp64 [N, r])."""
    W = _f64(W_bf)
    dYf, Af, Bf = _f64(dY), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    V = dYf @ Bf
    dX = dYf @ W + s * (V @ Af)
    dA, dB = adapter_grads(X, dY, A, B, alpha, r)
    return dX, dA, dB
