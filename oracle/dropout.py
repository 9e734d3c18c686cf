"""LoRA dropout on the adapter input -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

The pages' adapter configurations set ``lora_dropout = 0.05`` ([P1] "A
complete run on a 12 GB-class GPU"; [P5] "Walking through the tooling") but
do not define it.  Reading taken here: the standard inverted dropout of the
adapter's input, as the PEFT ``LoraConfig`` they pass it to applies it --
x is dropped before A, the frozen path W x sees the undropped x:

    Xd = (mask * X) / (1 - p)             mask[m, k] in {0, 1}
    U  = Xd A^T
    Y  = X W^T + s U B^T,                  s = alpha / r
    V  = dY B
    dX = dY W + s (V A) * mask / (1 - p)   (the adapter path's gradient
                                            passes back through the mask)
    dA = s V^T Xd
    dB = s dY^T U

The mask is a function of (seed, element position) only, so the backward
regenerates it from the seed instead of storing it.  Element (m, k) of the
[M, K] input has flat index e = m K + k; the generator is Philox4x32-10
(Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
3", SC'11), a counter-based generator: counter (lo32(e >> 2), hi32(e >> 2),
0, 0), key (lo32(seed), hi32(seed)); u = output word (e & 3); the element is
kept iff u >= floor(p * 2^32).  p = 0 keeps everything.

Pinned by: the generator's published known-answer vectors; the drop rate;
p = 0 equals the plain layer exactly; central finite differences of
<dY, Y> with the mask held fixed; the seed average of the dropped adapter
term converging to the undropped one (inverted scaling is unbiased).
"""

from __future__ import annotations

import math

import numpy as np

from .qlora_linear import _f64, lora_scale

# Philox4x32 round multipliers and key increments (Salmon et al., SC'11).
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_LO = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of 32-bit counter words.

    Each round multiplies words 0 and 2 by the round constants into 64-bit
    products, and the new state is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
    hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key is bumped by (W0, W1) between
    rounds.  Returns four uint32 arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _LO for c in (c0, c1, c2, c3))
    k0 &= 0xFFFFFFFF
    k1 &= 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = _M0 * c0  # < 2^64: exact in uint64
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _LO
        hi1, lo1 = p1 >> np.uint64(32), p1 & _LO
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def dropout_threshold(p: float) -> int:
    """floor(p * 2^32): an element is dropped iff its word is below this."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(math.floor(p * 4294967296.0))  # exact: scaling by 2^32


def dropout_words(n: int, seed: int) -> np.ndarray:
    """The generator word of flat elements 0 .. n-1 (uint32 [n])."""
    e = np.arange(n, dtype=np.uint64)
    q = e >> np.uint64(2)
    nq = int((n + 3) // 4)
    qq = np.arange(nq, dtype=np.uint64)
    zero = np.zeros(nq, dtype=np.uint64)
    out = philox4x32_10(qq & _LO, qq >> np.uint64(32), zero, zero, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    words = np.stack(out, axis=1)  # [nq, 4]
    return words[q.astype(np.int64), (e & np.uint64(3)).astype(np.int64)]


def dropout_mask(M: int, K: int, p: float, seed: int) -> np.ndarray:
    """bool [M, K]: True where element (m, k) of the adapter input is kept."""
    thr = dropout_threshold(p)
    if M * K == 0:
        return np.ones((M, K), dtype=bool)
    return (dropout_words(M * K, seed).astype(np.uint64) >= np.uint64(thr)).reshape(M, K)


def _dropped(X, mask, p):
    return _f64(X) * mask / (1.0 - p)


def linear_fwd_dropout(W_bf, X, A, B, alpha: float, r: int, mask, p: float):
    """Returns (Y fp64 [M, N], U fp64 [M, r]) with the adapter input dropped."""
    W = _f64(W_bf)
    Xf, Af, Bf = _f64(X), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    U = _dropped(X, mask, p) @ Af.T
    Y = Xf @ W.T + s * (U @ Bf.T)
    return Y, U


def linear_bwd_dropout(W_bf, X, dY, A, B, alpha: float, r: int, mask, p: float):
    """Returns (dX fp64 [M, K], dA fp64 [r, K], dB fp64 [N, r])."""
    W = _f64(W_bf)
    dYf, Af, Bf = _f64(dY), _f64(A), _f64(B)
    s = lora_scale(alpha, r)
    Xd = _dropped(X, mask, p)
    U = Xd @ Af.T
    V = dYf @ Bf
    dX = dYf @ W + s * (V @ Af) * mask / (1.0 - p)
    dA = s * (V.T @ Xd)
    dB = s * (dYf.T @ U)
    return dX, dA, dB
