"""Merging the adapter into the frozen weight -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

The pages ship a trained adapter by folding it into a 16-bit copy of the
base and re-quantizing that for serving, and warn that the re-quantized
weight drifts from what was evaluated ([P1] "Shipping: merge, re-quantize,
verify"; [P5] "QLoRA", "Walking through the tooling": at inference
W' = W + scaled B A).

Readings (listed in the design notes):

* The base is the decoded NF4 weight W_bf (bf16): the frozen weight the
  adapter was trained against.
* The merged weight is kept in bf16, the pages' 16-bit compute dtype:
  W_m = RNE_bf16(W_bf + s B A), s = fp32(alpha / r), computed exactly
  (fp64 holds every product of two bf16 values and these short sums) and
  rounded once.
* Re-quantization is the same NF4 + double-quantization codec applied to
  W_m (exactly widened to fp32).
"""

from __future__ import annotations

import numpy as np

from .nf4_dq import dequant, f64_from_bf16_bits, quantize_nf4_dq
from .qlora_linear import lora_scale


def bf16_bits_from_f64(x) -> np.ndarray:
    """Round fp64 values to bf16, round to nearest even, in one step.

    Normal bf16 range only (|x| in [2^-126, 2^128)) or zero; raises
    otherwise.  Pinned against exact rational rounding and against torch's
    conversion for fp32-exact values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    nz = x != 0
    ax = np.abs(x[nz])
    m, e = np.frexp(ax)              # ax = m * 2^e, m in [0.5, 1)
    M = np.rint(m * 256.0)           # 8 significant bits, ties to even
    up = M == 256.0
    M = np.where(up, 128.0, M)
    e = e + up
    exp_field = e - 1 + 127          # value = (M / 128) * 2^(e - 1)
    if np.any(exp_field < 1) or np.any(exp_field > 254):
        raise ValueError("value outside the normal bf16 range")
    bits = (exp_field.astype(np.uint32) << 7) | (M.astype(np.uint32) - 128)
    bits |= (x[nz] < 0).astype(np.uint32) << 15
    out[nz] = bits.astype(np.uint16)
    return out


def merge(W_bf_bits, A_bits, B_bits, alpha: float, r: int):
    """W_m = RNE_bf16(W_bf + s B A).  Returns (exact fp64 values, bf16 bits).

    W_bf_bits [n, k], A_bits [r, k], B_bits [n, r]: bf16 bit patterns.
    r == 0 (no adapter) gives W_bf.
    """
    W = f64_from_bf16_bits(W_bf_bits)
    if r == 0:
        return W, np.asarray(W_bf_bits, dtype=np.uint16).copy()
    s = lora_scale(alpha, r)
    A = f64_from_bf16_bits(A_bits)
    B = f64_from_bf16_bits(B_bits)
    exact = W + s * (B @ A)
    return exact, bf16_bits_from_f64(exact)


def requantize(Wm_bits, n_out: int, k_in: int) -> dict:
    """The codec applied to the merged weight (exact fp32 widening)."""
    return quantize_nf4_dq(f64_from_bf16_bits(Wm_bits).astype(np.float32).reshape(n_out, k_in))


def requant_drift(Wm_bits, q: dict, n_out: int, k_in: int) -> float:
    """Relative Frobenius distance between the re-quantized weight (decoded)
    and the merged weight it was made from."""
    _, wb = dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], n_out, k_in)
    a = f64_from_bf16_bits(wb)
    b = f64_from_bf16_bits(Wm_bits)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
