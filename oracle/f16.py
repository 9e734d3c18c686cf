"""fp16 compute dtype -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

The pages' loading code computes in bf16 and names fp16 as the choice on
GPUs without bf16 ([P1] "A complete run on a 12 GB-class GPU": the
``bnb_4bit_compute_dtype`` line).  The fp16 instance is the same layer with
every 16-bit quantity in IEEE binary16 instead of bf16:

* the dequantized weight: W_f16 = RNE_fp16(fp32(T[c] * fp32(q8 * s2)));
* the activations, the adapter matrices and the outputs are fp16.

The forward and backward definitions are those of
:mod:`oracle.qlora_linear`, applied to exact fp64 upcasts of the fp16 inputs
and of W_f16.

Pinned by: round-to-nearest-even against exact rational rounding on crafted
values (halfway cases, the subnormal range, overflow), the exact upcast, and
the fp16 dequant equal to the bf16 dequant's fp32 values rounded to fp16.
"""

from __future__ import annotations

import numpy as np

from .nf4_dq import dequant


def f16_bits_from_f32(x) -> np.ndarray:
    """fp32 -> IEEE binary16 bits, round to nearest even (numpy's cast;
    values from 65520 up become infinity)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f64_from_f16_bits(bits) -> np.ndarray:
    """Exact upcast of binary16 bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant_f16(codes, absmax_q8, absmax_scale, n_out: int, k_in: int, first_block: int = 0):
    """Decode to fp32 and to fp16 bits: W_f16 = RNE_fp16(fp32(T[c] * a'))."""
    w, _ = dequant(codes, absmax_q8, absmax_scale, n_out, k_in, first_block=first_block)
    return w, f16_bits_from_f32(w)
