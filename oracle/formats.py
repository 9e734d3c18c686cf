"""Storage-format variants of the frozen weight -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

The pages justify the stored format against two alternatives:

* block scales kept as one fp32 absmax per 64 weights, 4.5 bits per weight,
  which double quantization cuts to about 4.127 ([P1] "The mechanism in
  brief"; [P2] "The three QLoRA ideas"; [P4] "NF4 and double
  quantisation");
* evenly spaced 4-bit levels ("plain int4"), which waste levels on rare
  large values, so NF4 has the lower error on bell-shaped weights ([P2]
  "Follow-up questions to expect").

Four formats, all with blocks of 64 and absmax normalisation:

    format    levels                         block scale
    nf4_dq    NF4 (:func:`oracle.nf4_table`) q8 code + fp32 step per 256 blocks
    nf4       NF4                            fp32 absmax per block
    int4_dq   uniform: -1 + 2 i / 15         q8 code + fp32 step per 256 blocks
    int4      uniform                        fp32 absmax per block

Reading for "plain int4": 16 levels evenly spaced over [-1, 1] (the fp64
values rounded to fp32), coded exactly like NF4 -- nearest level by
counting round-down midpoint thresholds, ties to the lower level.  Decoding
is w = fp32(T[c] * a') with a' = fp32(q8 * s2) (double quantized) or the
fp32 absmax itself.

Pinned by: nf4_dq here equals :func:`oracle.quantize_nf4_dq`; the uniform
table's spacing, symmetry and extremes; exact brute-force nearest-level codes
for the uniform table; the dequant formula and error bound per format; the
pages' bits-per-weight figures; and the error ordering the pages claim
(NF4 below int4 on normal weights; double quantization costing little).
"""

from __future__ import annotations

import numpy as np

from .nf4_dq import (
    BLOCK,
    block_absmax,
    double_quantize,
    nf4_table,
    nf4_thresholds,
    pack_codes,
    unpack_codes,
    bf16_bits_from_f32,
    bits_per_weight,
)

FORMATS = ("nf4_dq", "nf4", "int4_dq", "int4")


def uniform_int4_table() -> np.ndarray:
    """16 evenly spaced levels over [-1, 1]: fp32 RNE of -1 + 2 i / 15."""
    return np.array([-1.0 + 2.0 * i / 15.0 for i in range(16)], dtype=np.float64).astype(np.float32)


def format_table(fmt: str) -> np.ndarray:
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    return nf4_table() if fmt.startswith("nf4") else uniform_int4_table()


def is_double_quantized(fmt: str) -> bool:
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    return fmt.endswith("_dq")


def table_codes(w_flat: np.ndarray, absmax: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Nearest level of fp32(w / absmax) in `table`, ties to the lower level
    (count of round-down midpoint thresholds strictly below x); absmax == 0
    gives x = 0."""
    blocks = np.asarray(w_flat, dtype=np.float32).reshape(-1, BLOCK)
    a = np.asarray(absmax, dtype=np.float32)
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)  # IEEE fp32 division
    x = np.where(a[:, None] > 0, x, np.float32(0.0)).astype(np.float32)
    theta = nf4_thresholds(table)
    return np.searchsorted(theta, x.ravel(), side="left").astype(np.uint8)


def quantize_format(W: np.ndarray, fmt: str) -> dict:
    """fp32 [N, K] -> dict with ``codes`` (packed), and either ``absmax_q8``
    + ``absmax_scale`` (double quantized) or ``absmax`` (fp32 per block)."""
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % BLOCK != 0:
        raise ValueError("W must be [N, K] with K % 64 == 0")
    flat = W.ravel()
    absmax = block_absmax(flat)
    code = table_codes(flat, absmax, format_table(fmt))
    out = {"codes": pack_codes(code), "code": code, "absmax": absmax}
    if is_double_quantized(fmt):
        q8, s2 = double_quantize(absmax)
        out["absmax_q8"] = q8
        out["absmax_scale"] = s2
    return out


def dequant_format(q: dict, n_out: int, k_in: int, fmt: str):
    """Returns (w fp32 [N, K], W_bf bf16 bits [N, K])."""
    T = format_table(fmt)
    c = unpack_codes(q["codes"])
    nb = c.size // BLOCK
    if is_double_quantized(fmt):
        s2 = np.asarray(q["absmax_scale"], dtype=np.float32)
        a = (np.asarray(q["absmax_q8"], dtype=np.uint8)[:nb].astype(np.float32)
             * s2[np.arange(nb) // 256]).astype(np.float32)
    else:
        a = np.asarray(q["absmax"], dtype=np.float32)[:nb]
    w = (T[c].reshape(nb, BLOCK) * a[:, None]).astype(np.float32).reshape(n_out, k_in)
    return w, bf16_bits_from_f32(w)


def format_bits_per_weight(n_weights: int, fmt: str) -> float:
    return bits_per_weight(n_weights, double_quant=is_double_quantized(fmt))


def quant_error(W: np.ndarray, fmt: str) -> float:
    """Relative Frobenius error of the decoded (fp32) weight."""
    W = np.asarray(W, dtype=np.float32)
    w, _ = dequant_format(quantize_format(W, fmt), W.shape[0], W.shape[1], fmt)
    d = w.astype(np.float64) - W.astype(np.float64)
    return float(np.linalg.norm(d) / np.linalg.norm(W.astype(np.float64)))
