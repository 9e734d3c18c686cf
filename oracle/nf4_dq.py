"""NF4 codec with double-quantized block scales -- CPU oracle.

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).  numpy, written step by step
in the order the pages describe the format:

1. a 16-level table at quantiles of the normal distribution
   ([P1] "The mechanism in brief"; [P2] "The three QLoRA ideas";
   [P4] "NF4 and double quantisation");
2. the weight split into blocks of 64 values, each with its own fp32 absmax
   ([P1] "The mechanism in brief"; [P4] "NF4 and double quantisation");
3. every value normalised by its block absmax and given the code of the
   nearest level, two 4-bit codes per byte ([P4] "Where 24 GB goes", ledger
   term A, prices the codes at half a byte per weight);
4. the block absmaxes themselves stored as 8-bit codes, one 32-bit scale per
   256 blocks ([P1] "The mechanism in brief"; [P2] "The three QLoRA ideas");
5. dequantization back to bf16, the compute dtype of the matmul
   ([P1] "The mechanism in brief"; [P4] "The idea in one line").

Readings where the pages are silent (each listed in the design notes):

* NF4 grid: 8 positive quantiles, 7 negative, plus an exact zero, with tail
  offset ``TAIL_OFFSET``; normalised so the extreme levels are -1 and +1.
  The offset value is **parity unpinned** by the pages (they only say
  "quantiles of a normal distribution"); everything else about the table is
  pinned by invariants and by an erf-based closed form.
* Flatten order is row-major; K is a multiple of 64 so blocks never straddle
  rows.
* x = fp32(w / absmax) by IEEE division; absmax 0 gives x = 0.
* Nearest level with exact ties going to the lower (more negative) level.
* Low nibble holds the even-indexed element.
* Double quantization is unsigned linear: s2 = fp32(groupmax / 255),
  q8 = RNE(fp32(absmax / s2)) clamped to [0, 255]; a zero group gives
  s2 = 0 and q8 = 0; the last group may be partial.
* Dequant is w = fp32(T[c] * fp32(q8 * s2)), then round-to-nearest-even bf16.
"""

from __future__ import annotations

import statistics

import numpy as np

BLOCK = 64  # weights per absmax block
GROUP = 256  # blocks per second-level scale

# Tail offset of the quantile grid: the mean of 1 - 1/(2*15) and 1 - 1/(2*16).
# The pages give no value for it (parity unpinned); this is the offset of the
# construction in the paper the pages cite.
TAIL_OFFSET = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


def _normal_quantile(p: float) -> float:
    """Standard normal inverse CDF in fp64 (stdlib NormalDist)."""
    return statistics.NormalDist().inv_cdf(p)


def nf4_table_fp64() -> np.ndarray:
    """The 16 NF4 levels in fp64, ascending.

    Positive side: quantiles at 0.5 + (d - 0.5) * j / 8 for j = 1..8;
    negative side: minus the quantiles at 0.5 + (d - 0.5) * j / 7 for
    j = 1..7; plus an exact 0.  All divided by the quantile at d, so the
    extremes are exactly -1 and +1.

    Pinned by: invariants (16 levels, sorted, exact 0, 7 negative / 8
    positive, extremes +-1), the erf closed form (Phi(T_j * Phi^-1(d)) is
    evenly spaced on each side), and a second, independent inverse normal
    (scipy) giving the bit-identical fp32 table.
    """
    d = TAIL_OFFSET
    step = d - 0.5
    pos = [_normal_quantile(0.5 + step * (j / 8.0)) for j in range(1, 9)]
    neg = [-_normal_quantile(0.5 + step * (j / 7.0)) for j in range(1, 8)]
    top = _normal_quantile(d)
    levels = sorted(neg + [0.0] + pos)
    return np.array([v / top for v in levels], dtype=np.float64)


def nf4_table() -> np.ndarray:
    """fp32 table: RNE of the fp64 levels."""
    return nf4_table_fp64().astype(np.float32)


def _round_down_to_f32(x: float) -> np.float32:
    f = np.float32(x)
    if float(f) > x:
        f = np.nextafter(f, np.float32(-np.inf))
    return f


def nf4_thresholds(table: np.ndarray | None = None) -> np.ndarray:
    """Decision thresholds theta_i = RD_fp32((T_i + T_{i+1}) / 2), i = 0..14.

    The midpoint of two fp32 numbers is exact in fp64.  For fp32 x,
    ``x > theta_i`` holds exactly when x is strictly closer to T_{i+1} than
    to T_i, so counting exceeded thresholds gives the nearest level with
    ties to the lower one.  Pinned by exact brute force (fractions).
    """
    t = nf4_table() if table is None else np.asarray(table, dtype=np.float32)
    mids = [(float(t[i]) + float(t[i + 1])) / 2.0 for i in range(15)]
    return np.array([_round_down_to_f32(m) for m in mids], dtype=np.float32)


# --------------------------------------------------------------------------
# bf16 helpers (bit patterns held in uint16)
# --------------------------------------------------------------------------

def bf16_bits_from_f32(x) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bits.

    Finite inputs only.  Pinned against torch's fp32 -> bf16 conversion and
    hand-made ties.
    """
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    rounded = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def f64_from_bf16_bits(bits) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# quantization steps
# --------------------------------------------------------------------------

def block_absmax(w_flat: np.ndarray) -> np.ndarray:
    """fp32 max |w| of each block of 64 consecutive weights (exact)."""
    blocks = np.asarray(w_flat, dtype=np.float32).reshape(-1, BLOCK)
    return np.max(np.abs(blocks), axis=1).astype(np.float32)


def nearest_codes(w_flat: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """4-bit code of each weight: nearest level to fp32(w / absmax).

    Returns one uint8 code (0..15) per weight.  absmax == 0 gives x = 0,
    which is code 7 (the exact zero level).
    """
    blocks = np.asarray(w_flat, dtype=np.float32).reshape(-1, BLOCK)
    a = np.asarray(absmax, dtype=np.float32)
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)  # IEEE fp32 division
    x = np.where(a[:, None] > 0, x, np.float32(0.0)).astype(np.float32)
    theta = nf4_thresholds()
    # number of thresholds strictly below x
    codes = np.searchsorted(theta, x.ravel(), side="left")
    return codes.astype(np.uint8)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte: element 2j in the low nibble, 2j+1 in the high."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << np.uint8(4))).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & np.uint8(0x0F)
    out[1::2] = p >> np.uint8(4)
    return out


def double_quantize(absmax: np.ndarray):
    """Second level: 8-bit codes for the block absmaxes, one fp32 scale per
    256 consecutive blocks ([P1] "The mechanism in brief").

    Returns (q8 uint8[nb], s2 float32[ceil(nb/256)]).
    """
    a = np.asarray(absmax, dtype=np.float32)
    nb = a.size
    ng = (nb + GROUP - 1) // GROUP
    padded = np.zeros(ng * GROUP, dtype=np.float32)
    padded[:nb] = a
    gmax = padded.reshape(ng, GROUP).max(axis=1).astype(np.float32)
    s2 = (gmax / np.float32(255.0)).astype(np.float32)
    s2_per_block = np.repeat(s2, GROUP)[:nb]
    safe = np.where(s2_per_block > 0, s2_per_block, np.float32(1.0)).astype(np.float32)
    ratio = (a / safe).astype(np.float32)  # IEEE fp32 division
    q = np.clip(np.rint(ratio), 0.0, 255.0)  # rint = round half to even
    q = np.where(s2_per_block > 0, q, 0.0)
    return q.astype(np.uint8), s2


def quantize_nf4_dq(W: np.ndarray):
    """Quantize an fp32 [N, K] weight (K % 64 == 0).

    Returns a dict with ``codes`` (uint8[N*K/2]), ``absmax_q8`` (uint8[nb]),
    ``absmax_scale`` (float32[ng]) and, for checks, the pre-DQ fp32
    ``absmax`` and the unpacked ``code`` array.
    Codes use the fp32 absmax before double quantization.
    """
    W = np.asarray(W, dtype=np.float32)
    if W.ndim != 2 or W.shape[1] % BLOCK != 0:
        raise ValueError("W must be [N, K] with K % 64 == 0")
    flat = W.ravel()
    absmax = block_absmax(flat)
    code = nearest_codes(flat, absmax)
    q8, s2 = double_quantize(absmax)
    return {
        "codes": pack_codes(code),
        "absmax_q8": q8,
        "absmax_scale": s2,
        "absmax": absmax,
        "code": code,
    }


def quantize_groups(W_flat: np.ndarray, groups) -> dict:
    """Quantize only the listed DQ groups of a flattened weight.

    Groups are independent (each is 256 consecutive blocks), so this equals
    slicing the output of :func:`quantize_nf4_dq`.  Used to check very
    large weights on a sample.  Returns per-group dicts keyed by group id.
    """
    W_flat = np.asarray(W_flat, dtype=np.float32).ravel()
    nb = W_flat.size // BLOCK
    out = {}
    for g in groups:
        b0 = g * GROUP
        b1 = min(nb, b0 + GROUP)
        seg = W_flat[b0 * BLOCK:b1 * BLOCK]
        absmax = block_absmax(seg)
        code = nearest_codes(seg, absmax)
        q8, s2 = double_quantize(absmax)
        assert s2.size == 1
        out[int(g)] = {
            "codes": pack_codes(code),
            "absmax_q8": q8,
            "absmax_scale": s2,
            "absmax": absmax,
        }
    return out


def dequant(codes: np.ndarray, absmax_q8: np.ndarray, absmax_scale: np.ndarray,
            n_out: int, k_in: int, first_block: int = 0):
    """Decode to fp32 and bf16.

    a' = fp32(q8 * s2);  w = fp32(T[c] * a');  W_bf = RNE_bf16(w).
    ``first_block`` lets a slice that starts at block ``first_block`` of the
    full matrix find its group scale.  Returns (w_fp32 [N, K], W_bf uint16
    bits [N, K]).
    """
    T = nf4_table()
    c = unpack_codes(codes)
    nb = c.size // BLOCK
    q = np.asarray(absmax_q8, dtype=np.uint8)[:nb].astype(np.float32)
    s2 = np.asarray(absmax_scale, dtype=np.float32)
    gidx = (np.arange(nb) + first_block) // GROUP - first_block // GROUP
    a = (q * s2[gidx]).astype(np.float32)
    w = (T[c].reshape(nb, BLOCK) * a[:, None]).astype(np.float32)
    w = w.reshape(n_out, k_in)
    return w, bf16_bits_from_f32(w)


# --------------------------------------------------------------------------
# storage accounting
# --------------------------------------------------------------------------

def storage_bytes(n_weights: int, double_quant: bool = True) -> int:
    """Bytes of the stored format for n_weights (a multiple of 64).

    With double quantization: codes (n/2) + one byte per block + 4 bytes per
    group of 256 blocks.  Without: codes + one fp32 absmax per block.
    """
    if n_weights % BLOCK:
        raise ValueError("n_weights must be a multiple of 64")
    nb = n_weights // BLOCK
    if double_quant:
        ng = (nb + GROUP - 1) // GROUP
        return n_weights // 2 + nb + 4 * ng
    return n_weights // 2 + 4 * nb


def bits_per_weight(n_weights: int, double_quant: bool = True) -> float:
    return 8.0 * storage_bytes(n_weights, double_quant) / n_weights
