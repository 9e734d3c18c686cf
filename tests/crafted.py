"""Crafted quantizer inputs shared by the CPU and GPU tests.

Values are placed, not computed by the method: for a block absmax a and a
table of 16 levels, the weights fp32(theta_i * a) and fp32(T_i * a) (theta_i
the round-down midpoint thresholds the oracle defines) and their 1..4-ulp
neighbours, in blocks that also hold +-a.  Absmaxes that are not powers of
two make the reciprocal 1 / a inexact, so these blocks probe the quantize
kernel's fast path right at its decision boundaries.
"""

import numpy as np

import oracle

F = np.float32


def _bf16_round(v):
    """fp32 values rounded to bf16 (RNE) and widened back to fp32."""
    bits = oracle.bf16_bits_from_f32(np.asarray(v, dtype=F))
    return (bits.astype(np.uint32) << 16).view(F)


def _bf16_step(v, up):
    """Next bf16 value above (up) or below a bf16-representable fp32 value."""
    b = (np.asarray(v, dtype=F).view(np.uint32) >> 16).astype(np.int64)
    neg = b >= 0x8000
    mag = b & 0x7FFF
    if (up and not neg) or (not up and neg):
        mag = mag + 1
    elif mag == 0:  # +-0 stepping away from the sign: to the other side
        return F(2.0 ** -133) * (F(1) if up else F(-1))
    else:
        mag = mag - 1
    nb = (mag | (0x8000 if neg else 0)) & 0xFFFF
    return (np.array([nb], dtype=np.uint32) << 16).view(F)[0]


def absmax_set(rng, n):
    """A fixed list of awkward absmaxes plus n log-uniform ones in [1e-6, 10]."""
    fixed = [0.0371, 0.02913, 6.0, 3.0, 0.1, 1.7e-3, 0.05123456, 7.3e-5, 123.456, 1.0 / 3.0]
    rand = list(np.exp(rng.uniform(np.log(1e-6), np.log(10.0), n)).astype(F))
    return [F(a) for a in fixed] + rand


def near_threshold_blocks(table, absmaxes, rng, bf16=False):
    """Blocks [n, 64] of fp32 values (bf16-representable when bf16=True)."""
    theta = oracle.nf4_thresholds(table).astype(F)
    blocks = []
    for a in absmaxes:
        a = F(a)
        if bf16:
            a = _bf16_round(a)[()]
        vals = []
        for base in list((theta * a).astype(F)) + list((np.asarray(table, dtype=F) * a).astype(F)):
            v = _bf16_round(base)[()] if bf16 else base
            vals.append(v)
            up, dn = v, v
            for _ in range(4):
                if bf16:
                    up, dn = _bf16_step(up, True), _bf16_step(dn, False)
                else:
                    up, dn = np.nextafter(up, F(np.inf)), np.nextafter(dn, F(-np.inf))
                vals.append(up)
                vals.append(dn)
        vals = np.array(vals, dtype=F)
        vals = vals[np.abs(vals) <= a]
        rng.shuffle(vals)
        for s in range(0, vals.size, 62):
            chunk = vals[s:s + 62]
            blk = np.zeros(64, dtype=F)
            blk[0], blk[1] = a, -a if rng.random() < 0.5 else a
            blk[2:2 + chunk.size] = chunk
            blocks.append(blk)
    return np.stack(blocks)


def zero_threshold_underflow_block():
    """{6, 3 * 2^-149, 2.8, ...}: under a table whose middle threshold is 0,
    w / a rounds to +0 while w * fp32(1 / a) rounds to the smallest
    subnormal."""
    blk = np.full(64, F(2.8), dtype=F)
    blk[0] = F(6.0)
    blk[1] = F(3 * 2.0 ** -149)
    return blk


def as_weight(blocks, blocks_per_row=8):
    """Blocks -> an [n_out, 64 * blocks_per_row] weight, n_out a multiple of
    8, padded with N(0, 0.02^2) blocks."""
    rng = np.random.default_rng(5)
    per = 8 * blocks_per_row
    nb = -(-blocks.shape[0] // per) * per
    pad = (rng.standard_normal((nb - blocks.shape[0], 64)) * 0.02).astype(F)
    allb = np.concatenate([blocks.astype(F), pad])
    return allb.reshape(-1, 64 * blocks_per_row)
