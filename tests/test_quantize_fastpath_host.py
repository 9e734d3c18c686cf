"""CPU check of the rule the quantize kernel uses to pick each 4-bit code.

The code of weight w in a block with absmax a is defined from the IEEE fp32
quotient x = fp32(w / a): the number of decision thresholds below x ([P1]
"The mechanism in brief": nearest of 16 levels after absmax normalisation;
the oracle's ``nearest_codes`` / ``formats.table_codes``).  The kernel avoids
the division on its common path: it forms x' = fp32(w * fp32(1 / a)), finds
the table cell of x' (256 cells of width 1/128 over [-1, 1], each holding a
candidate count and the next threshold t), and compares x' with t.  Only a
block in which some x' lies within max(2^-20 |t|, 2^-100) of its t is coded
again from the quotient itself; a block whose absmax is below 2^-100 is
scaled by 2^64 first.

This test restates that rule in numpy fp32 (round to nearest even,
subnormals kept, as on the GPU) and checks that it gives the oracle's codes
for random normal weights, for weights placed a few ulps around every
threshold (and every level) of blocks with absmaxes that are not powers of
two, for tiny and subnormal blocks, and for the NF4 and the evenly spaced
tables.  It also shows the absolute floor is needed: without it, a block
{6, 3 * 2^-149, 2.8, ...} gets the wrong code under the evenly spaced table, whose
middle threshold is exactly 0 (the quotient rounds to 0, the product to the
smallest subnormal).
"""

import numpy as np
import pytest

import oracle
from oracle import formats

from crafted import absmax_set, near_threshold_blocks, zero_threshold_underflow_block

F = np.float32


def _search_table(theta):
    """cand[i] = thresholds below the start of cell i - 1 (cell i covers
    [(i - 128) / 128, (i - 127) / 128)); per cell the candidate threshold
    (2.0 past the last one: never exceeded, never close)."""
    theta64 = theta.astype(np.float64)
    cand = np.zeros(256, dtype=np.int64)
    for i in range(256):
        start = -np.inf if i == 0 else (i - 1) / 128.0 - 1.0
        cand[i] = int(np.sum(theta64 < start))
    t = np.where(cand < 15, theta[np.minimum(cand, 14)], F(2.0)).astype(F)
    return cand, t


def _lookup(x, cand, tcell):
    cell = np.trunc(x * F(128) + F(128))  # x * 128 is exact; one rounding in the add
    cell = np.clip(np.nan_to_num(cell), 0, 255).astype(np.int64)
    return cand[cell], tcell[cell]


def emulate_codes(W, table, floor=2.0 ** -100):
    """The kernel's decision rule on fp32 blocks W [nblocks, 64]."""
    W = np.asarray(W, dtype=F)
    theta = oracle.nf4_thresholds(table)
    cand, tcell = _search_table(theta)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore", under="ignore"):
        am = np.max(np.abs(W), axis=1).astype(F)
        small = am < F(2.0 ** -100)
        Ws = np.where(small[:, None], W * F(2.0 ** 64), W).astype(F)
        amq = np.where(small, am * F(2.0 ** 64), am).astype(F)
        rcp = np.where(amq > 0, F(1) / np.where(amq > 0, amq, F(1)), F(0)).astype(F)
        xp = (Ws * rcp[:, None]).astype(F)
        c0, t = _lookup(xp, cand, tcell)
        band = np.maximum(np.abs(t) * F(2.0 ** -20), F(floor)).astype(F)
        nd = np.min((np.abs(xp - t) - band).astype(F), axis=1)
        code = c0 + (xp > t)
        near = nd <= 0
        x = np.where(amq[:, None] > 0, Ws / np.where(amq > 0, amq, F(1))[:, None], F(0)).astype(F)
        c0x, tx = _lookup(x, cand, tcell)
        exact_path = c0x + (x > tx)
    code = np.where(near[:, None], exact_path, code)
    return code.astype(np.uint8), near


def exact_codes(W, table):
    W = np.asarray(W, dtype=F)
    flat = W.ravel()
    return formats.table_codes(flat, oracle.block_absmax(flat), table).reshape(W.shape)


TABLES = {"nf4": oracle.nf4_table(), "int4": formats.uniform_int4_table()}


@pytest.mark.parametrize("name", ["nf4", "int4"])
def test_fast_path_matches_division_random(name):
    """About 12 M normal weights (sigma 0.02, and a second batch spanning
    many scales): the fast path agrees with the quotient everywhere, and only
    a small share of blocks needs the quotient."""
    rng = np.random.default_rng(2024)
    table = TABLES[name]
    W = (rng.standard_normal((150_000, 64), dtype=F) * F(0.02)).astype(F)
    got, near = emulate_codes(W, table)
    assert np.array_equal(got, exact_codes(W, table))
    if name == "nf4":
        assert near.mean() < 1e-3, near.mean()
    scales = np.exp(rng.uniform(np.log(1e-30), np.log(1e10), (37_500, 1))).astype(F)
    W2 = (rng.standard_normal((37_500, 64), dtype=F) * scales).astype(F)
    got2, _ = emulate_codes(W2, table)
    assert np.array_equal(got2, exact_codes(W2, table))


@pytest.mark.parametrize("name", ["nf4", "int4"])
def test_fast_path_matches_division_near_thresholds(name):
    """Weights at fp32(theta_i * a), fp32(T_i * a) and 1..4 ulps around them,
    in blocks whose absmax is not a power of two (the reciprocal inexact)."""
    rng = np.random.default_rng(7)
    table = TABLES[name]
    W = near_threshold_blocks(table, absmax_set(rng, 300), rng)
    got, near = emulate_codes(W, table)
    assert np.array_equal(got, exact_codes(W, table))
    assert near.any()  # the band is exercised


@pytest.mark.parametrize("name", ["nf4", "int4"])
def test_fast_path_tiny_and_subnormal_blocks(name):
    """Blocks with absmax below 2^-100 (scaled by 2^64 first), subnormal
    weights beside large ones, zeros and negative zeros."""
    rng = np.random.default_rng(11)
    table = TABLES[name]
    blocks = []
    for a in [2.0 ** -101, 3.1e-35, 1e-38, 2.0 ** -126, 7e-44]:
        blocks.append((rng.uniform(-1, 1, 64) * a).astype(F))
        blocks[-1][0] = F(a)
    sub = np.arange(1, 64, dtype=np.float64) * 2.0 ** -149
    for a in [6.0, 3.0, 1.0, 12.0, 2.0 ** 20 * 3, 0.75]:
        blk = np.concatenate([[a], sub[:63] * rng.choice([-1, 1], 63)]).astype(F)
        blocks.append(blk)
    blocks.append(np.zeros(64, dtype=F))
    blocks.append(-np.zeros(64, dtype=F))
    W = np.stack(blocks)
    got, _ = emulate_codes(W, table)
    assert np.array_equal(got, exact_codes(W, table))


def test_absolute_floor_is_needed_for_a_zero_threshold():
    """Under the evenly spaced table (middle threshold exactly 0) the block
    {6, 3 * 2^-149, 2.8, ...}: w / a rounds to +0 (code 7) while
    w * fp32(1/6) rounds to the smallest subnormal (code 8).  The relative
    band alone (2^-20 |t| = 0) misses it (2.8 / 6 is far from every
    threshold, and no weight is 0); the 2^-100 floor sends the block to the
    quotient."""
    table = TABLES["int4"]
    assert oracle.nf4_thresholds(table)[7] == 0.0
    blk = zero_threshold_underflow_block()[None, :]
    ref = exact_codes(blk, table)
    assert ref[0, 1] == 7
    with_floor, _ = emulate_codes(blk, table)
    without, _ = emulate_codes(blk, table, floor=0.0)
    assert np.array_equal(with_floor, ref)
    assert without[0, 1] == 8  # the rule without the floor would be wrong here


def test_near_threshold_bf16_blocks_on_the_rule():
    """The bf16-input codec (re-quantizing a merged weight) widens bf16
    exactly and runs the same rule: bf16 values a few bf16 ulps around every
    threshold of bf16 absmaxes."""
    rng = np.random.default_rng(13)
    table = TABLES["nf4"]
    W = near_threshold_blocks(table, absmax_set(rng, 200), rng, bf16=True)
    assert np.array_equal(oracle.bf16_bits_from_f32(W).astype(np.uint32) << 16, W.view(np.uint32))
    got, _ = emulate_codes(W, table)
    assert np.array_equal(got, exact_codes(W, table))
