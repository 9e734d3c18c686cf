"""Pins of the storage-format variants (CPU only).

nf4_dq must equal the main codec; the uniform table is checked against its
definition; its codes against exact brute force; each decode against its
formula and error bound; the storage cost against the pages' printed
figures; and the error ordering against the pages' claims ([P2] "Follow-up
questions to expect": NF4 beats evenly spaced int4 on bell-shaped weights;
[P2] "The three QLoRA ideas": double quantization saves about 0.37 bits per
weight).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _normal_weight(seed, shape=(256, 1024), sigma=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def test_uniform_table_definition():
    t = formats.uniform_int4_table()
    assert t.dtype == np.float32 and t.size == 16
    assert t[0] == -1 and t[15] == 1
    assert np.all(np.diff(t) > 0)
    assert np.array_equal(t, -t[::-1])  # symmetric, so no exact zero level
    for i in range(16):  # fp32 RNE of the exact rational -1 + 2 i / 15
        exact = Fraction(-1) + Fraction(2 * i, 15)
        lo = Fraction(float(np.nextafter(t[i], np.float32(-2))))
        hi = Fraction(float(np.nextafter(t[i], np.float32(2))))
        v = Fraction(float(t[i]))
        assert abs(v - exact) <= abs(lo - exact) and abs(v - exact) <= abs(hi - exact)


def test_nf4_dq_format_equals_main_codec():
    W = _normal_weight(1, (64, 512))
    a = formats.quantize_format(W, "nf4_dq")
    b = oracle.quantize_nf4_dq(W)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["absmax_q8"], b["absmax_q8"])
    assert np.array_equal(a["absmax_scale"].view(np.uint32), b["absmax_scale"].view(np.uint32))
    wa, ba = formats.dequant_format(a, 64, 512, "nf4_dq")
    wb, bb = oracle.dequant(b["codes"], b["absmax_q8"], b["absmax_scale"], 64, 512)
    assert np.array_equal(ba, bb) and np.array_equal(wa.view(np.uint32), wb.view(np.uint32))


def _brute_codes(w64, table):
    w = np.asarray(w64, dtype=np.float32)
    a = np.float32(max(abs(float(v)) for v in w))
    out = []
    for v in w:
        x = np.float32(0.0) if a == 0 else np.float32(v) / a
        xf = Fraction(float(x))
        d = [abs(xf - Fraction(float(t))) for t in table]
        out.append(d.index(min(d)))  # exact ties: the lower level
    return out


def test_uniform_codes_brute_force_with_ties():
    t = formats.uniform_int4_table()
    rng = np.random.default_rng(3)
    blk = (rng.standard_normal(64) * 0.02).astype(np.float32)
    blk[0] = 1.0  # absmax 1: x == w below
    # exact fp32 midpoints of neighbouring levels where they are
    # representable (ties), and the floats just above and below them
    j = 1
    for i in range(15):
        mid = (float(t[i]) + float(t[i + 1])) / 2
        if float(np.float32(mid)) == mid and j + 3 <= 64:
            blk[j] = np.float32(mid)
            blk[j + 1] = np.nextafter(np.float32(mid), np.float32(2))
            blk[j + 2] = np.nextafter(np.float32(mid), np.float32(-2))
            j += 3
    assert j > 4  # some midpoints are ties
    W = np.tile(blk, 4).reshape(4, 64)
    W[1] *= np.float32(-0.5)
    W[2] = 0.0
    q = formats.quantize_format(W, "int4")
    for r in range(4):
        assert list(q["code"][64 * r:64 * (r + 1)]) == _brute_codes(W[r], t), r


@pytest.mark.parametrize("fmt", formats.FORMATS)
def test_decode_formula_and_error_bound(fmt):
    W = _normal_weight(5, (32, 256))
    q = formats.quantize_format(W, fmt)
    w, wb = formats.dequant_format(q, 32, 256, fmt)
    T = formats.format_table(fmt)
    c = q["code"].reshape(-1, 64)
    if formats.is_double_quantized(fmt):
        a = (q["absmax_q8"].astype(np.float32) * q["absmax_scale"][np.arange(c.shape[0]) // 256]).astype(np.float32)
    else:
        a = q["absmax"]
        assert np.array_equal(a, np.abs(W.reshape(-1, 64)).max(axis=1))  # stored exactly
    assert np.array_equal(w.reshape(-1, 64), (T[c] * a[:, None]).astype(np.float32))
    assert np.array_equal(wb, oracle.bf16_bits_from_f32(w))
    # |w - w_dq| <= absmax * max gap / 2 (+ the scale's own error when DQ)
    gap = float(np.max(np.diff(T.astype(np.float64))))
    am = np.abs(W.reshape(-1, 64)).max(axis=1).astype(np.float64)
    err = np.abs(w.reshape(-1, 64).astype(np.float64) - W.reshape(-1, 64))
    slack = np.abs(a.astype(np.float64) - am) if formats.is_double_quantized(fmt) else 0 * am
    assert np.all(err <= (am * gap / 2 + slack)[:, None] * (1 + 1e-6) + 1e-12)


def test_bits_per_weight_against_page_figures():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        fig = json.load(f)
    n = 4096 * 4096
    assert round(formats.format_bits_per_weight(n, "nf4_dq"), 3) == fig["bits_per_weight_dq"]["value"]
    assert round(formats.format_bits_per_weight(n, "int4_dq"), 3) == fig["bits_per_weight_dq"]["value"]
    assert formats.format_bits_per_weight(n, "nf4") == fig["bits_per_weight_no_dq"]["value"]
    assert formats.format_bits_per_weight(n, "int4") == fig["bits_per_weight_no_dq"]["value"]


def test_error_ordering_the_pages_claim():
    W = _normal_weight(11)
    e = {f: formats.quant_error(W, f) for f in formats.FORMATS}
    # NF4 beats evenly spaced levels at the same storage, with and without DQ
    assert e["nf4_dq"] < e["int4_dq"] and e["nf4"] < e["int4"]
    # double quantization costs little error for its 0.37-bit saving
    assert e["nf4"] <= e["nf4_dq"] < 1.02 * e["nf4"]
    assert e["int4"] <= e["int4_dq"] < 1.02 * e["int4"]
    # the existing NF4-DQ figure (same seed and shape as the main pins)
    assert 0.08 < e["nf4_dq"] < 0.10
    # and the int4 figure matches the plain evenly spaced nearest-level
    # computation written independently
    blocks = W.reshape(-1, 64).astype(np.float64)
    am = np.abs(blocks).max(axis=1, keepdims=True)
    lv = np.linspace(-1, 1, 16)
    wu = lv[np.argmin(np.abs((blocks / am)[..., None] - lv), axis=-1)] * am
    e_plain = np.linalg.norm(wu - blocks) / np.linalg.norm(blocks)
    assert abs(e["int4"] - e_plain) < 1e-4
