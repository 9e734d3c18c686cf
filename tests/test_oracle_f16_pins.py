"""Pins of the fp16 oracle (CPU only).

fp16 rounding is tied to exact rational round-to-nearest-even (ties to even,
subnormals, overflow to infinity); the fp16 dequant to the fp32 values of the
main dequant rounded once; and the fp16 layer (the plain definition on exact
upcasts) to the same properties the bf16 layer is pinned by.
"""

from fractions import Fraction

import numpy as np

import oracle
from oracle import f16


def _rne_f16_exact(x: float) -> float:
    """binary16 round-to-nearest-even of the exact value of x, by rational
    arithmetic (11-bit significand, exponents -14..15, subnormal step
    2^-24, overflow past 65520 to infinity)."""
    q = Fraction(x)
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    if a >= Fraction(65520):
        return sign * float("inf")
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    if e < -14:  # subnormal: multiples of 2^-24
        step = Fraction(1, 2 ** 24)
    else:
        step = Fraction(2) ** (e - 10)
    n = abs(q) / step
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * step)


def test_f16_rounding_against_exact_rationals():
    vals = [0.0, 1.0, -1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 1.0 + 2 ** -11 + 2 ** -20,  # ties, above
            65504.0, 65519.0, 65520.0, 70000.0, -65520.0,  # top of the range, overflow
            2 ** -24, 2 ** -25, 3 * 2 ** -25, 2 ** -25 + 2 ** -40, 2 ** -14, 2 ** -14 - 2 ** -25,  # subnormals
            0.1, -0.3333, 0.02, 1e-6, 6.1e-5]
    rng = np.random.default_rng(1)
    vals += list((rng.standard_normal(2000) * 10.0 ** rng.uniform(-8, 4, 2000)).astype(np.float32))
    x = np.array(vals, dtype=np.float32)
    got = f16.f64_from_f16_bits(f16.f16_bits_from_f32(x))
    for xi, gi in zip(x, got):
        assert gi == _rne_f16_exact(float(xi)) or (np.isinf(gi) and np.isinf(_rne_f16_exact(float(xi)))), xi


def test_f16_upcast_is_exact():
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    v = f16.f64_from_f16_bits(bits)
    finite = np.isfinite(v)
    # round trip of every finite value (the sign of zero included)
    back = f16.f16_bits_from_f32(v[finite].astype(np.float32))
    assert np.array_equal(back, bits[finite])


def test_f16_dequant_is_one_rounding_of_the_fp32_decode():
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((16, 256), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    q = oracle.quantize_nf4_dq(W)
    w32, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], 16, 256)
    w, bits = f16.dequant_f16(q["codes"], q["absmax_q8"], q["absmax_scale"], 16, 256)
    assert np.array_equal(w, w32)
    ex = np.array([_rne_f16_exact(float(v)) for v in w32.ravel()]).reshape(w32.shape)
    assert np.array_equal(f16.f64_from_f16_bits(bits), ex)
    # fp16 keeps 3 more significand bits than bf16: never further from w32
    assert np.all(np.abs(f16.f64_from_f16_bits(bits) - w32) <= np.abs(oracle.f64_from_bf16_bits(wb) - w32))


def test_f16_layer_reduces_like_the_bf16_one():
    # B = 0: the plain product of the fp16 upcasts; the adapter term scales
    # with alpha (the definition does not depend on the 16-bit type)
    rng = np.random.default_rng(5)
    W = f16.f64_from_f16_bits(f16.f16_bits_from_f32(rng.standard_normal((6, 64)).astype(np.float32) * 0.02))
    X = f16.f64_from_f16_bits(f16.f16_bits_from_f32(rng.standard_normal((4, 64)).astype(np.float32)))
    A = f16.f64_from_f16_bits(f16.f16_bits_from_f32(rng.standard_normal((3, 64)).astype(np.float32) / 8))
    B = f16.f64_from_f16_bits(f16.f16_bits_from_f32(rng.standard_normal((6, 3)).astype(np.float32) / 100))
    Y0, _ = oracle.linear_fwd(W, X, A, np.zeros_like(B), 6.0, 3)
    np.testing.assert_allclose(Y0, X @ W.T, rtol=1e-14, atol=1e-14)
    Y1, _ = oracle.linear_fwd(W, X, A, B, 6.0, 3)
    Y2, _ = oracle.linear_fwd(W, X, A, B, 12.0, 3)
    np.testing.assert_allclose(Y2 - X @ W.T, 2 * (Y1 - X @ W.T), rtol=1e-12, atol=1e-15)
