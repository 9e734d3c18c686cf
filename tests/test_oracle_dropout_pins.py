"""Pins of the LoRA dropout oracle (CPU only).

The generator is tied to its published known-answer vectors; the mask to the
drop rate and independence a Bernoulli(p) mask must show; the dropped layer
to the plain layer at p = 0, to central finite differences with the mask
held fixed, and to unbiasedness of inverted dropout over many seeds.
"""

import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([int(w, 16) for w in line.split()])
    return rows


def test_philox_known_answer_vectors():
    rows = _kat()
    assert len(rows) == 3
    for w in rows:
        out = oracle.philox4x32_10([w[0]], [w[1]], [w[2]], [w[3]], w[4], w[5])
        assert [int(o[0]) for o in out] == w[6:10], [hex(int(o[0])) for o in out]


def test_philox_vectorised_equals_scalar_calls():
    # the array form evaluates every counter independently
    rng = np.random.default_rng(0)
    c = rng.integers(0, 2**32, size=(4, 17), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    full = oracle.philox4x32_10(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(17):
        one = oracle.philox4x32_10([c[0, i]], [c[1, i]], [c[2, i]], [c[3, i]], k0, k1)
        assert [int(o[0]) for o in one] == [int(f[i]) for f in full]


def test_dropout_words_follow_counter_layout():
    # element e takes word e & 3 of the block at counter e >> 2 (64-bit,
    # split lo / hi), key = the seed's two 32-bit halves
    seed = (0xDEADBEEF << 32) | 0x01234567
    n = 4 * 5 + 3
    words = oracle.dropout_words(n, seed)
    for e in range(n):
        q = e >> 2
        out = oracle.philox4x32_10([q & 0xFFFFFFFF], [q >> 32], [0], [0], 0x01234567, 0xDEADBEEF)
        assert int(words[e]) == int(out[e & 3][0])
    # the mask depends on the flat index only: [M, K] equals [1, M K]
    m1 = oracle.dropout_mask(6, 64, 0.3, seed)
    m2 = oracle.dropout_mask(1, 6 * 64, 0.3, seed)
    assert np.array_equal(m1.ravel(), m2.ravel())


@pytest.mark.parametrize("p", [0.05, 0.5])
def test_dropout_rate_and_independence(p):
    M, K = 512, 1024
    mask = oracle.dropout_mask(M, K, p, seed=11)
    n = M * K
    q = oracle.dropout_threshold(p) / 2**32
    dropped = n - int(mask.sum())
    sd = np.sqrt(n * q * (1 - q))
    assert abs(dropped - n * q) < 5 * sd
    x = mask.astype(np.float64).ravel()
    x -= x.mean()
    for lag in (1, 2, 3, 4, 64):  # neighbours, including the same Philox block
        corr = float(np.dot(x[:-lag], x[lag:]) / np.dot(x, x))
        assert abs(corr) < 5 / np.sqrt(n), (lag, corr)
    # another seed gives another mask
    other = oracle.dropout_mask(M, K, p, seed=12)
    assert (other != mask).mean() > q


def test_threshold_and_p_zero_keeps_all():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.05) == 214748364  # floor(0.05 * 2^32)
    assert oracle.dropout_threshold(0.5) == 2**31
    assert oracle.dropout_mask(3, 64, 0.0, seed=5).all()
    with pytest.raises(ValueError):
        oracle.dropout_threshold(1.0)


def _tiny(M=3, N=5, K=64, r=2, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, K)), rng.standard_normal((M, K)), rng.standard_normal((r, K)),
            rng.standard_normal((N, r)), rng.standard_normal((M, N)))


def test_p_zero_equals_plain_layer_exactly():
    W, X, A, B, dY = _tiny(M=4, N=6, K=128, r=3, seed=1)
    mask = oracle.dropout_mask(4, 128, 0.0, seed=9)
    Y0, U0 = oracle.linear_fwd(W, X, A, B, 6.0, 3)
    Y1, U1 = oracle.linear_fwd_dropout(W, X, A, B, 6.0, 3, mask, 0.0)
    assert np.array_equal(Y0, Y1) and np.array_equal(U0, U1)
    g0 = oracle.linear_bwd(W, X, dY, A, B, 6.0, 3)
    g1 = oracle.linear_bwd_dropout(W, X, dY, A, B, 6.0, 3, mask, 0.0)
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)


def test_dropped_frozen_path_is_untouched():
    # only the adapter input is dropped: with B = 0, Y is the plain product
    W, X, A, B, _ = _tiny(M=4, N=6, K=64, r=2, seed=2)
    mask = oracle.dropout_mask(4, 64, 0.5, seed=3)
    Y, _ = oracle.linear_fwd_dropout(W, X, A, np.zeros_like(B), 4.0, 2, mask, 0.5)
    np.testing.assert_allclose(Y, X @ W.T, rtol=1e-13, atol=1e-13)


def test_dropout_backward_matches_finite_differences():
    M, N, K, r = 3, 5, 64, 2
    W, X, A, B, dY = _tiny(M, N, K, r, seed=3)
    alpha, p = 4.0, 0.25
    mask = oracle.dropout_mask(M, K, p, seed=21)
    assert 0 < mask.sum() < mask.size
    dX, dA, dB = oracle.linear_bwd_dropout(W, X, dY, A, B, alpha, r, mask, p)

    def loss(X_, A_, B_):
        Y, _ = oracle.linear_fwd_dropout(W, X_, A_, B_, alpha, r, mask, p)
        return float(np.sum(dY * Y))

    h = 1e-3
    for arr, grad, name in ((X, dX, "X"), (A, dA, "A"), (B, dB, "B")):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            hi = arr.copy(); hi[idx] += h
            lo = arr.copy(); lo[idx] -= h
            args_hi = {"X": (hi, A, B), "A": (X, hi, B), "B": (X, A, hi)}[name]
            args_lo = {"X": (lo, A, B), "A": (X, lo, B), "B": (X, A, lo)}[name]
            num[idx] = (loss(*args_hi) - loss(*args_lo)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-7, atol=1e-8, err_msg=name)


def test_inverted_dropout_is_unbiased_over_seeds():
    # E[mask / (1 - p)] = 1: the seed average of the adapter term approaches
    # the undropped one (a missing or inverted 1 / (1 - p) fails this)
    M, N, K, r = 2, 3, 64, 2
    W, X, A, B, _ = _tiny(M, N, K, r, seed=4)
    alpha, p, n = 2.0, 0.3, 400
    s = oracle.lora_scale(alpha, r)
    ref = s * (X @ A.T) @ B.T
    acc = np.zeros_like(ref)
    for seed in range(n):
        mask = oracle.dropout_mask(M, K, p, seed=seed)
        Y, _ = oracle.linear_fwd_dropout(W, X, A, B, alpha, r, mask, p)
        acc += Y - X @ W.T
    mean = acc / n
    # per-element standard error of the mean of the dropped term
    q = oracle.dropout_threshold(p) / 2**32
    # Var(m / (1 - q)) = q / (1 - q) per element, independent over k:
    # Var(Y - X W^T)[i, n] = q / (1 - q) s^2 sum_k X[i, k]^2 (B A)[n, k]^2
    var = (q / (1 - q)) * s**2 * ((X**2) @ ((B @ A) ** 2).T)
    se = np.sqrt(var / n)
    assert np.all(np.abs(mean - ref) < 5 * se + 1e-12)
