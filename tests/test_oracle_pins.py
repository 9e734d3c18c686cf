"""Pins of the CPU oracle to things other than itself.

Each test ties one oracle function to what the pages print, to a closed form,
to an invariant, to exact brute force on tiny inputs, or to an independent
library routine, so that a plausible mistake (a dropped term, a wrong sign or
index, a transposed operand, a wrong tie-break) fails at least one of them.
CPU only.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import nf4_dq
from bit_nf4_quantized_double_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _figures():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- table ----

def _phi(x):
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def _phi_inv_bisect(p):
    """Inverse normal by bisection on math.erf -- independent of the
    oracle's stdlib routine."""
    lo, hi = -12.0, 12.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_table_invariants():
    T = oracle.nf4_table()
    assert T.dtype == np.float32 and T.size == _figures()["nf4_levels"]["value"]
    assert np.all(np.diff(T) > 0)
    assert T[0] == -1.0 and T[15] == 1.0
    assert T[7] == 0.0 and not np.signbit(T[7])
    assert np.sum(T < 0) == 7 and np.sum(T > 0) == 8


def test_table_closed_form_even_quantile_spacing():
    """Phi(T_j * Phi^-1(d)) is evenly spaced in probability on each side."""
    d = oracle.TAIL_OFFSET
    m = _phi_inv_bisect(d)
    T64 = oracle.nf4_table_fp64()
    T32 = oracle.nf4_table().astype(np.float64)
    for j in range(1, 9):  # positive side: index 7 + j
        target = 0.5 + (d - 0.5) * j / 8.0
        assert abs(_phi(T64[7 + j] * m) - target) < 1e-13
        assert abs(_phi(T32[7 + j] * m) - target) < 5e-8
    for j in range(1, 8):  # negative side: index 7 - j
        target = 0.5 + (d - 0.5) * j / 7.0
        assert abs((1.0 - _phi(T64[7 - j] * m)) - target) < 1e-13
        assert abs((1.0 - _phi(T32[7 - j] * m)) - target) < 5e-8


def test_table_second_inverse_normal_bit_identical():
    from scipy.special import ndtri
    d = oracle.TAIL_OFFSET
    step = d - 0.5
    pos = [ndtri(0.5 + step * (j / 8.0)) for j in range(1, 9)]
    neg = [-ndtri(0.5 + step * (j / 7.0)) for j in range(1, 8)]
    lv = np.array(sorted(neg + [0.0] + pos)) / ndtri(d)
    assert np.array_equal(lv.astype(np.float32).view(np.uint32),
                          oracle.nf4_table().view(np.uint32))


def test_thresholds_are_round_down_midpoints():
    T = oracle.nf4_table()
    th = oracle.nf4_thresholds()
    for i in range(15):
        mid = Fraction(float(T[i])) + Fraction(float(T[i + 1]))
        mid /= 2
        assert Fraction(float(th[i])) <= mid
        assert Fraction(float(np.nextafter(th[i], np.float32(np.inf)))) > mid


# ---------------------------------------------------------------- codes ----

def _brute_code(x32):
    """Exact nearest level (fractions), exact ties to the lower index."""
    T = oracle.nf4_table()
    xf = Fraction(float(x32))
    dists = [abs(xf - Fraction(float(t))) for t in T]
    best = min(dists)
    return dists.index(best)


def _brute_quantize_block(w64):
    w = np.asarray(w64, dtype=np.float32)
    a = np.float32(max(abs(float(v)) for v in w))
    out = []
    for v in w:
        x = np.float32(0.0) if a == 0 else np.float32(v) / a  # IEEE fp32 divide
        out.append(_brute_code(x))
    return a, out


def test_codes_brute_force_random_blocks():
    rng = np.random.default_rng(123)
    W = (rng.standard_normal((4, 128), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    q = oracle.quantize_nf4_dq(W)
    flat = W.ravel()
    for b in range(flat.size // 64):
        a, codes = _brute_quantize_block(flat[64 * b:64 * b + 64])
        assert q["absmax"][b] == a
        assert list(q["code"][64 * b:64 * b + 64]) == codes


def test_codes_brute_force_dense_sweep():
    """Nearest-level decision on 20k values spread over [-1, 1] plus the
    fp32 neighbours of every midpoint."""
    rng = np.random.default_rng(7)
    xs = list(rng.uniform(-1, 1, 20000).astype(np.float32))
    T = oracle.nf4_table()
    for i in range(15):
        mid = np.float32((float(T[i]) + float(T[i + 1])) / 2)
        for v in (mid, np.nextafter(mid, np.float32(2)), np.nextafter(mid, np.float32(-2))):
            xs.append(np.float32(v))
    xs = np.array(xs, dtype=np.float32)
    # absmax 1.0 block layout: put the values in blocks whose first value is 1.0
    n = xs.size
    nblk = (n + 62) // 63
    W = np.zeros(nblk * 64, dtype=np.float32)
    for b in range(nblk):
        W[64 * b] = 1.0
        seg = xs[63 * b:63 * b + 63]
        W[64 * b + 1:64 * b + 1 + seg.size] = seg
    codes = nf4_dq.nearest_codes(W, nf4_dq.block_absmax(W))
    for b in range(nblk):
        seg = xs[63 * b:63 * b + 63]
        for i, v in enumerate(seg):
            assert codes[64 * b + 1 + i] == _brute_code(v)


def test_codes_exact_ties_go_to_lower_level():
    T = oracle.nf4_table()
    ties = []
    for i in range(15):
        mid = (float(T[i]) + float(T[i + 1])) / 2
        if float(np.float32(mid)) == mid:
            ties.append((i, np.float32(mid)))
    assert len(ties) >= 1
    W = np.zeros(64, dtype=np.float32)
    W[0] = 1.0
    for j, (_, v) in enumerate(ties):
        W[1 + j] = v
    codes = nf4_dq.nearest_codes(W, nf4_dq.block_absmax(W))
    for j, (i, _) in enumerate(ties):
        assert codes[1 + j] == i  # the lower of the two levels


def test_codes_special_values():
    W = np.zeros((1, 256), dtype=np.float32)
    W[0, 0:64] = np.linspace(-0.03, 0.05, 64, dtype=np.float32)  # +absmax at the end
    W[0, 64:128] = -np.abs(np.linspace(-0.04, 0.01, 64, dtype=np.float32))  # -absmax first
    W[0, 128:192] = -0.0  # all negative zero
    sub = np.float32(1e-42)
    W[0, 192:256] = np.array([sub * (i % 7 - 3) for i in range(64)], dtype=np.float32)
    q = oracle.quantize_nf4_dq(W)
    c = q["code"]
    assert c[63] == 15  # w == +absmax -> x == 1
    assert c[64] == 0   # w == -absmax -> x == -1
    assert np.all(c[128:192] == 7) and q["absmax"][2] == 0.0
    for b in range(4):
        a, ref = _brute_quantize_block(W.ravel()[64 * b:64 * b + 64])
        assert list(c[64 * b:64 * b + 64]) == ref


def test_pack_low_nibble_first_and_roundtrip():
    codes = np.array([1, 2, 15, 0, 7, 8], dtype=np.uint8)
    p = nf4_dq.pack_codes(codes)
    assert list(p) == [0x21, 0x0F, 0x87]
    assert list(nf4_dq.unpack_codes(p)) == list(codes)


# ------------------------------------------------------ double quantize ----

def test_double_quant_group_max_and_bound():
    rng = np.random.default_rng(5)
    a = np.abs(rng.standard_normal(300).astype(np.float32)) * np.float32(0.05)
    a = a.astype(np.float32)
    q8, s2 = nf4_dq.double_quantize(a)
    assert s2.size == 2  # 300 blocks -> one full group and a partial one
    for g, (lo, hi) in enumerate([(0, 256), (256, 300)]):
        seg = a[lo:hi]
        assert s2[g] == np.float32(np.float32(seg.max()) / np.float32(255.0))
        assert q8[lo + int(np.argmax(seg))] == 255
        for i in range(lo, hi):
            err = abs(Fraction(int(q8[i])) * Fraction(float(s2[g])) - Fraction(float(a[i])))
            assert err <= Fraction(float(s2[g])) * Fraction(1, 2) * (1 + Fraction(1, 1 << 20))


def test_double_quant_brute_force_over_256_codes():
    rng = np.random.default_rng(6)
    a = (np.abs(rng.standard_normal(256)) * 0.05).astype(np.float32)
    q8, s2 = nf4_dq.double_quantize(a)
    s = Fraction(float(s2[0]))
    for i in range(256):
        af = Fraction(float(a[i]))
        errs = [abs(q * s - af) for q in range(256)]
        best = min(errs)
        # the chosen code is optimal up to the fp32 rounding of a / s2
        assert errs[int(q8[i])] - best <= s * Fraction(1, 1 << 16)


def test_double_quant_zero_group():
    a = np.zeros(256, dtype=np.float32)
    q8, s2 = nf4_dq.double_quantize(a)
    assert s2[0] == 0 and np.all(q8 == 0)


# --------------------------------------------------------------- dequant ----

def test_bf16_rounding_matches_torch_and_ties():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x00018000,
                     0x7F7FFFFF, 0x00000001, 0x80000000], dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_from_f32(x), ref)
    assert list(oracle.bf16_bits_from_f32(ties[:4])) == [0x3F80, 0x3F82, 0xBF80, 0xBF82]


def test_dequant_zero_code_and_error_bound():
    d = synth.workload_linear("cfg1", 0)
    W = d["W"]
    q = oracle.quantize_nf4_dq(W)
    w, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], 256, 256)
    zero = q["code"].reshape(256, 256) == 7
    assert np.all(wb[zero] == 0)
    T = oracle.nf4_table().astype(np.float64)
    half_gap = np.max(np.diff(T)) / 2
    a = np.repeat(q["absmax"].astype(np.float64), 64).reshape(256, 256)
    s2 = np.repeat(q["absmax_scale"].astype(np.float64), 256 * 64)[:256 * 256].reshape(256, 256)
    err = np.abs(W.astype(np.float64) - w.astype(np.float64))
    assert np.all(err <= half_gap * a + s2 / 2 + 1e-6 * a)
    # the largest-magnitude weight of the group-max block comes back to ~itself
    g_blk = int(np.argmax(q["absmax"][:256]))
    blk = W.ravel()[64 * g_blk:64 * g_blk + 64]
    i = int(np.argmax(np.abs(blk)))
    assert abs(float(w.ravel()[64 * g_blk + i]) - float(blk[i])) <= 2e-7 * abs(float(blk[i]))


def test_nf4_beats_uniform_int4_on_normal_weights():
    """NF4 (with double quantization) has lower error than evenly spaced
    4-bit levels on normal weights ([P2] follow-up questions)."""
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((256, 1024), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    q = oracle.quantize_nf4_dq(W)
    w, _ = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], 256, 1024)
    e_nf4 = np.linalg.norm(w - W) / np.linalg.norm(W)
    blocks = W.reshape(-1, 64).astype(np.float64)
    a = np.abs(blocks).max(axis=1, keepdims=True)
    lv = np.linspace(-1, 1, 16)
    x = blocks / a
    idx = np.argmin(np.abs(x[..., None] - lv), axis=-1)
    wu = lv[idx] * a
    e_u = np.linalg.norm(wu - blocks) / np.linalg.norm(blocks)
    assert e_nf4 < e_u
    assert 0.08 < e_nf4 < 0.10


# --------------------------------------------------------------- storage ----

def test_storage_accounting_against_page_figures():
    f = _figures()
    n = 4096 * 4096
    bpw = oracle.bits_per_weight(n)
    assert bpw == 4.126953125
    assert round(bpw, 3) == f["bits_per_weight_dq"]["value"]
    assert oracle.bits_per_weight(n, double_quant=False) == f["bits_per_weight_no_dq"]["value"]
    assert oracle.bits_per_weight(n, double_quant=False) - 4 == f["absmax_overhead_bits_no_dq"]["value"]
    assert 100 * (oracle.bits_per_weight(n, False) - 4) / 4 == f["absmax_overhead_pct_of_4bit"]["value"]
    assert round(bpw - 4, 3) == f["overhead_bits_dq"]["value"]
    saving = oracle.bits_per_weight(n, False) - bpw
    assert round(saving, 2) == f["dq_saving_bits"]["value"]
    assert abs(saving * 8e9 / 8 / 1e6 - f["dq_saving_8b_MB"]["value"]) / 370 < 0.02
    assert round(saving * 65e9 / 8 / 1e9, 1) == f["dq_saving_65b_GB"]["value"]
    p7 = f["ledger_7b_params"]["value"]
    nb7 = p7 / 64
    codes_gb = p7 / 2 / 1e9
    consts_gb = (nb7 + 4 * nb7 / 256) / 1e9
    assert round(codes_gb, 2) == f["ledger_7b_codes_GB"]["value"]
    assert round(consts_gb, 2) == f["ledger_7b_constants_GB"]["value"]
    bpp = oracle.storage_bytes(n) / n
    assert round(bpp, 2) == f["bytes_per_param_8b"]["value"]
    assert round(7e9 * bpp / 1e9, 1) == f["quantized_7e9_GB"]["value"]
    # actual arrays have exactly the accounted sizes
    W = np.zeros((256, 16384), dtype=np.float32)
    q = oracle.quantize_nf4_dq(W)
    nbytes = q["codes"].nbytes + q["absmax_q8"].nbytes + q["absmax_scale"].nbytes
    assert nbytes == oracle.storage_bytes(W.size)


def test_3b_workload_shapes_match_page_adapter_count():
    f = _figures()["lora_params_3b_r16_M"]
    per_layer = sum(f["rank"] * (lin.k_in + lin.n_out) for lin in synth.LAYERS["3b"])
    assert round(per_layer * f["layers"] / 1e6, 1) == f["value"]


# --------------------------------------------------------------- forward ----

def _tiny(M=3, N=5, K=64, r=2, seed=0):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K))
    X = rng.standard_normal((M, K))
    A = rng.standard_normal((r, K))
    B = rng.standard_normal((N, r))
    dY = rng.standard_normal((M, N))
    return W, X, A, B, dY


def test_forward_B_zero_is_plain_product():
    W, X, A, B, _ = _tiny(M=4, N=6, K=128, r=3)
    Y, _ = oracle.linear_fwd(W, X, A, np.zeros_like(B), 6.0, 3)
    for m in range(4):
        for n in range(6):
            exact = math.fsum(float(X[m, k]) * float(W[n, k]) for k in range(128))
            assert abs(Y[m, n] - exact) <= 1e-12 * (1 + abs(exact))


def test_forward_equals_merged_weight():
    W, X, A, B, _ = _tiny(M=4, N=6, K=128, r=3)
    alpha, r = 6.0, 3
    Y, _ = oracle.linear_fwd(W, X, A, B, alpha, r)
    s = float(np.float32(alpha) / np.float32(r))
    merged = W + s * (B @ A)
    Ym = np.array([[math.fsum(X[m, k] * merged[n, k] for k in range(128)) for n in range(6)]
                   for m in range(4)])
    assert np.max(np.abs(Y - Ym)) <= 1e-12 * np.max(np.abs(Ym))


def test_forward_rank_zero_is_plain_product():
    W, X, _, _, dY = _tiny(M=3, N=4, K=64, r=1)
    A0 = np.zeros((0, 64))
    B0 = np.zeros((4, 0))
    Y, U = oracle.linear_fwd(W, X, A0, B0, 16.0, 0)
    assert U.shape == (3, 0)
    np.testing.assert_array_equal(Y, X @ W.T)
    dX, dA, dB = oracle.linear_bwd(W, X, dY, A0, B0, 16.0, 0)
    np.testing.assert_array_equal(dX, dY @ W)
    assert dA.shape == (0, 64) and dB.shape == (4, 0)


def test_forward_adapter_term_scales_with_alpha():
    W, X, A, B, _ = _tiny()
    Y0, _ = oracle.linear_fwd(W, X, A, np.zeros_like(B), 4.0, 2)
    Y1, _ = oracle.linear_fwd(W, X, A, B, 4.0, 2)
    Y2, _ = oracle.linear_fwd(W, X, A, B, 8.0, 2)
    np.testing.assert_allclose(Y2 - Y0, 2 * (Y1 - Y0), rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- backward ----

def test_backward_matches_finite_differences():
    W, X, A, B, dY = _tiny(M=3, N=5, K=64, r=2, seed=3)
    alpha, r = 4.0, 2
    dX, dA, dB = oracle.linear_bwd(W, X, dY, A, B, alpha, r)

    def loss(X_, A_, B_):
        Y, _ = oracle.linear_fwd(W, X_, A_, B_, alpha, r)
        return float(np.sum(dY * Y))

    h = 1e-3
    for arr, grad, name in ((X, dX, "X"), (A, dA, "A"), (B, dB, "B")):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += h
            mth = arr.copy(); mth[idx] -= h
            if name == "X":
                num[idx] = (loss(p, A, B) - loss(mth, A, B)) / (2 * h)
            elif name == "A":
                num[idx] = (loss(X, p, B) - loss(X, mth, B)) / (2 * h)
            else:
                num[idx] = (loss(X, A, p) - loss(X, A, mth)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-7, atol=1e-8, err_msg=name)


def test_backward_dx_equals_merged_weight_and_no_dw():
    W, X, A, B, dY = _tiny(M=4, N=6, K=64, r=3, seed=4)
    alpha, r = 9.0, 3
    out = oracle.linear_bwd(W, X, dY, A, B, alpha, r)
    assert len(out) == 3  # dX, dA, dB -- there is no dW
    s = float(np.float32(alpha) / np.float32(r))
    merged = W + s * (B @ A)
    np.testing.assert_allclose(out[0], dY @ merged, rtol=1e-12, atol=1e-12)


def test_oracle_accepts_bf16_bits_exactly():
    d = synth.workload_linear("cfg1", 0)
    q = oracle.quantize_nf4_dq(d["W"])
    _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], 256, 256)
    Y, _ = oracle.linear_fwd(wb, d["X"], d["A"], d["B"], d["alpha"], d["r"])
    Wf = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).double().numpy()
    Xf = torch.from_numpy(d["X"].view(np.int16)).view(torch.bfloat16).double().numpy()
    Af = torch.from_numpy(d["A"].view(np.int16)).view(torch.bfloat16).double().numpy()
    Bf = torch.from_numpy(d["B"].view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_allclose(Y, Xf @ Wf.T + 2.0 * (Xf @ Af.T) @ Bf.T, rtol=1e-12, atol=1e-12)


def test_quantize_groups_equals_full_quantize():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((96, 512), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    full = oracle.quantize_nf4_dq(W)
    nb = W.size // 64
    ng = (nb + 255) // 256
    part = oracle.quantize_groups(W.ravel(), range(ng))
    for g in range(ng):
        b0, b1 = 256 * g, min(nb, 256 * g + 256)
        assert np.array_equal(part[g]["codes"], full["codes"][b0 * 32:b1 * 32])
        assert np.array_equal(part[g]["absmax_q8"], full["absmax_q8"][b0:b1])
        assert part[g]["absmax_scale"][0] == full["absmax_scale"][g]


def test_adapter_grads_are_the_backward_ones():
    """``adapter_grads`` is the dA, dB that ``linear_bwd`` returns (pinned
    there by finite differences), and the backward rows of a token subset
    are the same rows of the full backward (each row of dX depends on its
    own token only), which the full-size GPU tests rely on."""
    W, X, A, B, dY = _tiny(M=6, N=8, K=128, r=3, seed=9)
    alpha, r = 6.0, 3
    dX, dA, dB = oracle.linear_bwd(W, X, dY, A, B, alpha, r)
    gA, gB = oracle.adapter_grads(X, dY, A, B, alpha, r)
    assert np.array_equal(gA, dA) and np.array_equal(gB, dB)
    rows = np.array([1, 4])
    dXs, _, _ = oracle.linear_bwd(W, X[rows], dY[rows], A, B, alpha, r)
    np.testing.assert_allclose(dXs, dX[rows], rtol=1e-13, atol=1e-13)
    Ys, _ = oracle.linear_fwd(W, X[rows], A, B, alpha, r)
    Y, _ = oracle.linear_fwd(W, X, A, B, alpha, r)
    np.testing.assert_allclose(Ys, Y[rows], rtol=1e-13, atol=1e-13)
