"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (see the header of include/qlora.h for the contract):
* codes, absmax_q8, absmax_scale and the dequantized bf16 weight: bit-exact;
* Y, dX, dA, dB: relative Frobenius error <= 5e-3 and every element within
  2e-2 * max|ref| of the fp64 oracle.

Small shapes span several tiles with ragged tails; full-size shapes (the 7B
decoder layer, 70B few-token and dequant shapes) are compared on sampled
rows / groups the oracle computes one by one, plus exact full-tensor checks
where the oracle is cheap (dA, dB).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_double_amd import qlora, synth

pytestmark = pytest.mark.gpu

REL_FRO = 5e-3
ELEM = 2e-2


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t):
    if t.dtype == torch.bfloat16:
        return oracle.f64_from_bf16_bits(host_bits(t))
    return t.double().cpu().numpy()


def check_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    nref = np.linalg.norm(ref)
    err = np.linalg.norm(got - ref)
    rel = err / nref if nref > 0 else err
    worst = np.max(np.abs(got - ref)) if ref.size else 0.0
    bound = ELEM * (np.max(np.abs(ref)) if ref.size else 0.0)
    assert rel <= REL_FRO, f"{what}: rel Frobenius {rel:.3e} > {REL_FRO}"
    assert worst <= bound + (0 if nref > 0 else 1e-30), f"{what}: max |err| {worst:.3e} > {bound:.3e}"


def gpu_quantize(W):
    return qlora.quantize(torch.from_numpy(np.ascontiguousarray(W)).cuda())


def check_codec_exact(w, q, W_bf_ref=None):
    assert np.array_equal(w.codes.cpu().numpy(), q["codes"]), "codes"
    assert np.array_equal(w.absmax_q8.cpu().numpy(), q["absmax_q8"]), "absmax_q8"
    assert np.array_equal(w.absmax_scale.cpu().numpy().view(np.uint32),
                          q["absmax_scale"].view(np.uint32)), "absmax_scale"
    if W_bf_ref is not None:
        got = host_bits(qlora.dequant(w))
        assert np.array_equal(got, W_bf_ref), "dequantized bf16"


# ------------------------------------------------------------------ codec ----

def test_table_matches_oracle():
    t = np.array(qlora.nf4_table(), dtype=np.float32)
    assert np.array_equal(t.view(np.uint32), oracle.nf4_table().view(np.uint32))


def test_quantize_dequant_single_linear_bit_exact():
    _need_gpu()
    d = synth.workload_linear("cfg1", 0)
    q = oracle.quantize_nf4_dq(d["W"])
    _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], 256, 256)
    w = gpu_quantize(d["W"])
    torch.cuda.synchronize()
    check_codec_exact(w, q, wb)


def _edge_weight():
    """24 x 832 = 312 blocks: a full group and a partial one, with crafted
    blocks (exact ties, +-absmax, zeros, -0.0, subnormals, tiny blocks)."""
    rng = np.random.default_rng(77)
    W = (rng.standard_normal((24, 832), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    flat = W.ravel()
    T = oracle.nf4_table()
    ties = [np.float32((float(T[i]) + float(T[i + 1])) / 2) for i in range(15)]
    blk = np.zeros(64, dtype=np.float32)
    blk[0] = 1.0
    for j, v in enumerate(ties):
        blk[1 + j] = v
        blk[17 + j] = np.nextafter(v, np.float32(2))
        blk[33 + j] = np.nextafter(v, np.float32(-2))
    blk[49] = -1.0
    flat[0:64] = blk                   # crafted ties (absmax 1)
    flat[64:128] = 0.0                 # all zero block
    flat[128:192] = -0.0               # all negative zero
    flat[192:256] = np.float32(1e-42) * np.arange(-32, 32, dtype=np.float32)  # subnormals
    flat[256:320] = np.linspace(-0.05, 0.03, 64, dtype=np.float32)            # -absmax first
    flat[320:384] *= np.float32(1e-6)  # block far below the group max (q8 small)
    flat[256 * 64:257 * 64] = 0.0      # first block of the partial group
    return flat.reshape(24, 832)


def test_quantize_edge_cases_bit_exact():
    _need_gpu()
    W = _edge_weight()
    q = oracle.quantize_nf4_dq(W)
    _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], 24, 832)
    check_codec_exact(gpu_quantize(W), q, wb)


def test_quantize_zero_group_bit_exact():
    _need_gpu()
    W = np.zeros((64, 512), dtype=np.float32)  # 512 blocks = 2 groups
    W[32:, :] = np.random.default_rng(3).standard_normal((32, 512)).astype(np.float32) * 0.02
    q = oracle.quantize_nf4_dq(W)
    assert q["absmax_scale"][0] == 0
    _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], 64, 512)
    check_codec_exact(gpu_quantize(W), q, wb)


@pytest.mark.parametrize("fmt", ["nf4_dq", "nf4", "int4_dq", "int4"])
def test_quantize_near_threshold_bit_exact(fmt):
    """Blocks whose absmax is not a power of two (so 1 / absmax is inexact),
    holding weights at fp32(theta_i * a), fp32(T_i * a) and 1..4 ulps around
    them for every threshold of the format's table; under the evenly spaced
    tables also the block whose quotient underflows to 0 beside a zero
    threshold.  Codes, block scales and the decoded bf16 weight bit-exact."""
    from oracle import formats
    import crafted
    _need_gpu()
    rng = np.random.default_rng(17)
    table = formats.format_table(fmt)
    blocks = crafted.near_threshold_blocks(table, crafted.absmax_set(rng, 60), rng)
    if fmt.startswith("int4"):
        blocks = np.concatenate([blocks, crafted.zero_threshold_underflow_block()[None, :]])
    W = np.ascontiguousarray(crafted.as_weight(blocks))
    n, k = W.shape
    q = formats.quantize_format(W, fmt)
    _, wb = formats.dequant_format(q, n, k, fmt)
    w = qlora.quantize_format(torch.from_numpy(W).cuda(), fmt)
    out = qlora.dequant_format(w)
    torch.cuda.synchronize()
    assert np.array_equal(w.codes.cpu().numpy(), q["codes"]), "codes"
    if fmt.endswith("_dq"):
        assert np.array_equal(w.scales.cpu().numpy(), q["absmax_q8"]), "q8"
        assert np.array_equal(w.absmax_scale.cpu().numpy().view(np.uint32),
                              q["absmax_scale"].view(np.uint32)), "s2"
    else:
        assert np.array_equal(w.scales.cpu().numpy().view(np.uint32), q["absmax"].view(np.uint32)), "absmax"
    assert np.array_equal(host_bits(out), wb), "dequantized bf16"
    if fmt == "nf4_dq":  # the main codec entry point on the same weight
        qm = oracle.quantize_nf4_dq(W)
        check_codec_exact(gpu_quantize(W), qm, wb)


def test_quantize_bf16_near_threshold_bit_exact():
    """The bf16-input codec (re-quantizing a merged weight) on bf16 weights a
    few bf16 ulps around every NF4 threshold of bf16 absmaxes that are not
    powers of two: bit-exact against the oracle's codec of the widened
    values."""
    import crafted
    _need_gpu()
    rng = np.random.default_rng(19)
    blocks = crafted.near_threshold_blocks(oracle.nf4_table(), crafted.absmax_set(rng, 60), rng, bf16=True)
    W = np.ascontiguousarray(crafted.as_weight(blocks))
    bits = oracle.bf16_bits_from_f32(W)
    Wf = (bits.astype(np.uint32) << 16).view(np.float32)  # the padding blocks rounded too
    q = oracle.quantize_nf4_dq(Wf)
    _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], *W.shape)
    w = qlora.quantize(dev_bf16(bits))
    torch.cuda.synchronize()
    check_codec_exact(w, q, wb)


@pytest.mark.parametrize("workload,index", [("7b", 4), ("7b", 6), ("70b", 0), ("70b", 1)])
def test_quantize_dequant_full_size_sampled_groups(workload, index):
    """Full-size weights quantized and dequantized on the GPU; 64 sampled
    DQ groups (plus the first and last) checked bit-exact by the oracle."""
    _need_gpu()
    lin = synth.LAYERS[workload][index]
    rng = synth.rng_for(workload, index)
    W = synth.draw(rng, (lin.n_out, lin.k_in), 0.02)
    w = gpu_quantize(W)
    wbf = qlora.dequant(w)
    torch.cuda.synchronize()
    nb = W.size // 64
    ng = (nb + 255) // 256
    groups = sorted(set([0, ng - 1] + list(np.random.default_rng(1).choice(ng, 64, replace=False))))
    part = oracle.quantize_groups(W.ravel(), groups)
    codes = w.codes.cpu().numpy()
    q8 = w.absmax_q8.cpu().numpy()
    s2 = w.absmax_scale.cpu().numpy()
    wflat = wbf.view(-1)
    for g in groups:
        b0, b1 = 256 * g, min(nb, 256 * g + 256)
        ref = part[g]
        assert np.array_equal(codes[b0 * 32:b1 * 32], ref["codes"]), g
        assert np.array_equal(q8[b0:b1], ref["absmax_q8"]), g
        assert s2[g].view(np.uint32) == ref["absmax_scale"][0].view(np.uint32), g
        _, wb = oracle.dequant(ref["codes"], ref["absmax_q8"], ref["absmax_scale"], 1, (b1 - b0) * 64,
                               first_block=b0)
        got = host_bits(wflat[b0 * 64:b1 * 64])
        assert np.array_equal(got, wb.ravel()), g


# ----------------------------------------------------------- fp16 instance ----

def dev_f16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).cuda()


def f64h(t):
    if t.dtype == torch.float16:
        return oracle.f16.f64_from_f16_bits(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


def test_f16_dequant_bit_exact():
    _need_gpu()
    rng = np.random.default_rng(8)
    for W in (_edge_weight(), (rng.standard_normal((136, 1984), dtype=np.float32) * np.float32(0.02))):
        W = np.ascontiguousarray(W, dtype=np.float32)
        q = oracle.quantize_nf4_dq(W)
        _, hb = oracle.f16.dequant_f16(q["codes"], q["absmax_q8"], q["absmax_scale"], *W.shape)
        w = gpu_quantize(W)
        out = qlora.dequant(w, dtype=torch.float16)
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), hb)


F16_SHAPES = [
    (16, 256, 256, 8, 16.0),
    (100, 200, 192, 16, 32.0),
    (300, 520, 640, 64, 128.0),
    (17, 136, 320, 17, 5.0),
    (257, 384, 512, 0, 0.0),
    (5, 1000, 384, 16, 32.0),     # few-token kernel
    (16, 4104, 320, 64, 128.0),   # few-token kernel, partial tile
    (130, 1024, 2048, 16, 32.0),  # split reduction in both products
    (16, 8192, 8192, 16, 32.0),   # few-token split across workgroups; dX split 4 ways
    (3, 4104, 1088, 16, 32.0),    # few-token kernel with 16 waves
]


@pytest.mark.parametrize("M,N,K,r,alpha", F16_SHAPES)
def test_f16_forward_backward_parity(M, N, K, r, alpha):
    _need_gpu()
    rng = np.random.default_rng(M * 5 + N + 1)
    d = synth.linear_inputs(N, K, M, r, rng, dtype="f16")
    q = oracle.quantize_nf4_dq(d["W"])
    _, hb = oracle.f16.dequant_f16(q["codes"], q["absmax_q8"], q["absmax_scale"], N, K)
    Wh = oracle.f16.f64_from_f16_bits(hb)
    Xh, dYh = oracle.f16.f64_from_f16_bits(d["X"]), oracle.f16.f64_from_f16_bits(d["dY"])
    Ah = oracle.f16.f64_from_f16_bits(d["A"]) if r > 0 else np.zeros((0, K))
    Bh = oracle.f16.f64_from_f16_bits(d["B"]) if r > 0 else np.zeros((N, 0))
    w = gpu_quantize(d["W"])
    X, dY = dev_f16(d["X"]), dev_f16(d["dY"])
    A = dev_f16(d["A"]) if r > 0 else None
    B = dev_f16(d["B"]) if r > 0 else None
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    assert Y.dtype == torch.float16
    dX, dA, dB = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U)
    torch.cuda.synchronize()
    Yr, Ur = oracle.linear_fwd(Wh, Xh, Ah, Bh, alpha, r)
    dXr, dAr, dBr = oracle.linear_bwd(Wh, Xh, dYh, Ah, Bh, alpha, r)
    check_close(f64h(Y), Yr, "Y fp16")
    check_close(f64h(dX), dXr, "dX fp16")
    if r > 0 and alpha != 0:
        check_close(f64h(U), oracle.lora_scale(alpha, r) * Ur, "U~ fp16")
        check_close(f64(dA), dAr, "dA fp16")
        check_close(f64(dB), dBr, "dB fp16")


def test_f16_full_7b_linear_sampled():
    """The 7B gate linear at 2048 tokens in fp16: Y and dX on 32 sampled
    rows, dA and dB in full, against the oracle's fp16 weight."""
    _need_gpu()
    d = synth.workload_linear("7b", 4, dtype="f16")
    N, K, M, r, alpha = d["n_out"], d["k_in"], d["m"], d["r"], d["alpha"]
    q = oracle.quantize_nf4_dq(d["W"])
    _, hb = oracle.f16.dequant_f16(q["codes"], q["absmax_q8"], q["absmax_scale"], N, K)
    w = gpu_quantize(d["W"])
    X, dY, A, B = dev_f16(d["X"]), dev_f16(d["dY"]), dev_f16(d["A"]), dev_f16(d["B"])
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    dX, dA, dB = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(2).choice(M, 32, replace=False))
    Wh = oracle.f16.f64_from_f16_bits(hb)
    Xh, dYh = oracle.f16.f64_from_f16_bits(d["X"]), oracle.f16.f64_from_f16_bits(d["dY"])
    Ah, Bh = oracle.f16.f64_from_f16_bits(d["A"]), oracle.f16.f64_from_f16_bits(d["B"])
    Yr, _ = oracle.linear_fwd(Wh, Xh[rows], Ah, Bh, alpha, r)
    dXr, _, _ = oracle.linear_bwd(Wh, Xh[rows], dYh[rows], Ah, Bh, alpha, r)
    check_close(f64h(Y)[rows], Yr, "Y fp16 sampled")
    check_close(f64h(dX)[rows], dXr, "dX fp16 sampled")
    dAr, dBr = oracle.adapter_grads(Xh, dYh, Ah, Bh, alpha, r)
    check_close(f64(dA), dAr, "dA fp16")
    check_close(f64(dB), dBr, "dB fp16")


# ------------------------------------------------------- format variants ----

@pytest.mark.parametrize("fmt", ["nf4_dq", "nf4", "int4_dq", "int4"])
def test_format_variants_bit_exact(fmt):
    """Every storage-format variant: codes, block scales and the decoded bf16
    weight bit-exact against the oracle, on the edge-case weight (ties,
    +-absmax, zeros, -0.0, subnormals, a partial group) and a normal one
    spanning several groups."""
    from oracle import formats
    _need_gpu()
    rng = np.random.default_rng(31)
    for W in (_edge_weight(), (rng.standard_normal((136, 1984), dtype=np.float32) * np.float32(0.02))):
        W = np.ascontiguousarray(W, dtype=np.float32)
        n, k = W.shape
        q = formats.quantize_format(W, fmt)
        _, wb = formats.dequant_format(q, n, k, fmt)
        w = qlora.quantize_format(torch.from_numpy(W).cuda(), fmt)
        out = qlora.dequant_format(w)
        torch.cuda.synchronize()
        assert np.array_equal(w.codes.cpu().numpy(), q["codes"]), "codes"
        if fmt.endswith("_dq"):
            assert np.array_equal(w.scales.cpu().numpy(), q["absmax_q8"]), "q8"
            assert np.array_equal(w.absmax_scale.cpu().numpy().view(np.uint32),
                                  q["absmax_scale"].view(np.uint32)), "s2"
        else:
            assert np.array_equal(w.scales.cpu().numpy().view(np.uint32), q["absmax"].view(np.uint32)), "absmax"
        assert np.array_equal(host_bits(out), wb), "dequantized bf16"


def test_format_nf4_dq_equals_main_codec():
    _need_gpu()
    d = synth.workload_linear("cfg1", 0)
    Wt = torch.from_numpy(d["W"]).cuda()
    a = qlora.quantize(Wt)
    b = qlora.quantize_format(Wt, "nf4_dq")
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.absmax_q8, b.scales)
    assert torch.equal(a.absmax_scale, b.absmax_scale)
    assert torch.equal(qlora.dequant(a).view(torch.int16), qlora.dequant_format(b).view(torch.int16))


# ------------------------------------------------------- forward/backward ----

SHAPES = [
    # (M, N, K, r, alpha)
    (16, 256, 256, 8, 16.0),      # the single-linear case
    (100, 200, 192, 16, 32.0),    # ragged M, N and K tiles
    (1, 64, 64, 1, 1.0),
    (17, 136, 320, 17, 5.0),      # rank not a multiple of 16
    (300, 520, 640, 64, 128.0),   # maximum rank
    (257, 384, 512, 0, 0.0),      # no adapter
    (33, 128, 128, 16, 0.0),      # alpha = 0
    (130, 1024, 2048, 16, 32.0),  # several full tiles; split reduction (fwd 4, dX 2)
    (300, 2048, 2048, 16, 32.0),  # split reduction, 4 splits in both products
    (50, 1000, 1088, 16, 32.0),   # 2 uneven forward splits (9 + 8 steps), ragged tails
    (77, 136, 2240, 17, 5.0),     # forward split 4 ways, last split one step short
    (40, 2200, 640, 16, 32.0),    # dX split 4 ways (9, 9, 9, 8 steps), ragged last step
    (64, 264, 4096, 8, 16.0),     # forward split 8 ways over a partial column tile
    (16, 2048, 1024, 16, 32.0),   # few-token forward; dX (GEMM) split 4 ways at 16 tokens
    (1, 1024, 2048, 8, 16.0),     # one token: dX split 2 ways over a single row
    (40, 512, 8192, 16, 32.0),    # row passes at their most splits: 8 partial sums in the GEMM prologue
    (70, 328, 6400, 24, 48.0),    # 6 row-pass splits, the last one chunk short; 24 ranks
    (20, 64, 64, 16, 32.0),       # GEMM path over a single 64-deep step (half a 128-wide chunk)
    (40, 8192, 512, 16, 32.0),    # the row pass over dY at 8 splits: V~ from 8 partials in the dX prologue
]


def _case(M, N, K, r, seed):
    rng = np.random.default_rng(seed)
    d = synth.linear_inputs(N, K, M, r, rng)
    q = oracle.quantize_nf4_dq(d["W"])
    _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], N, K)
    return d, q, wb


def _dev_inputs(d, r):
    X = dev_bf16(d["X"])
    A = dev_bf16(d["A"]) if r > 0 else None
    B = dev_bf16(d["B"]) if r > 0 else None
    dY = dev_bf16(d["dY"])
    return X, A, B, dY


@pytest.mark.parametrize("M,N,K,r,alpha", SHAPES)
def test_forward_parity(M, N, K, r, alpha):
    _need_gpu()
    d, q, wb = _case(M, N, K, r, seed=M * 7 + N)
    w = gpu_quantize(d["W"])
    X, A, B, _ = _dev_inputs(d, r)
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    torch.cuda.synchronize()
    Yr, Ur = oracle.linear_fwd(wb, d["X"], d["A"], d["B"], alpha, r)
    check_close(f64(Y), Yr, "Y")
    if r > 0:
        s = oracle.lora_scale(alpha, r)
        check_close(f64(U), s * Ur, "U~")
    # forward without U_out (workspace path) gives the same bits
    Y2, _ = qlora.linear_fwd(w, X, A, B, r, alpha, return_u=False)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))


# Few-token forward (M <= 16 runs a dedicated kernel): partial 16-row tiles
# (n_out % 16 == 8), half 128-wide chunks (k_in % 128 == 64), ranks that are
# not multiples of 8, and tile counts that select every work split (1 to 8
# tiles per wave, 1 to 8 waves per reduction), a full 16-token tile with a
# single tile per workgroup, a long reduction at M = 1, and ranks 1 and 17.
FEW_SHAPES = [
    (1, 8, 64, 0, 0.0),
    (2, 264, 192, 3, 6.0),
    (5, 1000, 384, 16, 32.0),
    (16, 4104, 320, 64, 128.0),
    (7, 40000, 128, 8, 16.0),
    (16, 28672, 64, 16, 32.0),
    (3, 32768, 64, 5, 8.0),
    (16, 2048, 1088, 32, 64.0),
    (11, 512, 4096, 0, 0.0),
    (16, 136, 2048, 16, 32.0),
    (1, 8192, 8192, 16, 32.0),
    (4, 520, 640, 17, 34.0),
    (9, 1032, 960, 1, 2.0),
    (16, 8192, 8192, 16, 32.0),   # reduction split 4 ways across workgroups (8 tiles each)
    (9, 8192, 8256, 17, 34.0),    # split 17 + 17 + 17 + 14 chunks, half a chunk at the end
    (6, 5000, 1088, 17, 34.0),    # 16 waves, 2 tiles each; most waves hold only padding chunks
]


@pytest.mark.parametrize("M,N,K,r,alpha", FEW_SHAPES)
def test_few_token_forward_parity(M, N, K, r, alpha):
    _need_gpu()
    d, q, wb = _case(M, N, K, r, seed=M * 13 + N + K)
    w = gpu_quantize(d["W"])
    X, A, B, _ = _dev_inputs(d, r)
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    torch.cuda.synchronize()
    Yr, Ur = oracle.linear_fwd(wb, d["X"], d["A"], d["B"], alpha, r)
    check_close(f64(Y), Yr, "Y")
    if r > 0:
        check_close(f64(U), oracle.lora_scale(alpha, r) * Ur, "U~")
    Y2, _ = qlora.linear_fwd(w, X, A, B, r, alpha, return_u=False)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))


@pytest.mark.parametrize("M,N,K,r,alpha", SHAPES)
def test_backward_parity(M, N, K, r, alpha):
    _need_gpu()
    d, q, wb = _case(M, N, K, r, seed=M * 11 + K)
    w = gpu_quantize(d["W"])
    X, A, B, dY = _dev_inputs(d, r)
    _, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    dX, dA, dB = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U)
    torch.cuda.synchronize()
    dXr, dAr, dBr = oracle.linear_bwd(wb, d["X"], d["dY"], d["A"], d["B"], alpha, r)
    check_close(f64(dX), dXr, "dX")
    if r > 0:
        if alpha == 0:
            assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0
        else:
            check_close(f64(dA), dAr, "dA")
            check_close(f64(dB), dBr, "dB")
        # U recomputed inside the backward gives the same bits
        dX2, dA2, dB2 = qlora.linear_bwd(w, X, dY, A, B, r, alpha, None)
        torch.cuda.synchronize()
        assert torch.equal(dX.view(torch.int16), dX2.view(torch.int16))
        assert torch.equal(dA, dA2) and torch.equal(dB, dB2)


def _tiled_bytes(M, R):
    """The fragment-tiled activation copy a GEMM reads (r = 0: the only
    required workspace)."""
    return -(-M // 32) * 32 * (-(-R // 64) * 64) * 2


def test_split_reduction_room_is_optional():
    """Few output tiles: with room in the workspace the products split the
    reduction; with only the required part (r = 0: the tiled activations)
    they run unsplit; with less the call is refused.  Both results match the
    oracle."""
    _need_gpu()
    M, N, K, r, alpha = 130, 1024, 2048, 0, 0.0
    fwd_req, bwd_req = _tiled_bytes(M, K), _tiled_bytes(M, N)
    assert qlora.workspace_bytes(qlora.QLORA_OP_FWD, M, N, K, r) > fwd_req
    assert qlora.workspace_bytes(qlora.QLORA_OP_BWD, M, N, K, r) > bwd_req
    d, q, wb = _case(M, N, K, r, seed=5)
    w = gpu_quantize(d["W"])
    X, _, _, dY = _dev_inputs(d, r)
    Ys, _ = qlora.linear_fwd(w, X, None, None, r, alpha)
    dXs, _, _ = qlora.linear_bwd(w, X, dY, None, None, r, alpha)
    L = qlora.lib()
    cw = w._c()
    Yu = torch.empty_like(Ys)
    dXu = torch.empty_like(dXs)
    wsf = torch.empty(fwd_req, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(bwd_req, dtype=torch.uint8, device="cuda")
    assert L.qlora_linear_fwd(ctypes.byref(cw), X.data_ptr(), M, None, None, 0, 0.0, Yu.data_ptr(), None,
                              wsf.data_ptr(), fwd_req - 256, qlora._stream()) == -4  # QLORA_ERR_WORKSPACE
    assert L.qlora_linear_fwd(ctypes.byref(cw), X.data_ptr(), M, None, None, 0, 0.0, Yu.data_ptr(), None,
                              wsf.data_ptr(), fwd_req, qlora._stream()) == 0
    assert L.qlora_linear_bwd(ctypes.byref(cw), X.data_ptr(), dY.data_ptr(), M, None, None, 0, 0.0, None,
                              dXu.data_ptr(), None, None, wsb.data_ptr(), bwd_req - 256, qlora._stream()) == -4
    assert L.qlora_linear_bwd(ctypes.byref(cw), X.data_ptr(), dY.data_ptr(), M, None, None, 0, 0.0, None,
                              dXu.data_ptr(), None, None, wsb.data_ptr(), bwd_req, qlora._stream()) == 0
    torch.cuda.synchronize()
    Yr, _ = oracle.linear_fwd(wb, d["X"], d["A"], d["B"], alpha, r)
    dXr, _, _ = oracle.linear_bwd(wb, d["X"], d["dY"], d["A"], d["B"], alpha, r)
    for got, ref, what in ((Ys, Yr, "Y split"), (Yu, Yr, "Y unsplit"), (dXs, dXr, "dX split"),
                           (dXu, dXr, "dX unsplit")):
        check_close(f64(got), ref, what)


def test_backward_deterministic_and_weight_untouched():
    _need_gpu()
    d, q, wb = _case(513, 1024, 768, 16, seed=5)
    w = gpu_quantize(d["W"])
    before = [t.clone() for t in (w.codes, w.absmax_q8, w.absmax_scale)]
    X, A, B, dY = _dev_inputs(d, 16)
    Y1, U = qlora.linear_fwd(w, X, A, B, 16, 32.0)
    r1 = qlora.linear_bwd(w, X, dY, A, B, 16, 32.0, U)
    Y2, _ = qlora.linear_fwd(w, X, A, B, 16, 32.0)
    r2 = qlora.linear_bwd(w, X, dY, A, B, 16, 32.0, U)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(r1[0].view(torch.int16), r2[0].view(torch.int16))
    assert torch.equal(r1[1], r2[1]) and torch.equal(r1[2], r2[2])
    for b, t in zip(before, (w.codes, w.absmax_q8, w.absmax_scale)):
        assert torch.equal(b, t)


def test_empty_tokens():
    _need_gpu()
    d, q, wb = _case(1, 128, 128, 8, seed=9)
    w = gpu_quantize(d["W"])
    X = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    A, B = dev_bf16(d["A"]), dev_bf16(d["B"])
    Y, U = qlora.linear_fwd(w, X, A, B, 8, 16.0)
    dA = torch.full((8, 128), 7.0, device="cuda")
    dB = torch.full((128, 8), 7.0, device="cuda")
    dX, dA, dB = qlora.linear_bwd(w, X, torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"),
                                  A, B, 8, 16.0, None, dA=dA, dB=dB)
    torch.cuda.synchronize()
    assert Y.shape == (0, 128) and dX.shape == (0, 128)
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) == 0


def test_autograd_module_matches_entry_points():
    _need_gpu()
    d, q, wb = _case(64, 256, 256, 16, seed=21)
    Wt = torch.from_numpy(d["W"]).cuda()
    A = dev_bf16(d["A"]).float()
    B = dev_bf16(d["B"]).float()
    mod = qlora.QLoRALinear(Wt, r=16, alpha=32.0, A=A, B=B)
    X = dev_bf16(d["X"]).requires_grad_(True)
    Y = mod(X)
    dY = dev_bf16(d["dY"])
    Y.backward(dY)
    torch.cuda.synchronize()
    Yr, _ = oracle.linear_fwd(wb, d["X"], d["A"], d["B"], 32.0, 16)
    dXr, dAr, dBr = oracle.linear_bwd(wb, d["X"], d["dY"], d["A"], d["B"], 32.0, 16)
    check_close(f64(Y.detach()), Yr, "module Y")
    check_close(f64(X.grad), dXr, "module dX")
    check_close(f64(mod.A.grad.float()), dAr, "module dA")
    check_close(f64(mod.B.grad.float()), dBr, "module dB")


@pytest.mark.parametrize("p", [0.0, 0.05])
def test_autograd_module_fp16(p):
    """The nn.Module in the fp16 instance (adapter held in fp16, X and the
    incoming gradient fp16), without and with LoRA dropout: its results are
    bit for bit those of the entry points, and match the oracle's fp16
    forward and backward."""
    _need_gpu()
    M, N, K, r, alpha = 64, 256, 256, 16, 32.0
    rng = np.random.default_rng(23)
    d = synth.linear_inputs(N, K, M, r, rng, dtype="f16")
    Wt = torch.from_numpy(d["W"]).cuda()
    A16, B16 = dev_f16(d["A"]), dev_f16(d["B"])
    mod = qlora.QLoRALinear(Wt, r=r, alpha=alpha, A=A16.float(), B=B16.float(), lora_dropout=p,
                            dtype=torch.float16)
    assert mod.A.dtype == torch.float16 and mod.B.dtype == torch.float16
    X = dev_f16(d["X"]).requires_grad_(True)
    torch.manual_seed(5)
    Y = mod(X)
    dY = dev_f16(d["dY"])
    Y.backward(dY)
    torch.cuda.synchronize()
    assert Y.dtype == torch.float16 and X.grad.dtype == torch.float16
    # the seed the module drew for this step
    torch.manual_seed(5)
    seed = int(torch.randint(0, 2**62, (1,)).item()) if p else 0
    Ye, Ue = qlora.linear_fwd(mod.w, X.detach(), A16, B16, r, alpha, dropout_p=p, seed=seed)
    dXe, dAe, dBe = qlora.linear_bwd(mod.w, X.detach(), dY, A16, B16, r, alpha, Ue, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    assert torch.equal(Y.detach().view(torch.int16), Ye.view(torch.int16))
    assert torch.equal(X.grad.view(torch.int16), dXe.view(torch.int16))
    assert torch.equal(mod.A.grad, dAe.to(torch.float16)) and torch.equal(mod.B.grad, dBe.to(torch.float16))
    q = oracle.quantize_nf4_dq(d["W"])
    _, hb = oracle.f16.dequant_f16(q["codes"], q["absmax_q8"], q["absmax_scale"], N, K)
    Wh = oracle.f16.f64_from_f16_bits(hb)
    Xh, dYh = oracle.f16.f64_from_f16_bits(d["X"]), oracle.f16.f64_from_f16_bits(d["dY"])
    Ah, Bh = oracle.f16.f64_from_f16_bits(d["A"]), oracle.f16.f64_from_f16_bits(d["B"])
    mask = oracle.dropout_mask(M, K, p, seed) if p else np.ones((M, K), dtype=bool)
    Yr, _ = oracle.linear_fwd_dropout(Wh, Xh, Ah, Bh, alpha, r, mask, p)
    dXr, dAr, dBr = oracle.linear_bwd_dropout(Wh, Xh, dYh, Ah, Bh, alpha, r, mask, p)
    check_close(f64h(Y.detach()), Yr, "module Y fp16")
    check_close(f64h(X.grad), dXr, "module dX fp16")
    check_close(f64(dAe), dAr, "module dA fp16")
    check_close(f64(dBe), dBr, "module dB fp16")


F16_DROP_SHAPES = [
    # GEMM path with ragged tiles; few-token path; dX split 4 ways
    (100, 200, 192, 16, 32.0, 0.05),
    (5, 1000, 384, 16, 32.0, 0.05),
    (300, 2048, 2048, 17, 34.0, 0.1),
]


@pytest.mark.parametrize("M,N,K,r,alpha,p", F16_DROP_SHAPES)
def test_f16_dropout_forward_backward_parity(M, N, K, r, alpha, p):
    """LoRA dropout in the fp16 instance against the oracle's dropped layer
    on the fp16 values."""
    _need_gpu()
    rng = np.random.default_rng(M * 3 + N)
    d = synth.linear_inputs(N, K, M, r, rng, dtype="f16")
    q = oracle.quantize_nf4_dq(d["W"])
    _, hb = oracle.f16.dequant_f16(q["codes"], q["absmax_q8"], q["absmax_scale"], N, K)
    Wh = oracle.f16.f64_from_f16_bits(hb)
    Xh, dYh = oracle.f16.f64_from_f16_bits(d["X"]), oracle.f16.f64_from_f16_bits(d["dY"])
    Ah, Bh = oracle.f16.f64_from_f16_bits(d["A"]), oracle.f16.f64_from_f16_bits(d["B"])
    w = gpu_quantize(d["W"])
    X, dY, A, B = dev_f16(d["X"]), dev_f16(d["dY"]), dev_f16(d["A"]), dev_f16(d["B"])
    seed = _drop_seed(M, N) ^ 0xF16
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha, dropout_p=p, seed=seed)
    dX, dA, dB = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    mask = oracle.dropout_mask(M, K, p, seed)
    Yr, Ur = oracle.linear_fwd_dropout(Wh, Xh, Ah, Bh, alpha, r, mask, p)
    dXr, dAr, dBr = oracle.linear_bwd_dropout(Wh, Xh, dYh, Ah, Bh, alpha, r, mask, p)
    check_close(f64h(Y), Yr, "Y fp16 dropout")
    check_close(f64h(U), oracle.lora_scale(alpha, r) * Ur, "U~ fp16 dropout")
    check_close(f64h(dX), dXr, "dX fp16 dropout")
    check_close(f64(dA), dAr, "dA fp16 dropout")
    check_close(f64(dB), dBr, "dB fp16 dropout")


# ------------------------------------------------------------ LoRA dropout ----

DROP_SHAPES = [
    # (M, N, K, r, alpha, p): GEMM path with ragged tiles, the few-token path,
    # a rank that is not a multiple of 8, a heavy drop rate
    (100, 200, 192, 16, 32.0, 0.05),
    (300, 520, 640, 64, 128.0, 0.05),
    (5, 1000, 384, 16, 32.0, 0.05),
    (17, 136, 320, 17, 5.0, 0.3),
    (257, 384, 512, 8, 16.0, 0.5),
    (300, 2048, 2048, 16, 32.0, 0.1),  # dX with the reduction split 4 ways
    (9, 8192, 8256, 17, 34.0, 0.1),    # few-token forward split across workgroups
]


def _drop_seed(M, N):
    return (0x5EED << 40) | (M * 1009 + N)  # exercises both key words


@pytest.mark.parametrize("M,N,K,r,alpha,p", DROP_SHAPES)
def test_dropout_forward_backward_parity(M, N, K, r, alpha, p):
    _need_gpu()
    d, q, wb = _case(M, N, K, r, seed=M * 17 + N + K)
    w = gpu_quantize(d["W"])
    X, A, B, dY = _dev_inputs(d, r)
    seed = _drop_seed(M, N)
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha, dropout_p=p, seed=seed)
    dX, dA, dB = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    mask = oracle.dropout_mask(M, K, p, seed)
    Yr, Ur = oracle.linear_fwd_dropout(wb, d["X"], d["A"], d["B"], alpha, r, mask, p)
    dXr, dAr, dBr = oracle.linear_bwd_dropout(wb, d["X"], d["dY"], d["A"], d["B"], alpha, r, mask, p)
    s = oracle.lora_scale(alpha, r)
    check_close(f64(Y), Yr, "Y")
    check_close(f64(U), s * Ur, "U~")
    check_close(f64(dX), dXr, "dX")
    check_close(f64(dA), dAr, "dA")
    check_close(f64(dB), dBr, "dB")
    # the backward regenerates the mask when it recomputes U~
    dX2, dA2, dB2 = qlora.linear_bwd(w, X, dY, A, B, r, alpha, None, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), dX2.view(torch.int16))
    assert torch.equal(dA, dA2) and torch.equal(dB, dB2)


def test_dropout_p_zero_equals_plain_entry_points():
    _need_gpu()
    M, N, K, r, alpha = 100, 200, 192, 16, 32.0
    d, q, wb = _case(M, N, K, r, seed=3)
    w = gpu_quantize(d["W"])
    X, A, B, dY = _dev_inputs(d, r)
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    g = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U)
    L = qlora.lib()
    cw = w._c()
    Y0 = torch.empty_like(Y)
    U0 = torch.empty_like(U)
    ws = qlora.new_workspace(qlora.QLORA_OP_BWD, M, N, K, r, "cuda")
    st = L.qlora_linear_fwd_dropout(ctypes.byref(cw), X.data_ptr(), M, A.data_ptr(), B.data_ptr(), r, alpha,
                                    0.0, 99, Y0.data_ptr(), U0.data_ptr(), ws.data_ptr(), ws.numel(),
                                    qlora._stream())
    assert st == 0
    dX0 = torch.empty_like(g[0])
    dA0 = torch.empty_like(g[1])
    dB0 = torch.empty_like(g[2])
    st = L.qlora_linear_bwd_dropout(ctypes.byref(cw), X.data_ptr(), dY.data_ptr(), M, A.data_ptr(),
                                    B.data_ptr(), r, alpha, 0.0, 99, U0.data_ptr(), dX0.data_ptr(),
                                    dA0.data_ptr(), dB0.data_ptr(), ws.data_ptr(), ws.numel(), qlora._stream())
    assert st == 0
    torch.cuda.synchronize()
    for a, b in ((Y, Y0), (U, U0), (g[0], dX0)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(g[1], dA0) and torch.equal(g[2], dB0)


def test_dropout_mask_bit_exact_in_every_kernel():
    """The kept / dropped pattern itself, bit for bit, against the oracle's
    mask.  W = 0 makes dX = keep * (V~ A) exactly (the dX GEMM's mask at
    every (m, k)); one-hot rows of X (row m has its single 1 at column k_m,
    all distinct) make U~[m, :] = s_d keep(m, k_m) A[:, k_m] and
    dA[:, k_m] = keep(m, k_m) V~[m, :] (the rowdot's and the coldot's
    mask)."""
    _need_gpu()
    M, N, K, r, alpha, p = 256, 128, 512, 16, 32.0, 0.3
    rng = np.random.default_rng(12)
    seed = 0xABCDEF0123456789
    W = np.zeros((N, K), dtype=np.float32)
    w = gpu_quantize(W)
    km = (np.arange(M) * 7 + 3) % K
    Xh = np.zeros((M, K), dtype=np.float32)
    Xh[np.arange(M), km] = 1.0
    A = rng.standard_normal((r, K)).astype(np.float32)
    B = rng.standard_normal((N, r)).astype(np.float32)
    dY = rng.standard_normal((M, N)).astype(np.float32)
    Xb, Ab, Bb, dYb = (synth.to_bf16_bits(t) for t in (Xh, A, B, dY))
    X, Ad, Bd, dYd = (dev_bf16(t) for t in (Xb, Ab, Bb, dYb))
    Y, U = qlora.linear_fwd(w, X, Ad, Bd, r, alpha, dropout_p=p, seed=seed)
    dX, dA, dB = qlora.linear_bwd(w, X, dYd, Ad, Bd, r, alpha, U, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    mask = oracle.dropout_mask(M, K, p, seed)
    assert 0.6 < mask.mean() < 0.8
    Af = oracle.f64_from_bf16_bits(Ab)
    Vt = f64(dYd) @ oracle.f64_from_bf16_bits(Bb)  # nonzero rows almost surely
    # dX GEMM: nonzero exactly where kept (V~ A is nonzero everywhere here)
    assert np.all(np.abs(Vt @ Af) > 0)
    assert np.array_equal(f64(dX) != 0, mask)
    # rowdot (U~): row m is zero iff (m, k_m) was dropped
    row_kept = mask[np.arange(M), km]
    assert np.array_equal(np.any(f64(U) != 0, axis=1), row_kept)
    # coldot (dA): column k_m is zero iff (m, k_m) was dropped
    assert np.array_equal(np.any(f64(dA)[:, km] != 0, axis=0), row_kept)
    other = np.setdiff1d(np.arange(K), km)
    assert np.count_nonzero(f64(dA)[:, other]) == 0


# ------------------------------------------------- full-size, sampled rows ----

@pytest.mark.parametrize("index", [0, 4, 6])
def test_full_7b_linear_sampled(index):
    """A 7B decoder-layer linear at M = 2048 (the timed configuration):
    Y and dX on 48 sampled rows, dA and dB in full."""
    _need_gpu()
    d = synth.workload_linear("7b", index)
    N, K, M, r, alpha = d["n_out"], d["k_in"], d["m"], d["r"], d["alpha"]
    q = oracle.quantize_nf4_dq(d["W"])
    _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], N, K)
    w = gpu_quantize(d["W"])
    X, A, B, dY = _dev_inputs(d, r)
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    dX, dA, dB = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U)
    torch.cuda.synchronize()
    check_codec_exact(w, q)
    rows = np.sort(np.random.default_rng(index).choice(M, 48, replace=False))
    # the oracle's forward and backward on the sampled token rows (each row
    # of Y and dX depends on its own token only), its adapter gradients over
    # every token
    Yr, _ = oracle.linear_fwd(wb, d["X"][rows], d["A"], d["B"], alpha, r)
    check_close(f64(Y)[rows], Yr, "Y rows")
    dXr, _, _ = oracle.linear_bwd(wb, d["X"][rows], d["dY"][rows], d["A"], d["B"], alpha, r)
    check_close(f64(dX)[rows], dXr, "dX rows")
    dAr, dBr = oracle.adapter_grads(d["X"], d["dY"], d["A"], d["B"], alpha, r)
    check_close(f64(dA), dAr, "dA")
    check_close(f64(dB), dBr, "dB")


def _full_linear_sampled(workload, index, nrows):
    """One linear of a full-size decoder layer at its token count: Y and dX on
    sampled rows, dA and dB in full, all against the oracle's quantization of
    the whole weight."""
    d = synth.workload_linear(workload, index)
    N, K, M, r, alpha = d["n_out"], d["k_in"], d["m"], d["r"], d["alpha"]
    q = oracle.quantize_nf4_dq(d["W"])
    _, wb = oracle.dequant(q["codes"], q["absmax_q8"], q["absmax_scale"], N, K)
    w = gpu_quantize(d["W"])
    X, A, B, dY = _dev_inputs(d, r)
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    dX, dA, dB = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U)
    torch.cuda.synchronize()
    check_codec_exact(w, q)
    rows = np.sort(np.random.default_rng(index + 100).choice(M, nrows, replace=False))
    Yr, _ = oracle.linear_fwd(wb, d["X"][rows], d["A"], d["B"], alpha, r)
    dXr, _, _ = oracle.linear_bwd(wb, d["X"][rows], d["dY"][rows], d["A"], d["B"], alpha, r)
    dAr, dBr = oracle.adapter_grads(d["X"], d["dY"], d["A"], d["B"], alpha, r)
    check_close(f64(Y)[rows], Yr, f"{workload} Y rows")
    check_close(f64(dX)[rows], dXr, f"{workload} dX rows")
    check_close(f64(dA), dAr, f"{workload} dA")
    check_close(f64(dB), dBr, f"{workload} dB")


@pytest.mark.parametrize("index", [0, 1, 4, 6])  # q, k (3072 -> 1024), gate, down
def test_full_3b_linear_sampled(index):
    """3B-class decoder layer (width 3072, MLP 8192) at 2048 tokens."""
    _need_gpu()
    _full_linear_sampled("3b", index, 32)


@pytest.mark.parametrize("index", [0, 1, 4, 6])  # q, k (4096 -> 1024), gate (-> 14336), down
def test_full_8b_linear_sampled(index):
    """8B-class decoder layer at batch 4 x seq 2048 = 8192 tokens (32 row
    blocks: every band of the tile order)."""
    _need_gpu()
    _full_linear_sampled("8b", index, 24)


@pytest.mark.parametrize("index,M", [(0, 1), (0, 4), (0, 16), (1, 1), (1, 16)])
def test_few_token_70b_sampled_columns(index, M):
    """The 70B gate (8192 -> 28672) and down (28672 -> 8192) weights at M = 1,
    4, 16: 64 sampled output columns against rows of W the oracle quantizes
    group by group."""
    _need_gpu()
    d = synth.workload_linear("70b", index, m=M, with_grad=False)
    N, K, r, alpha = d["n_out"], d["k_in"], d["r"], d["alpha"]
    w = gpu_quantize(d["W"])
    X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
    Y, _ = qlora.linear_fwd(w, X, A, B, r, alpha)
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(M + 10 * index).choice(N, 64, replace=False))
    flat = d["W"].ravel()
    bpr = K // 64  # blocks per row
    Wrows = []
    for n in cols:
        b0 = n * bpr
        groups = sorted(set(range(b0 // 256, (b0 + bpr - 1) // 256 + 1)))
        part = oracle.quantize_groups(flat, groups)
        codes = np.concatenate([part[g]["codes"] for g in groups])
        q8 = np.concatenate([part[g]["absmax_q8"] for g in groups])
        s2 = np.concatenate([part[g]["absmax_scale"] for g in groups])
        gb0 = groups[0] * 256
        _, wbr = oracle.dequant(codes, q8, s2, 1, codes.size * 2, first_block=gb0)
        Wrows.append(wbr.ravel()[(b0 - gb0) * 64:(b0 - gb0 + bpr) * 64])
    # the oracle's forward on the sampled output features: their rows of the
    # dequantized weight and of B
    Yr, _ = oracle.linear_fwd(np.stack(Wrows), d["X"], d["A"], d["B"][cols], alpha, r)
    check_close(f64(Y)[:, cols], Yr, "Y sampled columns")


def test_few_token_u_finalize_fallback_against_oracle():
    """4 tokens on a 5120 x 64512 weight at rank 64: the down projection's
    partials (32 KB) do not fit in LDS beside the staged block scales
    (32 KB), so the launcher rounds them with a finalize pass before the
    few-token kernel.  U~ in full and 64 sampled output columns of Y against
    the oracle."""
    _need_gpu()
    M, N, K, r, alpha = 4, 5120, 64512, 64, 128.0
    d = synth.linear_inputs(N, K, M, r, np.random.default_rng(64512), with_grad=False)
    w = gpu_quantize(d["W"])
    X, A, B = dev_bf16(d["X"]), dev_bf16(d["A"]), dev_bf16(d["B"])
    Y, U = qlora.linear_fwd(w, X, A, B, r, alpha)
    torch.cuda.synchronize()
    del w
    cols = np.sort(np.random.default_rng(5).choice(N, 64, replace=False))
    flat = d["W"].ravel()
    bpr = K // 64
    Wrows = []
    for n in cols:
        b0 = n * bpr
        groups = sorted(set(range(b0 // 256, (b0 + bpr - 1) // 256 + 1)))
        part = oracle.quantize_groups(flat, groups)
        codes = np.concatenate([part[g]["codes"] for g in groups])
        q8 = np.concatenate([part[g]["absmax_q8"] for g in groups])
        s2 = np.concatenate([part[g]["absmax_scale"] for g in groups])
        gb0 = groups[0] * 256
        _, wbr = oracle.dequant(codes, q8, s2, 1, codes.size * 2, first_block=gb0)
        Wrows.append(wbr.ravel()[(b0 - gb0) * 64:(b0 - gb0 + bpr) * 64])
    Yr, Ur = oracle.linear_fwd(np.stack(Wrows), d["X"], d["A"], d["B"][cols], alpha, r)
    check_close(f64(Y)[:, cols], Yr, "Y sampled columns")
    check_close(f64(U), oracle.lora_scale(alpha, r) * Ur, "U~")


# ------------------------------------------------------ merge, re-quantize ----

MERGE_SHAPES = [
    # (N, K, r, alpha): ragged 64-row and 128-column tiles, ranks that are not
    # multiples of 8, more than 32 ranks, no adapter
    (256, 256, 8, 16.0),
    (200, 320, 3, 6.0),
    (136, 192, 17, 5.0),
    (96, 640, 33, 66.0),
    (64, 128, 64, 128.0),
    (72, 256, 0, 0.0),
    (1024, 4096, 16, 32.0),
    (520, 768, 16, 32.0),     # a workgroup with one partial 16-row block
    (264, 320, 40, 80.0),
]


def _near_tie(exact, wb, A, B, s, r):
    """Elements whose exact merged value lies closer to a bf16 rounding
    boundary than the fp32 evaluation error of W + s * sum_j B A can reach:
    (r + 2) * 2^-24 * (|W| + s * sum_j |B A|).  There the GPU may round to
    either neighbour."""
    b = oracle.bf16_bits_from_f64(exact)
    g = np.abs(oracle.f64_from_bf16_bits(b))
    # bf16 spacing at g, on the side of the exact value (just below a power
    # of two the spacing is half)
    e = np.floor(np.log2(np.where(g > 0, g, 1.0)))
    sp = 2.0 ** (e - 7)
    sp = np.where((np.abs(exact) < g) & (g == 2.0 ** e), sp / 2, sp)
    d = np.abs(np.abs(np.abs(exact) - g) - sp / 2)
    return d <= _merge_err_bound(wb, A, B, s, r), sp


def _merge_err_bound(wb, A, B, s, r):
    """Bound on the fp32 evaluation error of W + s * sum_j B A (MFMA sums and
    one multiply-add): (r + 2) * 2^-23 * (|W| + s * sum_j |B A|)."""
    mag = np.abs(oracle.f64_from_bf16_bits(wb))
    if r > 0:
        mag = mag + s * (np.abs(oracle.f64_from_bf16_bits(B)) @ np.abs(oracle.f64_from_bf16_bits(A)))
    return (r + 2) * 2.0 ** -23 * mag


@pytest.mark.parametrize("N,K,r,alpha", MERGE_SHAPES)
def test_merge_and_requantize_parity(N, K, r, alpha):
    _need_gpu()
    d, q, wb = _case(4, N, K, r, seed=N + 3 * K + r)
    w = gpu_quantize(d["W"])
    A = dev_bf16(d["A"]) if r > 0 else None
    B = dev_bf16(d["B"]) if r > 0 else None
    Wm = qlora.merge(w, A, B, r, alpha)
    torch.cuda.synchronize()
    exact, ref = oracle.merge(wb, d["A"], d["B"], alpha, r)
    got = host_bits(Wm)
    sc = oracle.lora_scale(alpha, r)
    tie, sp = _near_tie(exact, wb, d["A"], d["B"], sc, r)
    bad = (got != ref) & ~tie
    assert not bad.any(), (f"{bad.sum()} of {bad.size} differ; first at {np.argwhere(bad)[:4].tolist()}: "
                           f"got {got[bad][:4]} ref {ref[bad][:4]} exact {exact[bad][:4]}")
    # near a rounding boundary: within the evaluation error plus one spacing
    if tie.any():
        err = np.abs(oracle.f64_from_bf16_bits(got[tie]) - exact[tie])
        assert np.all(err <= _merge_err_bound(wb, d["A"], d["B"], sc, r)[tie] + sp[tie])
    # re-quantize on the GPU (bf16 input) and in the oracle: bit-exact on the
    # groups whose merged inputs agree bit for bit
    w2 = qlora.quantize(Wm)
    torch.cuda.synchronize()
    q2 = oracle.requantize(ref, N, K)
    same_blk = (got.reshape(-1, 64) == ref.reshape(-1, 64)).all(axis=1)
    codes = w2.codes.cpu().numpy().reshape(-1, 32)
    assert np.array_equal(codes[same_blk], q2["codes"].reshape(-1, 32)[same_blk])
    nb = same_blk.size
    grp_ok = np.array([same_blk[g * 256:(g + 1) * 256].all() for g in range((nb + 255) // 256)])
    q8 = w2.absmax_q8.cpu().numpy()
    blk_grp = np.arange(nb) // 256
    assert np.array_equal(q8[grp_ok[blk_grp]], q2["absmax_q8"][grp_ok[blk_grp]])
    assert np.array_equal(w2.absmax_scale.cpu().numpy()[grp_ok], q2["absmax_scale"][grp_ok])
    # the drift the pages warn about: the re-quantized weight vs the merged one
    drift = oracle.requant_drift(ref, q2, N, K)
    assert 0.0 <= drift < 0.2


def _check_merged_rows(got, exact, ref, wb, A, B, sc, r):
    tie, sp = _near_tie(exact, wb, A, B, sc, r)
    bad = (got != ref) & ~tie
    assert not bad.any(), (f"{bad.sum()} of {bad.size} differ; first at {np.argwhere(bad)[:4].tolist()}: "
                           f"got {got[bad][:4]} ref {ref[bad][:4]} exact {exact[bad][:4]}")
    if tie.any():
        err = np.abs(oracle.f64_from_bf16_bits(got[tie]) - exact[tie])
        assert np.all(err <= _merge_err_bound(wb, A, B, sc, r)[tie] + sp[tie])


def test_merge_and_requantize_70b_gate_sampled_rows():
    """Full-size merge (28672 x 8192, rank 16, the launch the bandwidth figure
    times) and re-quantization: 16 sampled row pairs -- each pair is one
    double-quantization group -- against the oracle's quantize, merge and
    re-quantize of those rows."""
    _need_gpu()
    d = synth.workload_linear("70b", 0, m=1, with_grad=False)
    N, K, r, alpha = d["n_out"], d["k_in"], d["r"], d["alpha"]
    assert (2 * K) % (64 * 256) == 0  # a row pair is exactly one group
    w = gpu_quantize(d["W"])
    Wm = qlora.merge(w, dev_bf16(d["A"]), dev_bf16(d["B"]), r, alpha)
    w2 = qlora.quantize(Wm)
    torch.cuda.synchronize()
    pairs = sorted(set([0, N // 2 - 1] + list(np.random.default_rng(7).choice(N // 2, 14, replace=False))))
    rows = np.array([2 * p + i for p in pairs for i in (0, 1)])
    part = oracle.quantize_groups(d["W"].ravel(), pairs)
    wb = np.concatenate([oracle.dequant(part[g]["codes"], part[g]["absmax_q8"], part[g]["absmax_scale"], 2, K,
                                        first_block=256 * g)[1] for g in pairs])
    exact, ref = oracle.merge(wb, d["A"], d["B"][rows], alpha, r)
    got = host_bits(Wm[torch.from_numpy(rows).cuda()])
    sc = oracle.lora_scale(alpha, r)
    _check_merged_rows(got, exact, ref, wb, d["A"], d["B"][rows], sc, r)
    codes = w2.codes.cpu().numpy()
    q8 = w2.absmax_q8.cpu().numpy()
    s2 = w2.absmax_scale.cpu().numpy()
    for i, g in enumerate(pairs):
        gref, gget = ref[2 * i:2 * i + 2], got[2 * i:2 * i + 2]
        if not np.array_equal(gref, gget):
            continue  # a near-tie rounded the other way: inputs differ
        q2 = oracle.requantize(gref, 2, K)
        assert np.array_equal(codes[g * 8192:(g + 1) * 8192], q2["codes"]), g
        assert np.array_equal(q8[g * 256:(g + 1) * 256], q2["absmax_q8"]), g
        assert s2[g].view(np.uint32) == q2["absmax_scale"][0].view(np.uint32), g


def test_quantize_into_preallocated_buffers():
    """quantize(W, out=w) overwrites w's buffers with the same result as a
    fresh quantization, also when they held another weight's codes."""
    _need_gpu()
    d = synth.workload_linear("cfg1", 0)
    q = oracle.quantize_nf4_dq(d["W"])
    w = gpu_quantize(np.ascontiguousarray(d["W"][::-1]))  # other contents, same shape
    got = qlora.quantize(torch.from_numpy(np.ascontiguousarray(d["W"])).cuda(), out=w)
    torch.cuda.synchronize()
    assert got is w
    check_codec_exact(w, q)


def test_quantize_bf16_input_bit_exact():
    _need_gpu()
    d = synth.workload_linear("cfg1", 0)
    Wb = synth.to_bf16_bits(d["W"])
    q = oracle.quantize_nf4_dq(oracle.f64_from_bf16_bits(Wb).astype(np.float32).reshape(d["W"].shape))
    w = qlora.quantize(dev_bf16(Wb).reshape(d["W"].shape))
    torch.cuda.synchronize()
    check_codec_exact(w, q)


# ------------------------------------------------------------ HIP graphs ----

@pytest.mark.parametrize("M,N,K,r,alpha", [(300, 2048, 2048, 16, 32.0), (16, 8192, 8192, 16, 32.0)])
def test_graph_capture_replays_match_eager(M, N, K, r, alpha):
    """The library allocates nothing and issues only kernels, so a forward +
    backward can be captured in a HIP graph.  Every replay (with eager work
    and synchronisation in between) must reproduce the eager results bit for
    bit, the split-reduction passes included."""
    _need_gpu()
    d, q, wb = _case(M, N, K, r, seed=M + N + K)
    w = gpu_quantize(d["W"])
    X, A, B, dY = _dev_inputs(d, r)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    U = torch.empty((M, r), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((r, K), dtype=torch.float32, device="cuda")
    dB = torch.empty((N, r), dtype=torch.float32, device="cuda")
    wsf = qlora.new_workspace(qlora.QLORA_OP_FWD, M, N, K, r, "cuda")
    wsb = qlora.new_workspace(qlora.QLORA_OP_BWD, M, N, K, r, "cuda")

    def run():
        qlora.linear_fwd(w, X, A, B, r, alpha, Y=Y, U=U, ws=wsf)
        qlora.linear_bwd(w, X, dY, A, B, r, alpha, U, dX=dX, dA=dA, dB=dB, ws=wsb)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (Y, U, dX, dA, dB)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (Y, U, dX, dA, dB):
            t.fill_(float(rep + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((Y, U, dX, dA, dB), ref, ("Y", "U~", "dX", "dA", "dB")):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), (rep, what)
    check_close(f64(ref[0]), oracle.linear_fwd(wb, d["X"], d["A"], d["B"], alpha, r)[0], "Y (graph case)")
