"""The bounds-checked build (libqlora_checked.so): every raw global store, and
every raw global load of caller-sized data, checks its index against the size
of the buffer it addresses; an access outside is skipped and counted
(qlora_debug_oob_count).  Each case runs the same inputs through the normal
library and the checked one: the outputs must agree bit for bit (the checks
change no arithmetic) and no access may have been out of range.

The shapes are the edge cases of every kernel's indexing: ragged row and
column tiles, a partial last group of 256 blocks, ranks that are not multiples
of 8 (or of 4), more than 32 ranks, no adapter, the few-token kernel at 1..16
tokens with and without its reduction split, split-reduction GEMM grids,
fp16, dropout, a backward that recomputes U~, and the allocation-free
forward.
"""

import os

import pytest
import torch

from bit_nf4_quantized_double_amd import qlora

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _same(a, b, what):
    if a is None and b is None:
        return
    assert a.dtype == b.dtype and a.shape == b.shape, what
    if a.dtype in (torch.bfloat16, torch.float16):
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    assert torch.equal(a, b), what


def _both(fn):
    """fn() with the normal library, then with the checked one; returns both
    results and the checked build's out-of-range count for the second run."""
    torch.cuda.synchronize()
    ref = fn()
    torch.cuda.synchronize()
    with qlora.library(qlora.LIB_CHECKED_PATH):
        qlora.debug_oob_count(reset=True)
        got = fn()
        torch.cuda.synchronize()
        oob = qlora.debug_oob_count(reset=True)
    return ref, got, oob


def _rand(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(dtype)


def test_normal_build_has_no_counter():
    _need_gpu()
    if os.environ.get("QLORA_LIBRARY") == "checked":
        pytest.skip("the whole run uses the bounds-checked build")
    with pytest.raises(RuntimeError, match="bounds-checked"):
        qlora.debug_oob_count()


CODEC_SHAPES = [(8, 64), (136, 192), (72, 768), (1024, 320)]  # partial last group of 256 blocks


@pytest.mark.parametrize("N,K", CODEC_SHAPES)
def test_codec_in_bounds(N, K):
    _need_gpu()
    W = _rand((N, K), N + K, 0.02, torch.float32)

    def run():
        w = qlora.quantize(W)
        wb = qlora.quantize(W.to(torch.bfloat16))
        out = [w.codes, w.absmax_q8, w.absmax_scale, wb.codes, wb.absmax_q8, wb.absmax_scale,
               qlora.dequant(w), qlora.dequant(w, dtype=torch.float16)]
        for fmt in qlora.FORMATS:
            fw = qlora.quantize_format(W, fmt)
            out += [fw.codes, fw.scales, qlora.dequant_format(fw)]
        return out

    ref, got, oob = _both(run)
    for i, (a, b) in enumerate(zip(ref, got)):
        _same(a, b, f"codec output {i}")
    assert oob == 0


MERGE_SHAPES = [(256, 256, 8), (200, 320, 3), (136, 192, 17), (96, 640, 33), (64, 128, 64), (72, 256, 0),
                (520, 768, 16), (264, 320, 40), (40, 192, 6)]


@pytest.mark.parametrize("N,K,r", MERGE_SHAPES)
def test_merge_in_bounds(N, K, r):
    _need_gpu()
    W = _rand((N, K), 3 * N + K, 0.02, torch.float32)
    w = qlora.quantize(W)
    A = _rand((max(r, 1), K), 5 + r, K ** -0.5)[:r].contiguous() if r else None
    B = _rand((N, max(r, 1)), 7 + r, 0.01)[:, :r].contiguous() if r else None
    ref, got, oob = _both(lambda: qlora.merge(w, A, B, r, 2.0 * max(r, 1)))
    _same(ref, got, "merged weight")
    assert oob == 0


# (M, N, K, r, dtype, dropout_p, pass U to the backward)
LINEAR_CASES = [
    (1, 256, 256, 8, torch.bfloat16, 0.0, True),
    (3, 136, 192, 5, torch.bfloat16, 0.0, False),      # few-token, ragged, U~ recomputed
    (7, 520, 768, 3, torch.float16, 0.0, True),
    (8, 1024, 4096, 16, torch.bfloat16, 0.0, False),   # few-token with a reduction split
    (5, 4104, 1088, 17, torch.float16, 0.0, False),    # few-token with 16 waves, ragged, U~ recomputed
    (16, 1024, 8192, 40, torch.bfloat16, 0.05, True),  # more than 32 ranks, dropout
    (16, 8, 64, 0, torch.bfloat16, 0.0, True),         # no adapter, one tile
    (17, 136, 192, 5, torch.bfloat16, 0.0, False),     # GEMM path, ragged, U~ recomputed
    (130, 1024, 2048, 0, torch.bfloat16, 0.0, True),   # split-reduction grid, no adapter
    (300, 2048, 2048, 16, torch.bfloat16, 0.0, True),  # split-reduction grid
    (300, 520, 960, 7, torch.float16, 0.05, False),    # fp16 with dropout, U~ recomputed
    (513, 1032, 1088, 64, torch.bfloat16, 0.0, True),  # ragged everything, the largest rank
]


@pytest.mark.parametrize("M,N,K,r,dt,p,pass_u", LINEAR_CASES)
def test_linear_in_bounds(M, N, K, r, dt, p, pass_u):
    _need_gpu()
    seed = M + 3 * N + 7 * K + r
    W = _rand((N, K), seed, 0.02, torch.float32)
    w = qlora.quantize(W)
    X = _rand((M, K), seed + 1, 1.0, dt)
    dY = _rand((M, N), seed + 2, 1.0, dt)
    A = _rand((max(r, 1), K), seed + 3, K ** -0.5, dt)[:r].contiguous() if r else None
    B = _rand((N, max(r, 1)), seed + 4, 0.01, dt)[:, :r].contiguous() if r else None
    alpha = 2.0 * max(r, 1)

    def run():
        Y, U = qlora.linear_fwd(w, X, A, B, r, alpha, dropout_p=p, seed=11)
        dX, dA, dB = qlora.linear_bwd(w, X, dY, A, B, r, alpha, U if pass_u else None, dropout_p=p, seed=11)
        return Y, U, dX, dA, dB

    ref, got, oob = _both(run)
    for a, b, what in zip(ref, got, ("Y", "U~", "dX", "dA", "dB")):
        _same(a, b, what)
    assert oob == 0


@pytest.mark.parametrize("M,N,K,r", [(4, 264, 320, 8), (40, 520, 768, 16)])
def test_noalloc_forward_in_bounds(M, N, K, r):
    _need_gpu()
    W = _rand((N, K), 9, 0.02, torch.float32)
    w = qlora.quantize(W)
    X = _rand((M, K), 10)
    A = _rand((r, K), 11, K ** -0.5)
    B = _rand((N, r), 12, 0.01)

    def run():
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        U = torch.empty((M, r), dtype=torch.bfloat16, device="cuda")
        return qlora.linear_fwd_noalloc(w, X, A, B, r, 16.0, Y, U)

    ref, got, oob = _both(run)
    _same(ref[0], got[0], "Y")
    _same(ref[1], got[1], "U~")
    assert oob == 0


def test_fewtoken_u_finalize_fallback_matches_staged():
    """When the down projection's partials do not fit in LDS beside the
    staged block scales (4 tokens, 5120 x 64512, rank 64: 32 KB of scales and
    32 KB of partials), the few-token launcher rounds them with a finalize
    pass first.  U~ depends only on X, A and the split of k_in, so a narrow
    weight (1024 outputs: the kernel adds the staged partials itself) must
    give the same U~ bit for bit; and the wide case runs in bounds."""
    _need_gpu()
    M, K, r, alpha = 4, 64512, 64, 128.0
    X = _rand((M, K), 21)
    A = _rand((r, K), 22, K ** -0.5)
    outs = {}
    for N in (1024, 5120):
        w = qlora.quantize(_rand((N, K), 23 + N, 0.02, torch.float32))
        B = _rand((N, r), 24, 0.01)
        ref, got, oob = _both(lambda: qlora.linear_fwd(w, X, A, B, r, alpha))
        _same(ref[0], got[0], f"Y ({N} outputs)")
        _same(ref[1], got[1], f"U~ ({N} outputs)")
        assert oob == 0
        outs[N] = ref[1]
        del w
    _same(outs[1024], outs[5120], "U~ through the finalize pass against U~ formed in the kernel")
