"""Host-side checks of the C ABI (CPU only, no GPU work).

The library must load, export every function include/qlora.h declares, build
the same NF4 table as the oracle, size workspaces, and reject bad arguments
on the host before anything is enqueued.  The bad-argument calls below pass
fake (never dereferenced) device pointers: each returns an error before any
HIP call.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from bit_nf4_quantized_double_amd import qlora

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")

OK, INVALID, SHAPE, ALIGN, WORKSPACE = 0, -1, -2, -3, -4
FAKE = 0x10000  # aligned, never dereferenced
FAKE_MIS = 0x10002


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qlora.LIB_PATH):
        from bit_nf4_quantized_double_amd import build
        build.build(verbose=False)
    return qlora.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported(L):
    names = _declared_functions()
    assert {"qlora_quantize_nf4_dq", "qlora_dequant", "qlora_linear_fwd", "qlora_linear_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_checked_build_exports_the_same_symbols(L):
    """The bounds-checked twin library is built beside the normal one and has
    the same entry points; the normal build reports that it has no counter
    (without touching the device)."""
    assert os.path.exists(qlora.LIB_CHECKED_PATH)
    C = ctypes.CDLL(qlora.LIB_CHECKED_PATH)
    for n in _declared_functions():
        assert hasattr(C, n), n
    N = ctypes.CDLL(os.path.join(os.path.dirname(qlora.LIB_CHECKED_PATH), "libqlora.so"))
    n = ctypes.c_uint64(7)
    N.qlora_debug_oob_count.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert N.qlora_debug_oob_count(ctypes.byref(n), 0) == INVALID
    assert N.qlora_debug_oob_count(None, 0) == INVALID
    assert n.value == 7


def test_library_table_matches_oracle_bitwise(L):
    t = np.array(qlora.nf4_table(), dtype=np.float32)
    assert np.array_equal(t.view(np.uint32), oracle.nf4_table().view(np.uint32))


def test_status_strings(L):
    for s in (OK, INVALID, SHAPE, ALIGN, WORKSPACE, -5):
        assert L.qlora_status_string(s).decode().startswith("QLORA_")


def _w(n_out=64, k_in=64, codes=FAKE, q8=FAKE, s2=FAKE):
    return qlora._CWeight(n_out, k_in, codes, q8, s2)


def test_weight_validation(L):
    s = 0
    assert L.qlora_dequant(None, FAKE, s) == INVALID
    assert L.qlora_dequant(ctypes.byref(_w(k_in=100)), FAKE, s) == SHAPE
    assert L.qlora_dequant(ctypes.byref(_w(n_out=12)), FAKE, s) == SHAPE
    assert L.qlora_dequant(ctypes.byref(_w(n_out=-8)), FAKE, s) == INVALID
    assert L.qlora_dequant(ctypes.byref(_w(codes=None)), FAKE, s) == INVALID
    assert L.qlora_dequant(ctypes.byref(_w(codes=FAKE_MIS)), FAKE, s) == ALIGN
    assert L.qlora_dequant(ctypes.byref(_w()), None, s) == INVALID
    assert L.qlora_dequant(ctypes.byref(_w()), FAKE_MIS, s) == ALIGN
    assert b"aligned" in L.qlora_last_error()
    # empty weight is a no-op
    assert L.qlora_dequant(ctypes.byref(_w(n_out=0)), None, s) == OK
    # more than 2^32 weights
    assert L.qlora_dequant(ctypes.byref(_w(n_out=1 << 20, k_in=1 << 13)), FAKE, s) == SHAPE


def test_quantize_validation(L):
    assert L.qlora_quantize_nf4_dq(None, 64, 64, FAKE, FAKE, FAKE, 0) == INVALID
    assert L.qlora_quantize_nf4_dq(FAKE, 64, 96, FAKE, FAKE, FAKE, 0) == SHAPE
    assert L.qlora_quantize_nf4_dq(FAKE_MIS, 64, 64, FAKE, FAKE, FAKE, 0) == ALIGN
    assert L.qlora_quantize_nf4_dq(FAKE, 0, 64, None, None, None, 0) == OK


def test_forward_validation(L):
    w = ctypes.byref(_w())
    f = L.qlora_linear_fwd
    assert f(w, FAKE, 16, FAKE, FAKE, -1, 2.0, FAKE, FAKE, None, 0, 0) == INVALID
    assert f(w, FAKE, 16, FAKE, FAKE, 65, 2.0, FAKE, FAKE, None, 0, 0) == SHAPE
    assert f(w, FAKE, 16, None, FAKE, 8, 2.0, FAKE, FAKE, None, 0, 0) == INVALID
    assert f(w, FAKE, -1, FAKE, FAKE, 8, 2.0, FAKE, FAKE, None, 0, 0) == INVALID
    assert f(w, None, 16, FAKE, FAKE, 8, 2.0, FAKE, FAKE, None, 0, 0) == INVALID
    assert f(w, FAKE_MIS, 16, FAKE, FAKE, 8, 2.0, FAKE, FAKE, None, 0, 0) == ALIGN
    assert f(w, FAKE, 16, FAKE, FAKE_MIS, 8, 2.0, FAKE, FAKE, None, 0, 0) == ALIGN
    # no U_out and no workspace
    assert f(w, FAKE, 16, FAKE, FAKE, 8, 2.0, FAKE, None, None, 0, 0) == WORKSPACE
    need = L.qlora_workspace_bytes(1, 16, 64, 64, 8)
    assert need >= 16 * 8 * 2
    assert f(w, FAKE, 16, FAKE, FAKE, 8, 2.0, FAKE, None, FAKE, need - 1, 0) == WORKSPACE
    # M == 0 is a no-op
    assert f(w, None, 0, FAKE, FAKE, 8, 2.0, None, None, None, 0, 0) == OK


def test_backward_validation(L):
    w = ctypes.byref(_w())
    b = L.qlora_linear_bwd
    args = dict(X=FAKE, dY=FAKE, M=16, A=FAKE, B=FAKE, r=8, alpha=2.0, U=None, dX=FAKE, dA=FAKE,
                dB=FAKE, ws=None, wsb=0)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return b(w, a["X"], a["dY"], a["M"], a["A"], a["B"], a["r"], a["alpha"], a["U"], a["dX"],
                 a["dA"], a["dB"], a["ws"], a["wsb"], 0)

    assert call() == WORKSPACE
    need = L.qlora_workspace_bytes(2, 16, 64, 64, 8)
    assert call(ws=FAKE, wsb=need - 1) == WORKSPACE
    assert call(dA=None) == INVALID
    assert call(dX=None) == INVALID
    assert call(dY=None) == INVALID
    assert call(dB=FAKE_MIS) == ALIGN
    assert call(r=99) == SHAPE
    assert call(U=FAKE_MIS, ws=FAKE, wsb=need) == ALIGN


def _tiled(M, R):
    """Bytes of the fragment-tiled activation copy the GEMMs read: 32-row
    blocks x whole 64-deep steps of 16-bit elements."""
    return -(-M // 32) * 32 * (-(-R // 64) * 64) * 2


def test_workspace_sizes(L):
    ws = L.qlora_workspace_bytes
    assert ws(1, 2048, 4096, 4096, 0) == _tiled(2048, 4096)  # the tiled X only
    # r = 16: the tiled X and the row pass's fp32 U~ partials, 4 splits of the
    # 32 chunks of 128 (64 row blocks x 4 splits fill the 256 compute units
    # a host without a GPU assumes)
    assert ws(1, 2048, 4096, 4096, 16) == _tiled(2048, 4096) + 4 * 2048 * 16 * 4
    # backward: U~ and V~ slots, the tiled dY, one region for the larger
    # of the row-pass partials of a U~ recompute (4 splits over k_in) and of
    # V~ (4 splits over n_out), and the keep mask of X as bits (one bit per
    # element of the 2048 x 4096 adapter input, used under dropout)
    b = ws(2, 2048, 11008, 4096, 16)
    assert b == 2 * 2048 * 16 * 2 + _tiled(2048, 11008) + 4 * 2048 * 16 * 4 + 2048 * 4096 // 8
    assert ws(2, 2048, 4096, 4096, 0) == _tiled(2048, 4096)  # the tiled dY only
    assert ws(9, 1, 1, 64, 1) == 0
    # few output tiles: optional room for a reduction split, also with r = 0
    # (8 tiles of 256 x 128 over 32 steps of 64: 4 splits of fp32 130 x 1024)
    assert ws(1, 130, 1024, 2048, 0) == _tiled(130, 2048) + 4 * 130 * 1024 * 4
    assert ws(1, 130, 1024, 2048, 16) >= 130 * 16 * 2 + _tiled(130, 2048) + 4 * 130 * 1024 * 4
    assert ws(2, 130, 1024, 2048, 0) == _tiled(130, 1024) + 2 * 130 * 2048 * 4  # dX: 16 tiles, 16 steps
    assert ws(1, 16, 1024, 2048, 0) == 0  # few-token kernel: no split
    # few-token kernel over a long reduction: 4 splits of fp32 16 x 8192
    assert ws(1, 16, 8192, 28672, 0) == 4 * 16 * 8192 * 4
    assert ws(1, 4, 8192, 28672, 0) == 0  # under 8 tokens: unsplit
    # few tokens with an adapter: U~, then the down projection's partials
    # (112 sub-chunks of 256 in 28 splits of 4: at most 32 KB of partials),
    # then the main product's split partials -- disjoint, since the few-token
    # kernel reads the first while it writes the second
    assert ws(1, 16, 8192, 28672, 16) == 16 * 16 * 2 + 28 * 16 * 16 * 4 + 4 * 16 * 8192 * 4
    assert ws(1, 1, 8192, 28672, 16) == 256 + 28 * 1 * 16 * 4  # (U~ rounded up to 256 bytes; no split)
    assert ws(1, 16, 64, 64, 65) == 0


def test_merge_and_bf16_quantize_validation(L):
    w = ctypes.byref(_w())
    m = L.qlora_merge
    assert m(w, FAKE, FAKE, 99, 2.0, FAKE, None) == SHAPE        # rank above the maximum
    assert m(w, None, FAKE, 8, 2.0, FAKE, None) == INVALID       # A missing with r > 0
    assert m(w, FAKE, FAKE, 8, 2.0, None, None) == INVALID       # no output
    assert m(w, FAKE, FAKE, 8, 2.0, FAKE_MIS, None) == ALIGN
    assert m(ctypes.byref(_w(k_in=96)), FAKE, FAKE, 8, 2.0, FAKE, None) == SHAPE  # k_in % 64
    assert m(ctypes.byref(_w(n_out=0)), FAKE, FAKE, 8, 2.0, FAKE, None) == OK    # empty weight
    q = L.qlora_quantize_nf4_dq_bf16
    assert q(None, 64, 64, FAKE, FAKE, FAKE, None) == INVALID
    assert q(FAKE_MIS, 64, 64, FAKE, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 64, 96, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, 0, 64, FAKE, FAKE, FAKE, None) == OK


def test_dropout_entry_points_validation(L):
    w = ctypes.byref(_w())
    f = L.qlora_linear_fwd_dropout
    b = L.qlora_linear_bwd_dropout
    for p in (-0.1, 1.0, 1.5, float("nan")):
        assert f(w, FAKE, 16, FAKE, FAKE, 8, 2.0, p, 7, FAKE, FAKE, None, 0, 0) == INVALID, p
        assert b(w, FAKE, FAKE, 16, FAKE, FAKE, 8, 2.0, p, 7, FAKE, FAKE, FAKE, FAKE, None, 0, 0) == INVALID, p
    assert b"dropout_p" in L.qlora_last_error()
    # a valid probability leaves the other checks as in the plain entry points
    assert f(w, FAKE, 16, FAKE, FAKE, 65, 2.0, 0.05, 7, FAKE, FAKE, None, 0, 0) == SHAPE
    assert f(w, FAKE_MIS, 16, FAKE, FAKE, 8, 2.0, 0.05, 7, FAKE, FAKE, None, 0, 0) == ALIGN
    assert f(w, FAKE, 16, FAKE, FAKE, 8, 2.0, 0.05, 7, FAKE, None, None, 0, 0) == WORKSPACE
    assert b(w, FAKE, FAKE, 16, FAKE, FAKE, 8, 2.0, 0.05, 7, None, FAKE, FAKE, FAKE, None, 0, 0) == WORKSPACE
    assert f(w, None, 0, FAKE, FAKE, 8, 2.0, 0.05, 7, None, None, None, 0, 0) == OK


def test_format_tables_match_oracle_bitwise(L):
    from oracle import formats
    for name, fid in qlora.FORMATS.items():
        t = np.array(qlora.format_table(name), dtype=np.float32)
        assert np.array_equal(t.view(np.uint32), formats.format_table(name).view(np.uint32)), name
    buf = (ctypes.c_float * 16)()
    assert L.qlora_format_table(4, buf) == INVALID
    assert L.qlora_format_table(-1, buf) == INVALID
    assert L.qlora_format_table(0, None) == INVALID


def test_format_entry_points_validation(L):
    q, d = L.qlora_quantize_format, L.qlora_dequant_format
    for fmt in (4, -1):
        assert q(fmt, FAKE, 64, 64, FAKE, FAKE, FAKE, 0) == INVALID
        assert d(fmt, 64, 64, FAKE, FAKE, FAKE, FAKE, 0) == INVALID
    assert b"format" in L.qlora_last_error()
    for fmt in range(4):
        assert q(fmt, FAKE, 64, 96, FAKE, FAKE, FAKE, 0) == SHAPE
        assert q(fmt, FAKE_MIS, 64, 64, FAKE, FAKE, FAKE, 0) == ALIGN
        assert q(fmt, FAKE, 64, 64, FAKE, FAKE_MIS, FAKE, 0) == ALIGN
        assert q(fmt, FAKE, 64, 64, None, FAKE, FAKE, 0) == INVALID
        assert d(fmt, 64, 64, FAKE, FAKE, FAKE, None, 0) == INVALID
        assert q(fmt, FAKE, 0, 64, None, None, None, 0) == OK
    # the step array is needed only with double quantization
    assert q(0, FAKE, 64, 64, FAKE, FAKE, None, 0) == INVALID
    assert q(2, FAKE, 64, 64, FAKE, FAKE, None, 0) == INVALID
    assert d(0, 64, 64, FAKE, FAKE, FAKE_MIS, FAKE, 0) == ALIGN


def test_plan_splits_are_never_empty(L):
    """Work splits of the few-token kernel and of the fused GEMM over a sweep
    of sizes and compute-unit counts (a whole MI355X and partitions of it):
    every split holds at least one chunk or step and together they cover the
    reduction."""
    checked = 0
    for cus in (256, 304, 128, 80, 32, 8):
        for M in (1, 4, 8, 9, 16, 17, 64, 100, 256, 300, 512, 2048):
            for N in (8, 64, 520, 1024, 4096, 8192, 11008, 28672):
                for K in (64, 1024, 4096, 8256, 11008, 28672, 65600):
                    for op in (1, 2):
                        p = qlora.plan(op, M, N, K, cus)
                        assert p["splits"] >= 1 and p["per_split"] >= 1
                        assert (p["splits"] - 1) * p["per_split"] < p["total"] <= p["splits"] * p["per_split"], \
                            (op, M, N, K, cus, p)
                        assert p["kernel"] == ("few_token" if op == 1 and M <= 16 else "gemm")
                        checked += 1
    assert checked == 6 * 12 * 8 * 7 * 2


def test_plan_few_token_example_without_empty_split(L):
    """N = 1024, K = 65600, M = 16 on 256 compute units: 513 chunks of 128.
    32 splits of 17 chunks would leave the last one empty; the planner
    settles on 31 splits."""
    p = qlora.plan(1, 16, 1024, 65600, 256)
    assert p["kernel"] == "few_token" and p["total"] == 513
    assert p["per_split"] == 17 and p["splits"] == 31


def test_plan_and_workspace_agree(L):
    """The workspace counts the split's partial sums for the device it sizes
    for (here: no device, so 256 compute units)."""
    for M, N, K in ((16, 8192, 28672), (16, 1024, 65600), (300, 2048, 2048), (130, 1024, 2048)):
        p = qlora.plan(1, M, N, K, 0)
        ws = qlora.workspace_bytes(1, M, N, K, 0)
        if p["splits"] > 1:
            assert ws >= p["splits"] * M * N * 4
        assert p == qlora.plan(1, M, N, K, 256)


def test_plan_rejects_bad_arguments(L):
    out = (ctypes.c_int64 * 4)()
    assert L.qlora_plan(3, 16, 64, 64, 0, out) == INVALID
    assert L.qlora_plan(1, -1, 64, 64, 0, out) == INVALID
    assert L.qlora_plan(1, 16, 64, 64, 0, None) == INVALID
