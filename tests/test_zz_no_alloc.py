"""The allocation-free forward (qlora_linear_fwd_noalloc) against the
workspace-taking forward (qlora_linear_fwd), through the C ABI.

The no-alloc entry point runs the same kernels with the library's fixed
per-GPU scratch as workspace, so its Y and U~ must equal those of
qlora_linear_fwd given a full workspace bit for bit.  Two calls in a row,
the second on a smaller input (the scratch keeps the first call's
contents), then a third in the few-token path; sizes beyond the scratch are
refused before anything is enqueued.
"""

import ctypes

import numpy as np
import pytest
import torch

from bit_nf4_quantized_double_amd import qlora, synth

pytestmark = pytest.mark.gpu

WORKSPACE_ERR = -4


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _inputs(M, N, K, r, seed):
    d = synth.linear_inputs(N, K, M, r, np.random.default_rng(seed))
    w = qlora.quantize(torch.from_numpy(d["W"]).cuda())
    X = _bf16(d["X"])
    A = _bf16(d["A"]) if r > 0 else None
    B = _bf16(d["B"]) if r > 0 else None
    return w, X, A, B


def _compare(M, N, K, r, alpha, seed):
    w, X, A, B = _inputs(M, N, K, r, seed)
    Yr, Ur = qlora.linear_fwd(w, X, A, B, r, alpha)  # full workspace from qlora_workspace_bytes
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    U = torch.full((M, r), float("nan"), dtype=torch.bfloat16, device="cuda") if r > 0 else None
    L = qlora.lib()
    cw = w._c()
    st = L.qlora_linear_fwd_noalloc(ctypes.byref(cw), X.data_ptr(), M, None if A is None else A.data_ptr(),
                                    None if B is None else B.data_ptr(), r, alpha, Y.data_ptr(),
                                    None if U is None else U.data_ptr(), qlora._stream())
    assert st == 0, L.qlora_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yr.view(torch.int16)), (M, N, K, r)
    if r > 0:
        assert torch.equal(U.view(torch.int16), Ur.view(torch.int16)), (M, N, K, r)


def test_noalloc_forward_matches_workspace_forward_twice():
    """A split GEMM forward, then a smaller ragged one, then a few-token one."""
    _need_gpu()
    _compare(300, 2048, 2048, 16, 32.0, seed=41)  # reduction split 4 ways, U~ partials
    _compare(100, 200, 192, 17, 5.0, seed=42)     # smaller, ragged tiles, rank 17
    _compare(16, 4104, 320, 64, 128.0, seed=43)   # few-token kernel, partial tile


def test_noalloc_forward_rejects_sizes_beyond_the_scratch():
    _need_gpu()
    L = qlora.lib()
    # the first of these whose forward needs more workspace than the scratch
    cands = [(8192, 4096, 14336, 16), (1 << 20, 1024, 1024, 64)]
    M, N, K, r = next(c for c in cands if qlora.workspace_bytes(qlora.QLORA_OP_FWD, *c) > 64 << 20)
    cw = qlora._CWeight(N, K, 0x10000, 0x10000, 0x10000)  # never dereferenced
    st = L.qlora_linear_fwd_noalloc(ctypes.byref(cw), 0x10000, M, 0x10000, 0x10000, r, 32.0, 0x10000, None, None)
    assert st == WORKSPACE_ERR
    assert "scratch" in L.qlora_last_error().decode()
