"""ctypes binding over libqlora.so (the C ABI in include/qlora.h).

Argument marshalling only: PyTorch supplies device memory (``data_ptr()``) and
the current HIP stream; every step of the computation runs in the library's
gfx950 kernels.  There is no CPU or PyTorch fallback -- a missing library, a
CPU tensor or a wrong dtype raises.

bf16 tensors are passed as their raw bits (the ABI takes uint16_t).
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the same library with every raw global access range checked (see
# qlora_debug_oob_count in include/qlora.h)
LIB_CHECKED_PATH = os.path.join(_HERE, "libqlora_checked.so")
# QLORA_LIBRARY=checked runs everything through the bounds-checked build
LIB_PATH = LIB_CHECKED_PATH if os.environ.get("QLORA_LIBRARY") == "checked" else os.path.join(_HERE, "libqlora.so")

QLORA_OK = 0
QLORA_OP_FWD = 1
QLORA_OP_BWD = 2
FORMATS = {"nf4_dq": 0, "nf4": 1, "int4_dq": 2, "int4": 3}  # QLORA_FORMAT_*
MAX_RANK = 64

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class _CWeight(ctypes.Structure):
    _fields_ = [("n_out", _c_i64), ("k_in", _c_i64), ("codes", _vp),
                ("absmax_q8", _vp), ("absmax_scale", _vp)]


_lib = None
_loaded = {}


def lib() -> ctypes.CDLL:
    """Load libqlora.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Route every call made inside the block through the library at `path`
    (e.g. LIB_CHECKED_PATH); the previous one is restored afterwards."""
    global _lib
    prev = _lib
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = prev


def debug_oob_count(reset: bool = True) -> int:
    """Out-of-range accesses the bounds-checked build skipped since the last
    reset (qlora_debug_oob_count; raises in the normal build)."""
    n = ctypes.c_uint64(0)
    _check(lib().qlora_debug_oob_count(ctypes.byref(n), 1 if reset else 0), "qlora_debug_oob_count")
    return int(n.value)


def _load(path: str) -> ctypes.CDLL:
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m bit_nf4_quantized_double_amd.build`")
    L = ctypes.CDLL(path)
    W = ctypes.POINTER(_CWeight)
    sig = {
        "qlora_quantize_nf4_dq": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
        "qlora_quantize_nf4_dq_bf16": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
        "qlora_merge": (ctypes.c_int, [W, _vp, _vp, _c_i32, ctypes.c_float, _vp, _vp]),
        "qlora_dequant": (ctypes.c_int, [W, _vp, _vp]),
        "qlora_dequant_f16": (ctypes.c_int, [W, _vp, _vp]),
        "qlora_linear_fwd_f16": (ctypes.c_int, [W, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                                _vp, _vp, _vp, ctypes.c_size_t, _vp]),
        "qlora_linear_bwd_f16": (ctypes.c_int, [W, _vp, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                                _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
        "qlora_linear_fwd": (ctypes.c_int, [W, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                            _vp, _vp, _vp, ctypes.c_size_t, _vp]),
        "qlora_linear_bwd": (ctypes.c_int, [W, _vp, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                            _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
        "qlora_linear_fwd_noalloc": (ctypes.c_int, [W, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                                    _vp, _vp, _vp]),
        "qlora_linear_fwd_dropout": (ctypes.c_int, [W, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                                    ctypes.c_double, ctypes.c_uint64,
                                                    _vp, _vp, _vp, ctypes.c_size_t, _vp]),
        "qlora_linear_bwd_dropout": (ctypes.c_int, [W, _vp, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                                    ctypes.c_double, ctypes.c_uint64,
                                                    _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
        "qlora_linear_fwd_dropout_f16": (ctypes.c_int, [W, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                                        ctypes.c_double, ctypes.c_uint64,
                                                        _vp, _vp, _vp, ctypes.c_size_t, _vp]),
        "qlora_linear_bwd_dropout_f16": (ctypes.c_int, [W, _vp, _vp, _c_i64, _vp, _vp, _c_i32, ctypes.c_float,
                                                        ctypes.c_double, ctypes.c_uint64,
                                                        _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
        "qlora_quantize_format": (ctypes.c_int, [ctypes.c_int, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
        "qlora_dequant_format": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp]),
        "qlora_format_table": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_float)]),
        "qlora_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_i32]),
        "qlora_plan": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                      ctypes.POINTER(_c_i64)]),
        "qlora_nf4_table": (None, [ctypes.POINTER(ctypes.c_float)]),
        "qlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "qlora_last_error": (ctypes.c_char_p, []),
        "qlora_time_next_gemm": (None, [_vp, _vp]),
        "qlora_debug_oob_count": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint64), ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _loaded[path] = L
    return L


def _check(status: int, what: str) -> None:
    if status != QLORA_OK:
        L = lib()
        raise RuntimeError(f"{what}: {L.qlora_status_string(status).decode()} "
                           f"({L.qlora_last_error().decode()})")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, dtype, name):
    return None if t is None else _dev(t, dtype, name)


@dataclass
class NF4Weight:
    """A frozen weight in NF4 with double-quantized block scales."""
    codes: torch.Tensor         # uint8 [n_out*k_in/2]
    absmax_q8: torch.Tensor     # uint8 [nb]
    absmax_scale: torch.Tensor  # float32 [ng]
    n_out: int
    k_in: int

    def _c(self) -> _CWeight:
        return _CWeight(self.n_out, self.k_in,
                        _dev(self.codes, torch.uint8, "codes"),
                        _dev(self.absmax_q8, torch.uint8, "absmax_q8"),
                        _dev(self.absmax_scale, torch.float32, "absmax_scale"))

    def nbytes(self) -> int:
        return self.codes.numel() + self.absmax_q8.numel() + 4 * self.absmax_scale.numel()


def nf4_table() -> list:
    buf = (ctypes.c_float * 16)()
    lib().qlora_nf4_table(buf)
    return list(buf)


def workspace_bytes(op: int, M: int, n_out: int, k_in: int, r: int) -> int:
    return int(lib().qlora_workspace_bytes(op, M, n_out, k_in, r))


def plan(op: int, M: int, n_out: int, k_in: int, compute_units: int = 0) -> dict:
    """The library's work split for the main product (qlora_plan)."""
    out = (_c_i64 * 4)()
    _check(lib().qlora_plan(op, M, n_out, k_in, compute_units, out), "qlora_plan")
    return {"kernel": {1: "gemm", 2: "few_token"}[out[0]], "splits": out[1], "per_split": out[2],
            "total": out[3]}


def _empty_u8(n, device):
    # 16-byte aligned even when n == 0
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)[:n]


def quantize(W: torch.Tensor, out: NF4Weight | None = None) -> NF4Weight:
    """fp32 or bf16 [n_out, k_in] GPU tensor -> NF4Weight (codes, q8, s2).
    ``out``: an NF4Weight of the same shape whose buffers are overwritten
    (no allocation)."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D [n_out, k_in]")
    n_out, k_in = W.shape
    nw = n_out * k_in
    nb = nw // 64
    ng = (nb + 255) // 256
    dev = W.device
    if out is not None:
        if (out.n_out, out.k_in) != (n_out, k_in):
            raise ValueError("out has a different shape")
        codes, q8, s2 = out.codes, out.absmax_q8, out.absmax_scale
        for t, dt, n, name in ((codes, torch.uint8, nw // 2, "out.codes"), (q8, torch.uint8, nb, "out.absmax_q8"),
                               (s2, torch.float32, ng, "out.absmax_scale")):
            _dev(t, dt, name)
            if t.device != dev or t.numel() < n:
                raise ValueError(f"{name} must be on W's device and hold {n} elements")
    else:
        codes = _empty_u8(nw // 2, dev)
        q8 = _empty_u8(nb, dev)
        s2 = torch.empty(max(ng, 4), dtype=torch.float32, device=dev)[:ng]
    if W.dtype == torch.bfloat16:
        st = lib().qlora_quantize_nf4_dq_bf16(_dev(W, torch.bfloat16, "W"), n_out, k_in, codes.data_ptr(),
                                              q8.data_ptr(), s2.data_ptr(), _stream())
        _check(st, "qlora_quantize_nf4_dq_bf16")
    else:
        st = lib().qlora_quantize_nf4_dq(_dev(W, torch.float32, "W"), n_out, k_in, codes.data_ptr(),
                                         q8.data_ptr(), s2.data_ptr(), _stream())
        _check(st, "qlora_quantize_nf4_dq")
    return out if out is not None else NF4Weight(codes, q8, s2, n_out, k_in)


@dataclass
class FormatWeight:
    """A weight in one of the storage-format variants (see FORMATS)."""
    fmt: str
    codes: torch.Tensor            # uint8 [n_out*k_in/2]
    scales: torch.Tensor           # uint8 q8 [nb] (*_dq) or float32 absmax [nb]
    absmax_scale: torch.Tensor | None  # float32 [ng] (*_dq) or None
    n_out: int
    k_in: int

    def nbytes(self) -> int:
        n = self.codes.numel() + self.scales.numel() * self.scales.element_size()
        return n + (0 if self.absmax_scale is None else 4 * self.absmax_scale.numel())


def format_table(fmt: str) -> list:
    buf = (ctypes.c_float * 16)()
    _check(lib().qlora_format_table(FORMATS[fmt], buf), "qlora_format_table")
    return list(buf)


def quantize_format(W: torch.Tensor, fmt: str) -> FormatWeight:
    """fp32 [n_out, k_in] GPU tensor -> FormatWeight in format ``fmt``."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D [n_out, k_in]")
    n_out, k_in = W.shape
    nw = n_out * k_in
    nb, dev = nw // 64, W.device
    ng = (nb + 255) // 256
    dq = fmt.endswith("_dq")
    codes = _empty_u8(nw // 2, dev)
    scales = _empty_u8(nb, dev) if dq else torch.empty(max(nb, 4), dtype=torch.float32, device=dev)[:nb]
    s2 = torch.empty(max(ng, 4), dtype=torch.float32, device=dev)[:ng] if dq else None
    st = lib().qlora_quantize_format(FORMATS[fmt], _dev(W, torch.float32, "W"), n_out, k_in, codes.data_ptr(),
                                     scales.data_ptr(), None if s2 is None else s2.data_ptr(), _stream())
    _check(st, "qlora_quantize_format")
    return FormatWeight(fmt, codes, scales, s2, n_out, k_in)


def dequant_format(w: FormatWeight, out: torch.Tensor | None = None) -> torch.Tensor:
    """Whole weight of a FormatWeight as bf16 [n_out, k_in]."""
    if out is None:
        out = torch.empty((w.n_out, w.k_in), dtype=torch.bfloat16, device=w.codes.device)
    st = lib().qlora_dequant_format(FORMATS[w.fmt], w.n_out, w.k_in, _dev(w.codes, torch.uint8, "codes"),
                                    w.scales.data_ptr(),
                                    None if w.absmax_scale is None else w.absmax_scale.data_ptr(),
                                    _dev(out, torch.bfloat16, "out"), _stream())
    _check(st, "qlora_dequant_format")
    return out


def merge(w: NF4Weight, A: torch.Tensor | None, B: torch.Tensor | None, r: int, alpha: float,
          out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [n_out, k_in] merged weight bf16(W_bf16 + (alpha/r) B A)."""
    if out is None:
        out = torch.empty((w.n_out, w.k_in), dtype=torch.bfloat16, device=w.codes.device)
    cw = w._c()
    st = lib().qlora_merge(ctypes.byref(cw), _opt(A, torch.bfloat16, "A"), _opt(B, torch.bfloat16, "B"), r,
                           float(alpha), _dev(out, torch.bfloat16, "out"), _stream())
    _check(st, "qlora_merge")
    return out


def dequant(w: NF4Weight, out: torch.Tensor | None = None, dtype=torch.bfloat16) -> torch.Tensor:
    """Whole weight as a bf16 (or, with dtype=torch.float16 or an fp16
    ``out``, fp16) [n_out, k_in] GPU tensor."""
    if out is not None:
        dtype = out.dtype
    if dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("dequant produces bf16 or fp16")
    if out is None:
        out = torch.empty((w.n_out, w.k_in), dtype=dtype, device=w.codes.device)
    cw = w._c()
    if dtype == torch.float16:
        st = lib().qlora_dequant_f16(ctypes.byref(cw), _dev(out, torch.float16, "out"), _stream())
        _check(st, "qlora_dequant_f16")
    else:
        st = lib().qlora_dequant(ctypes.byref(cw), _dev(out, torch.bfloat16, "out"), _stream())
        _check(st, "qlora_dequant")
    return out


def _elem(X: torch.Tensor):
    """16-bit element type of a product: bf16 or fp16, from the activations."""
    if X.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"X must be bf16 or fp16, got {X.dtype}")
    return X.dtype


def new_workspace(op: int, M: int, n_out: int, k_in: int, r: int, device) -> torch.Tensor:
    """A workspace for `op` at these sizes (reusable across calls)."""
    return torch.empty(max(1, workspace_bytes(op, M, n_out, k_in, r)), dtype=torch.uint8, device=device)


def _ws(nbytes: int, device, ws: torch.Tensor | None):
    """The caller's workspace when it is big enough, else a fresh one."""
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() >= nbytes:
        return ws, ws.numel()
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return t, nbytes


def linear_fwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None,
               r: int, alpha: float, *, Y: torch.Tensor | None = None,
               U: torch.Tensor | None = None, return_u: bool = True,
               ws: torch.Tensor | None = None, dropout_p: float = 0.0, seed: int = 0):
    """Y = X W^T + U~ B^T with U~ = bf16((alpha/r) X A^T).  Returns (Y, U~).

    dropout_p > 0: LoRA dropout of the adapter input with the keep mask of
    ``seed`` (qlora_linear_fwd_dropout); U~ = bf16(alpha/(r(1-p)) (keep X) A^T).
    """
    M = X.shape[0]
    dev = X.device
    et = _elem(X)
    if Y is None:
        Y = torch.empty((M, w.n_out), dtype=et, device=dev)
    if return_u and r > 0 and U is None:
        U = torch.empty((M, r), dtype=et, device=dev)
    wsb = workspace_bytes(QLORA_OP_FWD, M, w.n_out, w.k_in, r)
    wst, wsn = _ws(wsb, dev, ws)
    cw = w._c()
    head = (ctypes.byref(cw), _dev(X, et, "X"), M, _opt(A, et, "A"), _opt(B, et, "B"), r, float(alpha))
    tail = (_dev(Y, et, "Y"), _opt(U, et, "U"), None if wst is None else wst.data_ptr(), wsn, _stream())
    if et == torch.float16 and dropout_p:
        st = lib().qlora_linear_fwd_dropout_f16(*head, float(dropout_p), int(seed) & (2**64 - 1), *tail)
        _check(st, "qlora_linear_fwd_dropout_f16")
    elif et == torch.float16:
        st = lib().qlora_linear_fwd_f16(*head, *tail)
        _check(st, "qlora_linear_fwd_f16")
    elif dropout_p:
        st = lib().qlora_linear_fwd_dropout(*head, float(dropout_p), int(seed) & (2**64 - 1), *tail)
        _check(st, "qlora_linear_fwd_dropout")
    else:
        st = lib().qlora_linear_fwd(*head, *tail)
        _check(st, "qlora_linear_fwd")
    return Y, U


def linear_fwd_noalloc(w: NF4Weight, X: torch.Tensor, A: torch.Tensor | None, B: torch.Tensor | None,
                       r: int, alpha: float, Y: torch.Tensor, U: torch.Tensor | None = None):
    """qlora_linear_fwd_noalloc: the bf16 forward into caller-provided Y (and
    U~), with the library's fixed scratch as workspace (nothing allocated)."""
    cw = w._c()
    st = lib().qlora_linear_fwd_noalloc(ctypes.byref(cw), _dev(X, torch.bfloat16, "X"), X.shape[0],
                                        _opt(A, torch.bfloat16, "A"), _opt(B, torch.bfloat16, "B"), r,
                                        float(alpha), _dev(Y, torch.bfloat16, "Y"), _opt(U, torch.bfloat16, "U"),
                                        _stream())
    _check(st, "qlora_linear_fwd_noalloc")
    return Y, U


def linear_bwd(w: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor | None,
               B: torch.Tensor | None, r: int, alpha: float, U: torch.Tensor | None = None, *,
               dX: torch.Tensor | None = None, dA: torch.Tensor | None = None,
               dB: torch.Tensor | None = None, ws: torch.Tensor | None = None,
               dropout_p: float = 0.0, seed: int = 0):
    """Returns (dX bf16 [M,K], dA fp32 [r,K], dB fp32 [N,r]); never dW.

    dropout_p > 0: the backward of :func:`linear_fwd` with the same
    ``dropout_p`` and ``seed`` (qlora_linear_bwd_dropout).
    """
    M = X.shape[0]
    dev = X.device
    et = _elem(X)
    if dX is None:
        dX = torch.empty((M, w.k_in), dtype=et, device=dev)
    if r > 0 and dA is None:
        dA = torch.empty((r, w.k_in), dtype=torch.float32, device=dev)
    if r > 0 and dB is None:
        dB = torch.empty((w.n_out, r), dtype=torch.float32, device=dev)
    wsb = workspace_bytes(QLORA_OP_BWD, M, w.n_out, w.k_in, r)
    wst, wsn = _ws(wsb, dev, ws)
    cw = w._c()
    head = (ctypes.byref(cw), _dev(X, et, "X"), _dev(dY, et, "dY"), M,
            _opt(A, et, "A"), _opt(B, et, "B"), r, float(alpha))
    tail = (_opt(U, et, "U"), _dev(dX, et, "dX"),
            _opt(dA, torch.float32, "dA"), _opt(dB, torch.float32, "dB"),
            None if wst is None else wst.data_ptr(), wsn, _stream())
    if et == torch.float16 and dropout_p:
        st = lib().qlora_linear_bwd_dropout_f16(*head, float(dropout_p), int(seed) & (2**64 - 1), *tail)
        _check(st, "qlora_linear_bwd_dropout_f16")
    elif et == torch.float16:
        st = lib().qlora_linear_bwd_f16(*head, *tail)
        _check(st, "qlora_linear_bwd_f16")
    elif dropout_p:
        st = lib().qlora_linear_bwd_dropout(*head, float(dropout_p), int(seed) & (2**64 - 1), *tail)
        _check(st, "qlora_linear_bwd_dropout")
    else:
        st = lib().qlora_linear_bwd(*head, *tail)
        _check(st, "qlora_linear_bwd")
    return dX, dA, dB


class QLoRALinearFunction(torch.autograd.Function):
    """Autograd wrapper: forward saves U~ for the backward; no grad for W."""

    @staticmethod
    def forward(ctx, X, A, B, w: NF4Weight, r: int, alpha: float, dropout_p: float = 0.0, seed: int = 0):
        X2 = X.reshape(-1, w.k_in).contiguous()
        Y, U = linear_fwd(w, X2, A, B, r, alpha, dropout_p=dropout_p, seed=seed)
        ctx.save_for_backward(X2, A, B, U)
        ctx.w, ctx.r, ctx.alpha, ctx.xshape = w, r, alpha, X.shape
        ctx.dropout_p, ctx.seed = dropout_p, seed
        return Y.reshape(*X.shape[:-1], w.n_out)

    @staticmethod
    def backward(ctx, dY):
        X2, A, B, U = ctx.saved_tensors
        # the gradient arrives in the output's dtype, which is X's (bf16 or fp16)
        dY2 = dY.reshape(-1, ctx.w.n_out).contiguous().to(X2.dtype)
        dX, dA, dB = linear_bwd(ctx.w, X2, dY2, A, B, ctx.r, ctx.alpha, U,
                                dropout_p=ctx.dropout_p, seed=ctx.seed)
        gA = dA.to(A.dtype) if (A is not None and ctx.needs_input_grad[1]) else None
        gB = dB.to(B.dtype) if (B is not None and ctx.needs_input_grad[2]) else None
        return dX.reshape(ctx.xshape), gA, gB, None, None, None, None, None


class QLoRALinear(torch.nn.Module):
    """nn.Linear replacement: frozen NF4 weight + trainable 16-bit adapter.

    ``dtype`` is the compute dtype: bf16 (the pages' choice) or fp16 (the one
    they name for GPUs without bf16).  The adapter parameters are held in
    it, and inputs must come in it.
    """

    def __init__(self, weight_fp32: torch.Tensor, r: int = 16, alpha: float = 32.0,
                 A: torch.Tensor | None = None, B: torch.Tensor | None = None, lora_dropout: float = 0.0,
                 dtype=torch.bfloat16):
        super().__init__()
        if dtype not in (torch.bfloat16, torch.float16):
            raise TypeError("the compute dtype is bf16 or fp16")
        self.lora_dropout = float(lora_dropout)
        n_out, k_in = weight_fp32.shape
        self.w = quantize(weight_fp32.contiguous())
        self.r, self.alpha = r, float(alpha)
        dev = weight_fp32.device
        if A is None:
            A = torch.randn(r, k_in, device=dev) / (k_in ** 0.5)
        if B is None:
            B = torch.zeros(n_out, r, device=dev)
        self.A = torch.nn.Parameter(A.to(dtype).contiguous())
        self.B = torch.nn.Parameter(B.to(dtype).contiguous())

    def forward(self, X):
        # a fresh mask per training step (the seed is drawn from torch's host
        # generator); no dropout in eval mode
        p = self.lora_dropout if self.training else 0.0
        seed = int(torch.randint(0, 2**62, (1,)).item()) if p else 0
        return QLoRALinearFunction.apply(X, self.A, self.B, self.w, self.r, self.alpha, p, seed)
