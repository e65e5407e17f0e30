"""ctypes binding of ``libqlr.so`` (C ABI in ``include/qlr.h``).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's gfx950
kernels.  There is no CPU fallback: if the library cannot be loaded, every call
raises.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import threading
from dataclasses import dataclass
from typing import List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqlr.so")

FORMAT_VERSION = 1
BLOCK = 64
GROUP = 256

QLR_F32, QLR_F16, QLR_BF16 = 0, 1, 2
PATH_AUTO, PATH_F32, PATH_GEMV, PATH_GEMM = 0, 1, 2, 3
OP_QUANTIZE, OP_LINEAR, OP_LINEAR_BWD, OP_LINEAR_DBA = 0, 1, 2, 3
OP_QUANTIZE_OUTLIERS, OP_LINEAR_OUTLIERS, OP_LINEAR_WHA = 4, 5, 6

STATUS = {
    0: "QLR_OK", 1: "QLR_ERR_NULL", 2: "QLR_ERR_SHAPE", 3: "QLR_ERR_DTYPE", 4: "QLR_ERR_BITS",
    5: "QLR_ERR_BLOCK", 6: "QLR_ERR_ALIGN", 7: "QLR_ERR_NONFINITE", 8: "QLR_ERR_WORKSPACE",
    9: "QLR_ERR_ALIAS", 10: "QLR_ERR_HIP", 11: "QLR_ERR_FORMAT", 12: "QLR_ERR_PATH",
}


class QlrError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


class CQWeight(C.Structure):
    _fields_ = [
        ("format_version", C.c_uint32), ("bits", C.c_int32), ("block", C.c_int32),
        ("group", C.c_int32), ("rows", C.c_int64), ("cols", C.c_int64),
        ("codes", C.c_void_p), ("absmax_q8", C.c_void_p), ("absmax_c", C.c_void_p),
    ]


class CLayer(C.Structure):
    _fields_ = [
        ("w", C.POINTER(CQWeight)), ("x", C.c_void_p), ("A", C.c_void_p), ("B", C.c_void_p),
        ("r", C.c_int32), ("scale", C.c_float), ("y", C.c_void_p),
    ]


class CDba(C.Structure):
    _fields_ = [
        ("rank", C.c_int32), ("ell", C.c_int32), ("b1", C.c_void_p), ("b2", C.c_void_p),
        ("alpha", C.c_void_p), ("beta", C.c_void_p), ("gamma", C.c_void_p),
    ]


class CSparse(C.Structure):
    _fields_ = [
        ("rows", C.c_int64), ("cols", C.c_int64), ("nnz", C.c_int64), ("row_ptr", C.c_void_p),
        ("col", C.c_void_p), ("val", C.c_void_p), ("max_group_nnz", C.c_int64),
    ]


EXPORTS = {
    "qlr_version": (C.c_int, []),
    "qlr_status_string": (C.c_char_p, [C.c_int]),
    "qlr_last_error": (C.c_char_p, []),
    "qlr_codebook": (C.c_int, [C.c_int32, C.POINTER(C.c_float)]),
    "qlr_qweight_sizes": (C.c_int, [C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                    C.POINTER(C.c_size_t), C.POINTER(C.c_size_t),
                                    C.POINTER(C.c_size_t)]),
    "qlr_workspace_bytes": (C.c_int, [C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int32,
                                      C.POINTER(C.c_size_t)]),
    "qlr_quantize": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                               C.POINTER(CQWeight), C.c_void_p, C.c_size_t, C.c_void_p]),
    "qlr_quantize_async": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int32,
                                     C.c_int32, C.POINTER(CQWeight), C.c_void_p, C.c_size_t,
                                     C.c_void_p]),
    "qlr_dequantize": (C.c_int, [C.POINTER(CQWeight), C.c_void_p, C.c_int, C.c_void_p]),
    "qlr_linear_fwd": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.POINTER(CQWeight),
                                 C.c_void_p, C.c_void_p, C.c_int, C.c_int32, C.c_float,
                                 C.c_void_p, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qlr_linear_fwd_static": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.POINTER(CQWeight),
                                        C.c_void_p, C.c_void_p, C.c_int, C.c_int32, C.c_float,
                                        C.c_void_p, C.c_int, C.c_void_p]),
    "qlr_linear_fwd_mixed": (C.c_int, [C.POINTER(CLayer), C.c_int32, C.c_int64, C.c_int, C.c_int,
                                       C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qlr_linear_bwd": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_int64,
                                 C.POINTER(CQWeight), C.c_void_p, C.c_void_p, C.c_int, C.c_int32,
                                 C.c_float, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_size_t, C.c_void_p]),
    "qlr_linear_fwd_dba": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.POINTER(CQWeight), C.POINTER(CDba),
                                     C.c_void_p, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qlr_quantize_outliers": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                        C.c_int64, C.POINTER(CQWeight), C.POINTER(CSparse), C.c_void_p,
                                        C.c_size_t, C.c_void_p]),
    "qlr_linear_fwd_outliers": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.POINTER(CQWeight),
                                          C.POINTER(CSparse), C.c_void_p, C.c_void_p, C.c_int, C.c_int32,
                                          C.c_float, C.c_void_p, C.c_int, C.c_void_p, C.c_size_t,
                                          C.c_void_p]),
    "qlr_linear_fwd_wha": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.POINTER(CQWeight), C.POINTER(CSparse),
                                     C.c_int32, C.c_void_p, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qlr_force_path": (C.c_int, [C.c_int]),
}

_lib = None
_lock = threading.Lock()


def lib():
    """Load libqlr.so (building it first only if it does not exist).

    A library built from other sources than the ones in the tree is refused: the
    build stamps it with a hash of its sources, checked here against the tree.
    """
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            from .build import build, source_hash
            if not os.path.exists(LIB_PATH):
                build()
            handle = C.CDLL(LIB_PATH)
            try:
                built = (C.c_char * 65).in_dll(handle, "qlr_source_sha256").value.decode()
            except ValueError:
                built = ""
            if built != source_hash():
                raise RuntimeError(f"{LIB_PATH} was built from other sources than the ones in the tree; "
                                   "rebuild it (python -m quantized_base_fine_amd.build)")
            for name, (res, args) in EXPORTS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise QlrError(status, lib().qlr_last_error().decode())


# ---------------------------------------------------------------- host-only calls

def codebook(bits: int) -> List[float]:
    out = (C.c_float * (1 << bits))() if 1 <= bits <= 8 else (C.c_float * 1)()
    check(lib().qlr_codebook(bits, out))
    return list(out)


def qweight_sizes(rows: int, cols: int, bits: int, block: int = BLOCK):
    a, b, c = C.c_size_t(), C.c_size_t(), C.c_size_t()
    check(lib().qlr_qweight_sizes(rows, cols, bits, block, C.byref(a), C.byref(b), C.byref(c)))
    return a.value, b.value, c.value


def workspace_bytes(op: int, M: int = 0, N: int = 0, K: int = 0, r: int = 0) -> int:
    out = C.c_size_t()
    check(lib().qlr_workspace_bytes(op, M, N, K, r, C.byref(out)))
    return out.value


_tls = threading.local()


def force_path(path: int) -> None:
    check(lib().qlr_force_path(path))
    _tls.path = path


@contextlib.contextmanager
def path(p: int):
    prev = getattr(_tls, "path", PATH_AUTO)
    force_path(p)
    try:
        yield
    finally:
        force_path(prev)


# ---------------------------------------------------------------- device calls (torch memory)

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    return {torch.float32: QLR_F32, torch.float16: QLR_F16, torch.bfloat16: QLR_BF16}[t.dtype]


def _stream(device=None) -> C.c_void_p:
    torch = _torch()
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("qlr works on GPU tensors only")


@dataclass
class QWeight:
    """A quantized frozen weight: header + three device buffers (torch uint8/float32)."""
    bits: int
    rows: int
    cols: int
    codes: "object"
    absmax_q8: "object"
    absmax_c: "object"

    def c_struct(self) -> CQWeight:
        return CQWeight(FORMAT_VERSION, self.bits, BLOCK, GROUP, self.rows, self.cols,
                        self.codes.data_ptr(), self.absmax_q8.data_ptr(), self.absmax_c.data_ptr())

    @staticmethod
    def empty(rows: int, cols: int, bits: int, device) -> "QWeight":
        torch = _torch()
        cb, qb, kb = qweight_sizes(rows, cols, bits)
        return QWeight(bits, rows, cols,
                       torch.empty(max(cb, 1), dtype=torch.uint8, device=device),
                       torch.empty(max(qb, 1), dtype=torch.uint8, device=device),
                       torch.empty(max(kb // 4, 1), dtype=torch.float32, device=device))


def quantize(W, bits: int, out: Optional[QWeight] = None, ws=None, blocking: bool = True) -> QWeight:
    """Quantize a 2-D (rows x cols) float32/float16/bfloat16 device tensor."""
    torch = _torch()
    _require_cuda(W)
    W = W.contiguous()
    rows, cols = (W.shape[0], W.shape[1]) if W.dim() == 2 else (1, W.numel())
    qw = out or QWeight.empty(rows, cols, bits, W.device)
    if ws is None:
        ws = torch.empty(workspace_bytes(OP_QUANTIZE), dtype=torch.uint8, device=W.device)
    cw = qw.c_struct()
    fn = lib().qlr_quantize if blocking else lib().qlr_quantize_async
    check(fn(W.data_ptr(), _dt(W), rows, cols, bits, BLOCK, C.byref(cw), ws.data_ptr(),
             ws.numel(), _stream(W.device)))
    return qw


def dequantize(qw: QWeight, dtype=None):
    torch = _torch()
    dtype = dtype or torch.float32
    out = torch.empty((qw.rows, qw.cols), dtype=dtype, device=qw.codes.device)
    cw = qw.c_struct()
    check(lib().qlr_dequantize(C.byref(cw), out.data_ptr(), _dt(out), _stream(out.device)))
    return out


def linear(x, qw: QWeight, A=None, B=None, scale: float = 0.0, out_dtype=None, out=None, ws=None):
    """y = x W'^T + scale (x A^T) B^T; x (M, K) float32/bfloat16 on the GPU."""
    torch = _torch()
    _require_cuda(x, A, B)
    M = x.shape[0]
    r = 0 if A is None else A.shape[0]
    if x.shape[1] != qw.cols:
        raise ValueError("x columns must equal the weight's cols")
    if r > 0 and (A.shape != (r, qw.cols) or B.shape != (qw.rows, r) or A.dtype != B.dtype):
        raise ValueError("A must be (r, K) and B (N, r) with one dtype")
    y = out if out is not None else torch.empty((M, qw.rows), dtype=out_dtype or x.dtype, device=x.device)
    need = workspace_bytes(OP_LINEAR, M, qw.rows, qw.cols, r)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    abdt = _dt(A) if r > 0 else QLR_BF16
    cw = qw.c_struct()
    check(lib().qlr_linear_fwd(x.data_ptr(), _dt(x), M, C.byref(cw), _ptr(A), _ptr(B), abdt, r,
                               float(scale), y.data_ptr(), _dt(y), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(x.device)))
    return y


STATIC_SCRATCH_BYTES = 8 << 20


def linear_static(x, qw: QWeight, A=None, B=None, scale: float = 0.0, out_dtype=None, out=None):
    """``linear`` through qlr_linear_fwd_static: no workspace (the library's static per-GPU
    scratch of STATIC_SCRATCH_BYTES), nothing allocated by the library.  ``out`` avoids
    the output allocation too."""
    torch = _torch()
    _require_cuda(x, A, B)
    M = x.shape[0]
    r = 0 if A is None else A.shape[0]
    if x.shape[1] != qw.cols:
        raise ValueError("x columns must equal the weight's cols")
    if r > 0 and (A.shape != (r, qw.cols) or B.shape != (qw.rows, r) or A.dtype != B.dtype):
        raise ValueError("A must be (r, K) and B (N, r) with one dtype")
    y = out if out is not None else torch.empty((M, qw.rows), dtype=out_dtype or x.dtype, device=x.device)
    abdt = _dt(A) if r > 0 else QLR_BF16
    cw = qw.c_struct()
    check(lib().qlr_linear_fwd_static(x.data_ptr(), _dt(x), M, C.byref(cw), _ptr(A), _ptr(B), abdt, r,
                                      float(scale), y.data_ptr(), _dt(y), _stream(x.device)))
    return y


class LinearCall:
    """A prepared ``qlr_linear_fwd`` call: the arguments are marshalled once, so a
    repeated call (a decode loop) costs one foreign call.  The tensors are kept
    alive by the object; their contents may change between calls, their
    storage may not."""

    def __init__(self, x, qw: QWeight, A=None, B=None, scale: float = 0.0, out=None, ws=None,
                 out_dtype=None):
        torch = _torch()
        _require_cuda(x, A, B)
        M = x.shape[0]
        r = 0 if A is None else A.shape[0]
        if x.shape[1] != qw.cols:
            raise ValueError("x columns must equal the weight's cols")
        if r > 0 and (A.shape != (r, qw.cols) or B.shape != (qw.rows, r) or A.dtype != B.dtype):
            raise ValueError("A must be (r, K) and B (N, r) with one dtype")
        self.y = out if out is not None else torch.empty((M, qw.rows), dtype=out_dtype or x.dtype,
                                                         device=x.device)
        need = workspace_bytes(OP_LINEAR, M, qw.rows, qw.cols, r)
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        self._keep = (x, qw, A, B, ws)
        self._cw = qw.c_struct()
        abdt = _dt(A) if r > 0 else QLR_BF16
        self._args = (x.data_ptr(), _dt(x), M, C.byref(self._cw), _ptr(A), _ptr(B), abdt, r, float(scale),
                      self.y.data_ptr(), _dt(self.y), _ptr(ws), 0 if ws is None else ws.numel(),
                      _stream(x.device))
        self._fn = lib().qlr_linear_fwd

    def __call__(self):
        check(self._fn(*self._args))
        return self.y


class MixedCall:
    """A prepared ``qlr_linear_fwd_mixed`` call over independent linears with per-entry
    (bits, rank); each entry is dict(x, qw, A, B, scale[, y]).  Marshalled once; the
    tensors are kept alive by the object."""

    def __init__(self, entries: Sequence[dict], out_dtype=None, ws=None):
        torch = _torch()
        self.ys = []
        self._fn = None
        if not entries:
            return
        x0 = entries[0]["x"]
        M = x0.shape[0]
        cws = []
        need = 0
        abdt = QLR_BF16
        for e in entries:
            qw, x, A, B = e["qw"], e["x"], e.get("A"), e.get("B")
            _require_cuda(x, A, B)
            r = 0 if A is None else A.shape[0]
            if r > 0:
                abdt = _dt(A)
            y = e.get("y")
            if y is None:
                y = torch.empty((M, qw.rows), dtype=out_dtype or x.dtype, device=x.device)
            self.ys.append(y)
            cws.append(qw.c_struct())
            need += workspace_bytes(OP_LINEAR, M, qw.rows, qw.cols, r)
        arr = (CLayer * len(entries))()
        for i, e in enumerate(entries):
            r = 0 if e.get("A") is None else e["A"].shape[0]
            arr[i] = CLayer(C.pointer(cws[i]), e["x"].data_ptr(), _ptr(e.get("A")), _ptr(e.get("B")), r,
                            float(e.get("scale", 0.0)), self.ys[i].data_ptr())
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=x0.device)
        self._keep = (list(entries), cws, arr, ws)
        self._args = (arr, len(entries), M, _dt(x0), abdt, _dt(self.ys[0]), _ptr(ws),
                      0 if ws is None else ws.numel(), _stream(x0.device))
        self._fn = lib().qlr_linear_fwd_mixed

    def __call__(self):
        if self._fn is not None:
            check(self._fn(*self._args))
        return self.ys


def linear_mixed(entries: Sequence[dict], out_dtype=None, ws=None):
    """Independent linears with per-entry (bits, rank).  Each entry: dict(x, qw, A, B, scale[, y])."""
    return MixedCall(entries, out_dtype=out_dtype, ws=ws)()


class LinearBwdCall:
    """A prepared ``qlr_linear_bwd`` call: dx = dy W' + scale (dy B) A,
    dA = scale (dy B)^T x, dB = scale dy^T (x A^T).  dy (M, N) and x (M, K) on the
    GPU; dA and dB are float32; ``need_dx=False`` skips the input gradient.
    Marshalled once (the stream current at construction is used); the tensors
    are kept alive by the object."""

    def __init__(self, dy, x, qw: QWeight, A=None, B=None, scale: float = 0.0, dx_dtype=None,
                 need_dx: bool = True, dx=None, dA=None, dB=None, ws=None):
        torch = _torch()
        _require_cuda(dy, x, A, B)
        M = dy.shape[0]
        r = 0 if A is None else A.shape[0]
        if dy.shape[1] != qw.rows or (x is not None and x.shape != (M, qw.cols)):
            raise ValueError("dy must be (M, N) and x (M, K) for an N x K weight")
        if r > 0 and (A.shape != (r, qw.cols) or B.shape != (qw.rows, r) or A.dtype != B.dtype):
            raise ValueError("A must be (r, K) and B (N, r) with one dtype")
        dev = dy.device
        if need_dx and dx is None:
            dx = torch.empty((M, qw.cols), dtype=dx_dtype or dy.dtype, device=dev)
        self.dx = dx if need_dx else None
        if r > 0:
            self.dA = dA if dA is not None else torch.empty((r, qw.cols), dtype=torch.float32, device=dev)
            self.dB = dB if dB is not None else torch.empty((qw.rows, r), dtype=torch.float32, device=dev)
        else:
            self.dA = self.dB = None
        need = workspace_bytes(OP_LINEAR_BWD, M, qw.rows, qw.cols, r)
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        self._keep = (dy, x, qw, A, B, ws)
        self._cw = qw.c_struct()
        abdt = _dt(A) if r > 0 else QLR_BF16
        xdt = _dt(x) if x is not None else _dt(dy)
        self._args = (dy.data_ptr(), _dt(dy), _ptr(x), xdt, M, C.byref(self._cw), _ptr(A), _ptr(B), abdt, r,
                      float(scale), _ptr(self.dx), _dt(self.dx) if self.dx is not None else QLR_F32,
                      _ptr(self.dA), _ptr(self.dB), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
        self._fn = lib().qlr_linear_bwd

    def __call__(self):
        check(self._fn(*self._args))
        return self.dx, self.dA, self.dB


def linear_bwd(dy, x, qw: QWeight, A=None, B=None, scale: float = 0.0, dx_dtype=None, need_dx: bool = True):
    """Gradients (dx, dA, dB) of the layer for an upstream gradient dy; see LinearBwdCall."""
    return LinearBwdCall(dy, x, qw, A, B, scale, dx_dtype=dx_dtype, need_dx=need_dx)()


class DbaCall:
    """A prepared ``qlr_linear_fwd_dba`` call: y = x W'^T + the double-binary adapter
    branch.  ``b1`` (N, ceil(R/32)) and ``b2`` (R, ceil(K/32)) are int32/uint32
    device tensors of sign words; ``alpha`` (l, N), ``beta`` (l, R), ``gamma`` (l, K)
    float16 device tensors.  Marshalled once (the stream current at construction
    is used); the tensors are kept alive by the object."""

    def __init__(self, x, qw: QWeight, b1, b2, alpha, beta, gamma, out_dtype=None, out=None, ws=None):
        torch = _torch()
        _require_cuda(x, b1, b2, alpha, beta, gamma)
        M = x.shape[0]
        ell, R = beta.shape
        if x.shape[1] != qw.cols or alpha.shape != (ell, qw.rows) or gamma.shape != (ell, qw.cols):
            raise ValueError("x (M, K), alpha (l, N), beta (l, R), gamma (l, K) do not fit the weight")
        if b1.shape != (qw.rows, (R + 31) // 32) or b2.shape != (R, (qw.cols + 31) // 32):
            raise ValueError("sign words must be (N, ceil(R/32)) and (R, ceil(K/32))")
        if any(t.dtype != torch.float16 for t in (alpha, beta, gamma)):
            raise ValueError("alpha, beta, gamma must be float16")
        self.y = out if out is not None else torch.empty((M, qw.rows), dtype=out_dtype or x.dtype, device=x.device)
        need = workspace_bytes(OP_LINEAR_DBA, M, qw.rows, qw.cols, R * ell)
        if ws is None:
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
        tensors = [t.contiguous() for t in (b1, b2, alpha, beta, gamma)]
        self._keep = (x, qw, ws, tensors)
        self._cw = qw.c_struct()
        self._ad = CDba(R, ell, *[t.data_ptr() for t in tensors])
        self._args = (x.data_ptr(), _dt(x), M, C.byref(self._cw), C.byref(self._ad), self.y.data_ptr(),
                      _dt(self.y), ws.data_ptr(), ws.numel(), _stream(x.device))
        self._fn = lib().qlr_linear_fwd_dba

    def __call__(self):
        check(self._fn(*self._args))
        return self.y


def linear_dba(x, qw: QWeight, b1, b2, alpha, beta, gamma, out_dtype=None):
    """y = x W'^T + sum_i alpha_i * (((x * gamma_i) B2^T) * beta_i) B1^T; see DbaCall."""
    return DbaCall(x, qw, b1, b2, alpha, beta, gamma, out_dtype=out_dtype)()


@dataclass
class Sparse:
    """The CSR outlier side channel of a weight: row_ptr (rows + 1) and col (nnz)
    int32, val (nnz) float32, all on the device."""
    rows: int
    cols: int
    nnz: int
    row_ptr: "object"
    col: "object"
    val: "object"
    # largest entry count of a group of 128 rows starting at a multiple of 128 (set by
    # quantize_outliers), -1 when not known
    max_group_nnz: int = -1

    def c_struct(self) -> CSparse:
        return CSparse(self.rows, self.cols, self.nnz, self.row_ptr.data_ptr(), self.col.data_ptr(),
                       self.val.data_ptr(), self.max_group_nnz)

    @staticmethod
    def empty(rows: int, cols: int, nnz: int, device) -> "Sparse":
        torch = _torch()
        return Sparse(rows, cols, nnz, torch.empty(rows + 1, dtype=torch.int32, device=device),
                      torch.empty(max(nnz, 1), dtype=torch.int32, device=device),
                      torch.empty(max(nnz, 1), dtype=torch.float32, device=device))


def quantize_outliers(W, bits: int, k: int, out: Optional[QWeight] = None, sparse: Optional[Sparse] = None,
                      ws=None):
    """(QWeight of the dense part, Sparse residuals of the k largest-|w| entries) of a 2-D device tensor."""
    torch = _torch()
    _require_cuda(W)
    W = W.contiguous()
    rows, cols = W.shape
    qw = out or QWeight.empty(rows, cols, bits, W.device)
    sp = sparse or Sparse.empty(rows, cols, k, W.device)
    if ws is None:
        ws = torch.empty(workspace_bytes(OP_QUANTIZE_OUTLIERS, k, rows, cols), dtype=torch.uint8,
                         device=W.device)
    cw, cs = qw.c_struct(), sp.c_struct()
    check(lib().qlr_quantize_outliers(W.data_ptr(), _dt(W), rows, cols, bits, BLOCK, k, C.byref(cw), C.byref(cs),
                                      ws.data_ptr(), ws.numel(), _stream(W.device)))
    sp.max_group_nnz = int(cs.max_group_nnz)
    return qw, sp


class OutliersCall:
    """A prepared ``qlr_linear_fwd_outliers`` call: y = x W'^T + x S^T + scale (x A^T) B^T.
    Marshalled once (the stream current at construction is used); the tensors are
    kept alive by the object."""

    def __init__(self, x, qw: QWeight, sp: Sparse, A=None, B=None, scale: float = 0.0, out_dtype=None, out=None,
                 ws=None):
        torch = _torch()
        _require_cuda(x, A, B)
        M = x.shape[0]
        r = 0 if A is None else A.shape[0]
        if x.shape[1] != qw.cols or (sp.rows, sp.cols) != (qw.rows, qw.cols):
            raise ValueError("x (M, K) and the sparse part must fit the weight")
        if r > 0 and (A.shape != (r, qw.cols) or B.shape != (qw.rows, r) or A.dtype != B.dtype):
            raise ValueError("A must be (r, K) and B (N, r) with one dtype")
        self.y = out if out is not None else torch.empty((M, qw.rows), dtype=out_dtype or x.dtype, device=x.device)
        need = workspace_bytes(OP_LINEAR_OUTLIERS, M, qw.rows, qw.cols, r)
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        self._keep = (x, qw, sp, A, B, ws)
        self._cw, self._cs = qw.c_struct(), sp.c_struct()
        abdt = _dt(A) if r > 0 else QLR_BF16
        self._args = (x.data_ptr(), _dt(x), M, C.byref(self._cw), C.byref(self._cs), _ptr(A), _ptr(B), abdt, r,
                      float(scale), self.y.data_ptr(), _dt(self.y), _ptr(ws), 0 if ws is None else ws.numel(),
                      _stream(x.device))
        self._fn = lib().qlr_linear_fwd_outliers

    def __call__(self):
        check(self._fn(*self._args))
        return self.y


def linear_outliers(x, qw: QWeight, sp: Sparse, A=None, B=None, scale: float = 0.0, out_dtype=None):
    """y = x W'^T + x S^T + scale (x A^T) B^T; see OutliersCall."""
    return OutliersCall(x, qw, sp, A, B, scale, out_dtype=out_dtype)()


class WhaCall:
    """A prepared ``qlr_linear_fwd_wha`` call: y = x W'^T + x (F H^-1)^T with H the
    Walsh-Hadamard matrix in blocks of ``hblock`` columns and F the sparse
    coefficients (a ``Sparse`` of the weight's shape).  Marshalled once (the
    stream current at construction is used); the tensors are kept alive by the object."""

    def __init__(self, x, qw: QWeight, F: Sparse, hblock: int, out_dtype=None, out=None, ws=None):
        torch = _torch()
        _require_cuda(x)
        M = x.shape[0]
        if x.shape[1] != qw.cols or (F.rows, F.cols) != (qw.rows, qw.cols):
            raise ValueError("x (M, K) and F must fit the weight")
        self.y = out if out is not None else torch.empty((M, qw.rows), dtype=out_dtype or x.dtype, device=x.device)
        need = workspace_bytes(OP_LINEAR_WHA, M, qw.rows, qw.cols)
        if ws is None and need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        self._keep = (x, qw, F, ws)
        self._cw, self._cf = qw.c_struct(), F.c_struct()
        self._args = (x.data_ptr(), _dt(x), M, C.byref(self._cw), C.byref(self._cf), int(hblock), self.y.data_ptr(),
                      _dt(self.y), _ptr(ws), 0 if ws is None else ws.numel(), _stream(x.device))
        self._fn = lib().qlr_linear_fwd_wha

    def __call__(self):
        check(self._fn(*self._args))
        return self.y


def linear_wha(x, qw: QWeight, F: Sparse, hblock: int, out_dtype=None):
    """y = x W'^T + x (F H^-1)^T; see WhaCall."""
    return WhaCall(x, qw, F, hblock, out_dtype=out_dtype)()


def sparse_from_csr(rows: int, cols: int, row_ptr, col, val, device) -> Sparse:
    """A ``Sparse`` on the device from host CSR arrays (int32 offsets and columns, float32 values)."""
    torch = _torch()
    nnz = int(row_ptr[-1])
    sp = Sparse.empty(rows, cols, nnz, device)
    sp.row_ptr.copy_(torch.as_tensor(row_ptr, dtype=torch.int32))
    if nnz > 0:
        sp.col[:nnz].copy_(torch.as_tensor(col, dtype=torch.int32))
        sp.val[:nnz].copy_(torch.as_tensor(val, dtype=torch.float32))
    return sp
