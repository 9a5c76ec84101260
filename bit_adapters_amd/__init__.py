"""Python binding of libdbf, the gfx950 double-binary factorized linear layer.

The functions carry the names of the C entry points in include/dbf.h and do
argument marshalling only: they take torch tensors that live on the current
HIP device, pass their data pointers, sizes and the current stream to the
library, and raise ``DbfError`` on a non-zero status.  Every step of the
computation runs in the library's kernels; torch provides device memory and
the stream.  The library is loaded on first use; if ``libdbf.so`` has not been built
(``python -m bit_adapters_amd.build``) that use raises ImportError: there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libdbf.so")

_i64, _vp, _int, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t

DBF_OK, DBF_EINVAL, DBF_EDTYPE, DBF_EALIGN = 0, -1, -2, -3
DBF_EWORKSPACE, DBF_EDEVICE, DBF_EUNSUPPORTED, DBF_ELAUNCH = -4, -5, -6, -7
DBF_ESTALLED = -8
DBF_F16, DBF_BF16, DBF_F32, DBF_I8, DBF_I32 = 1, 2, 3, 4, 5
DBF_PATH_AUTO, DBF_PATH_DECODE, DBF_PATH_MFMA = 0, 1, 2
DBF_MAX_TERMS = 8
DBF_WS_HEAD_BYTES = 16640
DBF_MAX_ADAPTERS = 32
DBF_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = ("dbf_abi_version", "dbf_layout_version", "dbf_last_error",
           "dbf_packed_bytes", "dbf_pack", "dbf_unpack", "dbf_workspace_bytes",
           "dbf_linear_forward", "dbf_linear_forward_noalloc", "dbf_linear_forward_i8",
           "lordba_adapter_forward", "dbf_workspace_check",
           "dbf_bool_workspace_bytes", "dbf_bool_forward", "dbf_transpose_packed",
           "dbf_backward_workspace_bytes", "dbf_linear_backward",
           "lordba_multi_adapter_forward", "dbf_svid_workspace_bytes", "dbf_svid_extract")


class _CTerm(ctypes.Structure):
    _fields_ = [("b1", _vp), ("b2", _vp), ("alpha", _vp), ("beta", _vp),
                ("gamma", _vp)]


_lib_handle = None


def library() -> ctypes.CDLL:
    """The loaded libdbf.so (loaded on first use; there is no fallback)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIBRARY):
        raise ImportError(
            "libdbf.so is not built; run `python -m bit_adapters_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIBRARY)
    lib.dbf_abi_version.restype = _int
    lib.dbf_layout_version.restype = _int
    lib.dbf_last_error.restype = ctypes.c_char_p
    lib.dbf_packed_bytes.restype = _sz
    lib.dbf_packed_bytes.argtypes = [_i64, _i64]
    lib.dbf_pack.restype = _int
    lib.dbf_pack.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _vp]
    lib.dbf_unpack.restype = _int
    lib.dbf_unpack.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp]
    lib.dbf_workspace_bytes.restype = _sz
    lib.dbf_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _i64, _int]
    lib.dbf_linear_forward.restype = _int
    lib.dbf_linear_forward.argtypes = [
        ctypes.POINTER(_CTerm), _int, _i64, _i64, _i64, _vp, _int, _i64, _i64,
        _vp, _int, _i64, _int, _vp, _sz, _int, _vp]
    lib.dbf_linear_forward_noalloc.restype = _int
    lib.dbf_linear_forward_noalloc.argtypes = [
        ctypes.POINTER(_CTerm), _int, _i64, _i64, _i64, _vp, _int, _i64, _i64,
        _vp, _int, _i64, _int, _int, _vp]
    lib.dbf_linear_forward_i8.restype = _int
    lib.dbf_linear_forward_i8.argtypes = [
        ctypes.POINTER(_CTerm), _int, _i64, _i64, _i64, _vp, _i64, _i64, _vp,
        _vp, _vp, _int, _i64, _vp, _sz, _vp]
    lib.lordba_adapter_forward.restype = _int
    lib.lordba_adapter_forward.argtypes = [
        _vp, _i64, ctypes.POINTER(_CTerm), _int, _i64, _i64, _i64, _vp, _i64,
        _i64, _vp, _int, _i64, _vp, _sz, _vp]
    lib.dbf_workspace_check.restype = _int
    lib.dbf_workspace_check.argtypes = [_vp, _vp]
    lib.dbf_transpose_packed.restype = _int
    lib.dbf_transpose_packed.argtypes = [_vp, _i64, _i64, _vp, _vp]
    lib.dbf_backward_workspace_bytes.restype = _sz
    lib.dbf_backward_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _i64, _int]
    lib.dbf_linear_backward.restype = _int
    lib.dbf_linear_backward.argtypes = [
        ctypes.POINTER(_CTerm), ctypes.POINTER(_CTermT), _int, _i64, _i64, _i64,
        _vp, _int, _i64, _vp, _int, _i64, _i64, _vp, _int, _i64, _vp, _vp, _vp,
        _vp, _sz, _int, _vp]
    lib.lordba_multi_adapter_forward.restype = _int
    lib.lordba_multi_adapter_forward.argtypes = [
        _vp, _i64, ctypes.POINTER(_CTerm), _int, _i64, _i64, _i64, _vp, _vp, _i64, _i64,
        _vp, _int, _i64, _vp, _sz, _vp]
    lib.dbf_bool_workspace_bytes.restype = _sz
    lib.dbf_bool_workspace_bytes.argtypes = [_i64, _i64, _int, _i64, _int]
    lib.dbf_bool_forward.restype = _int
    lib.dbf_bool_forward.argtypes = [
        ctypes.POINTER(_CBool), _int, _i64, _i64, _vp, _int, _i64, _i64, _vp,
        _int, _i64, _int, _vp, _sz, _int, _vp]
    lib.dbf_svid_workspace_bytes.restype = _sz
    lib.dbf_svid_workspace_bytes.argtypes = [_i64, _i64]
    lib.dbf_svid_extract.restype = _int
    lib.dbf_svid_extract.argtypes = [
        _vp, _int, _i64, _i64, _i64, _int, ctypes.POINTER(_CBoolOut), _int, _vp, _vp, _sz, _vp]
    _lib_handle = lib
    return lib


class DbfError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("dbf status %d: %s" % (code, message))
        self.code = code


class DbfTerm(NamedTuple):
    """One term: packed b1 (N x R layout), packed b2 (R x M layout), fp16
    alpha (N), beta (R), gamma (M); None where the entry point allows."""
    b1: torch.Tensor
    b2: torch.Tensor
    alpha: Optional[torch.Tensor]
    beta: Optional[torch.Tensor]
    gamma: Optional[torch.Tensor]


_DT = {torch.float16: DBF_F16, torch.bfloat16: DBF_BF16,
       torch.float32: DBF_F32, torch.int8: DBF_I8, torch.int32: DBF_I32}


def _check(rc: int) -> None:
    if rc != DBF_OK:
        raise DbfError(rc, library().dbf_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return getattr(stream, "cuda_stream", stream)


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


class DbfTermT(NamedTuple):
    """The packed transposes of one term's factors: b1t (R x N layout) and
    b2t (M x R layout), from dbf_transpose_packed."""
    b1t: torch.Tensor
    b2t: torch.Tensor


class _CTermT(ctypes.Structure):
    _fields_ = [("b1t", _vp), ("b2t", _vp)]


class DbfBoolKernel(NamedTuple):
    """One boolean kernel of the Multi-Boolean form: packed signs w (N x M
    layout), fp16 s_in (M) and s_out (N)."""
    w: torch.Tensor
    s_in: torch.Tensor
    s_out: torch.Tensor


class _CBool(ctypes.Structure):
    _fields_ = [("w", _vp), ("s_in", _vp), ("s_out", _vp)]


class _CBoolOut(ctypes.Structure):
    _fields_ = [("w", _vp), ("s_in", _vp), ("s_out", _vp)]


def _bool_kernels(kernels: Sequence[DbfBoolKernel]):
    arr = (_CBool * max(1, len(kernels)))()
    for i, k in enumerate(kernels):
        arr[i] = _CBool(_ptr(k.w), _ptr(k.s_in), _ptr(k.s_out))
    return arr


def _terms(terms: Sequence[DbfTerm]):
    arr = (_CTerm * max(1, len(terms)))()
    for i, t in enumerate(terms):
        arr[i] = _CTerm(_ptr(t.b1), _ptr(t.b2), _ptr(t.alpha), _ptr(t.beta),
                        _ptr(t.gamma))
    return arr


def dbf_abi_version() -> int:
    return library().dbf_abi_version()


def dbf_layout_version() -> int:
    return library().dbf_layout_version()


def dbf_last_error() -> str:
    return library().dbf_last_error().decode()


def dbf_packed_bytes(rows: int, k: int) -> int:
    return int(library().dbf_packed_bytes(rows, k))


def dbf_workspace_bytes(N: int, M: int, R: int, n_terms: int, T: int,
                        path: int = DBF_PATH_AUTO) -> int:
    return int(library().dbf_workspace_bytes(N, M, R, n_terms, T, path))


def dbf_bool_workspace_bytes(N: int, M: int, n_kernels: int, T: int,
                             path: int = DBF_PATH_AUTO) -> int:
    return int(library().dbf_bool_workspace_bytes(N, M, n_kernels, T, path))


def dbf_bool_forward(kernels: Sequence[DbfBoolKernel], N: int, M: int,
                     x: torch.Tensor, y: Optional[torch.Tensor] = None,
                     y_dtype: torch.dtype = torch.float32,
                     accumulate: bool = False, ws: Optional[torch.Tensor] = None,
                     path: int = DBF_PATH_AUTO, stream=None) -> torch.Tensor:
    """y (+)= sum_k s_out_k . (Wb_k (s_in_k . x)) for x [T x M] (bf16 or f16)."""
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, N), dtype=y_dtype, device=x.device)
    ws, wsb = _workspace(dbf_bool_workspace_bytes(N, M, len(kernels), T, path),
                         x.device, ws)
    _check(library().dbf_bool_forward(
        _bool_kernels(kernels), len(kernels), N, M, _ptr(x), _DT.get(x.dtype, -1),
        T, _ld(x), _ptr(y), _DT.get(y.dtype, -1), _ld(y), int(accumulate),
        _ptr(ws), wsb, path, _stream(stream)))
    return y


def dbf_svid_workspace_bytes(N: int, M: int) -> int:
    return int(library().dbf_svid_workspace_bytes(N, M))


def dbf_svid_extract(w: torch.Tensor, n_kernels: int, iters: int = 32,
                     ws: Optional[torch.Tensor] = None, residual: bool = False,
                     stream=None):
    """Successive SVID of w [N x M] (f32, bf16 or f16, device) into n_kernels
    boolean kernels.  Returns a list of DbfBoolKernel (packed signs, fp16
    s_in, fp16 s_out), plus the float [n_kernels] squared residual norms if
    residual is set."""
    N, M = w.shape
    dev = w.device
    outs = [DbfBoolKernel(torch.empty(dbf_packed_bytes(N, M) // 4, dtype=torch.int32, device=dev),
                          torch.empty(M, dtype=torch.float16, device=dev),
                          torch.empty(N, dtype=torch.float16, device=dev))
            for _ in range(n_kernels)]
    arr = (_CBoolOut * n_kernels)()
    for i, k in enumerate(outs):
        arr[i] = _CBoolOut(_ptr(k.w), _ptr(k.s_in), _ptr(k.s_out))
    res = torch.empty(n_kernels, dtype=torch.float32, device=dev) if residual else None
    nb = dbf_svid_workspace_bytes(N, M)
    if ws is None:
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    _check(library().dbf_svid_extract(_ptr(w), _DT.get(w.dtype, -1), N, M, _ld(w), n_kernels,
                                       arr, iters, _ptr(res), _ptr(ws), ws.numel(),
                                       _stream(stream)))
    return (outs, res) if residual else outs


def dbf_transpose_packed(packed: torch.Tensor, rows: int, k: int,
                         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The packed layout of S^T (k x rows) from that of S (rows x k)."""
    if out is None:
        out = torch.empty(dbf_packed_bytes(k, rows) // 4, dtype=torch.int32,
                          device=packed.device)
    _check(library().dbf_transpose_packed(_ptr(packed), rows, k, _ptr(out), _stream(stream)))
    return out


def dbf_term_t(term: DbfTerm, N: int, M: int, R: int, stream=None) -> DbfTermT:
    """The transposes a term's backward needs, packed on the device."""
    return DbfTermT(dbf_transpose_packed(term.b1, N, R, stream=stream),
                    dbf_transpose_packed(term.b2, R, M, stream=stream))


def dbf_backward_workspace_bytes(N: int, M: int, R: int, n_terms: int, T: int,
                                 path: int = DBF_PATH_AUTO) -> int:
    return int(library().dbf_backward_workspace_bytes(N, M, R, n_terms, T, path))


def dbf_linear_backward(terms: Sequence[DbfTerm], tterms: Sequence[DbfTermT], N: int,
                        M: int, R: int, x: torch.Tensor, dy: torch.Tensor,
                        dx_dtype: torch.dtype = torch.float32, want_dx: bool = True,
                        want_scales: bool = True, ws: Optional[torch.Tensor] = None,
                        path: int = DBF_PATH_AUTO, stream=None):
    """(dx [T x M] or None, [(dalpha, dbeta, dgamma)] per term or None) for
    dy = dL/dy [T x N]."""
    T = x.shape[0]
    L_ = len(terms)
    dev = x.device
    dx = torch.empty((T, M), dtype=dx_dtype, device=dev) if want_dx else None
    da = db = dg = None
    if want_scales:
        da = torch.empty((L_, N), dtype=torch.float32, device=dev)
        db = torch.empty((L_, R), dtype=torch.float32, device=dev)
        dg = torch.empty((L_, M), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(dbf_backward_workspace_bytes(N, M, R, L_, T, path), dev, ws)
    tt = (_CTermT * max(1, L_))()
    for i, t in enumerate(tterms):
        tt[i] = _CTermT(_ptr(t.b1t), _ptr(t.b2t))
    _check(library().dbf_linear_backward(
        _terms(terms), tt, L_, N, M, R, _ptr(x), _DT.get(x.dtype, -1), _ld(x), _ptr(dy),
        _DT.get(dy.dtype, -1), _ld(dy), T, _ptr(dx), _DT.get(dx_dtype, -1),
        _ld(dx) if dx is not None else M, _ptr(da), _ptr(db), _ptr(dg), _ptr(ws), wsb,
        path, _stream(stream)))
    scales = [(da[i], db[i], dg[i]) for i in range(L_)] if want_scales else None
    return dx, scales


def lordba_multi_adapter_forward(w0: torch.Tensor, adapters: Sequence[DbfTerm], N: int,
                                 M: int, R: int, adapter_idx: torch.Tensor, x: torch.Tensor,
                                 y: Optional[torch.Tensor] = None,
                                 y_dtype: torch.dtype = torch.float32,
                                 ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y[t] = W0 x[t] + Delta W_{adapter_idx[t]} x[t] (int32 indices on the
    device, -1 = base only)."""
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, N), dtype=y_dtype, device=x.device)
    ws, wsb = _workspace(dbf_workspace_bytes(N, M, R, 1, T, DBF_PATH_DECODE), x.device, ws)
    _check(library().lordba_multi_adapter_forward(
        _ptr(w0), _ld(w0), _terms(adapters), len(adapters), N, M, R, _ptr(adapter_idx),
        _ptr(x), T, _ld(x), _ptr(y), _DT.get(y.dtype, -1), _ld(y), _ptr(ws), wsb,
        _stream(stream)))
    return y


def dbf_workspace_check(ws: Optional[torch.Tensor], stream=None) -> None:
    """Raise DbfError(DBF_ESTALLED) if a handoff wait of an earlier call on
    this workspace gave up (the head is then cleared); waits for the stream."""
    _check(library().dbf_workspace_check(_ptr(ws), _stream(stream)))


def dbf_pack(src: torch.Tensor, out: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """Pack the signs of src [rows x k] (int8/f16/bf16/f32, device) into the
    uint32 layout, returned as an int32 tensor of dbf_packed_bytes/4 words."""
    rows, k = src.shape
    nbytes = dbf_packed_bytes(rows, k)
    if out is None:
        out = torch.empty(nbytes // 4, dtype=torch.int32, device=src.device)
    _check(library().dbf_pack(_ptr(src), _DT.get(src.dtype, -1), rows, k, _ld(src),
                         _ptr(out), _stream(stream)))
    return out


def dbf_unpack(packed: torch.Tensor, rows: int, k: int,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int8, device=packed.device)
    _check(library().dbf_unpack(_ptr(packed), rows, k, _ptr(out), _ld(out),
                           _stream(stream)))
    return out


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    """The caller's workspace, or a new zeroed one (its first 256 bytes are
    the decode path's counters and must start at zero)."""
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def dbf_linear_forward(terms: Sequence[DbfTerm], N: int, M: int, R: int,
                       x: torch.Tensor, y: Optional[torch.Tensor] = None,
                       y_dtype: torch.dtype = torch.float32,
                       accumulate: bool = False, ws: Optional[torch.Tensor] = None,
                       path: int = DBF_PATH_AUTO, stream=None) -> torch.Tensor:
    """y (+)= sum_i Delta W_i x for x [T x M] (bf16 or f16)."""
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, N), dtype=y_dtype, device=x.device)
    ws, wsb = _workspace(dbf_workspace_bytes(N, M, R, len(terms), T, path),
                         x.device, ws)
    _check(library().dbf_linear_forward(
        _terms(terms), len(terms), N, M, R, _ptr(x), _DT.get(x.dtype, -1), T,
        _ld(x), _ptr(y), _DT.get(y.dtype, -1), _ld(y), int(accumulate),
        _ptr(ws), wsb, path, _stream(stream)))
    return y


def dbf_linear_forward_noalloc(terms: Sequence[DbfTerm], N: int, M: int, R: int,
                               x: torch.Tensor, y: Optional[torch.Tensor] = None,
                               y_dtype: torch.dtype = torch.float32,
                               accumulate: bool = False, path: int = DBF_PATH_AUTO,
                               stream=None) -> torch.Tensor:
    """dbf_linear_forward with the library's own scratch as workspace (no
    workspace argument; calls on one device must not overlap)."""
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, N), dtype=y_dtype, device=x.device)
    _check(library().dbf_linear_forward_noalloc(
        _terms(terms), len(terms), N, M, R, _ptr(x), _DT.get(x.dtype, -1), T,
        _ld(x), _ptr(y), _DT.get(y.dtype, -1), _ld(y), int(accumulate), path,
        _stream(stream)))
    return y


def dbf_linear_forward_i8(terms: Sequence[DbfTerm], N: int, M: int, R: int,
                          x: torch.Tensor, s1: Optional[torch.Tensor] = None,
                          s2: Optional[torch.Tensor] = None,
                          y: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None, stream=None):
    """Integer-activation variant; returns (s1, s2, y) as passed in."""
    T = x.shape[0]
    ws, wsb = _workspace(dbf_workspace_bytes(N, M, R, len(terms), T,
                                             DBF_PATH_DECODE), x.device, ws)
    ydt = _DT.get(y.dtype, -1) if y is not None else DBF_F32
    ldy = _ld(y) if y is not None else N
    _check(library().dbf_linear_forward_i8(
        _terms(terms), len(terms), N, M, R, _ptr(x), T, _ld(x), _ptr(s1),
        _ptr(s2), _ptr(y), ydt, ldy, _ptr(ws), wsb, _stream(stream)))
    return s1, s2, y


def lordba_adapter_forward(w0: torch.Tensor, terms: Sequence[DbfTerm], N: int,
                           M: int, R: int, x: torch.Tensor,
                           y: Optional[torch.Tensor] = None,
                           y_dtype: torch.dtype = torch.float32,
                           ws: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """y = W0 x + sum_i Delta W_i x (bf16 W0 [N x M] and x [T x M])."""
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, N), dtype=y_dtype, device=x.device)
    nb = dbf_workspace_bytes(N, M, R, len(terms), T, DBF_PATH_DECODE) if terms else 0
    ws, wsb = _workspace(nb, x.device, ws)
    _check(library().lordba_adapter_forward(
        _ptr(w0), _ld(w0), _terms(terms) if terms else None, len(terms), N, M,
        R, _ptr(x), T, _ld(x), _ptr(y), _DT.get(y.dtype, -1), _ld(y),
        _ptr(ws), wsb, _stream(stream)))
    return y
