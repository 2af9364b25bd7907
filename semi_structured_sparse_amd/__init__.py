"""Python binding of libnmsparse.so: batch-one N:M sparse matrix-vector product on MI355X.

Argument marshalling only: every step runs in the HIP kernels of the library; torch
provides device memory and the current stream. The names follow the C ABI in
include/nm_sparse.h (nm_pack, nm_spmv, nm_gemv_dense, ...). There is no CPU
fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libnmsparse.so")

PATTERNS = ((2, 4), (4, 8), (8, 16), (16, 32))
PATTERNS_QUARTER = ((1, 4), (2, 8), (4, 16), (8, 32))   # 25% density, single vector
ALL_PATTERNS = PATTERNS + PATTERNS_QUARTER

NM_OK, NM_ERR_NULL, NM_ERR_SHAPE, NM_ERR_PATTERN, NM_ERR_ALIGN, NM_ERR_TOO_WIDE, NM_ERR_HIP, NM_ERR_SCRATCH = range(8)

# Every symbol the public headers declare, with (restype, argtypes).
_c = ctypes
SIGNATURES = {
    "nm_values_count": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int, _c.c_int]),
    "nm_masks_count": (_c.c_size_t, [_c.c_int64, _c.c_int64]),
    "nm_max_cols": (_c.c_int64, []),
    "nm_pack": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                           _c.c_int, _c.c_int, _c.c_void_p]),
    "nm_unpack": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                             _c.c_int, _c.c_int, _c.c_void_p]),
    "nm_spmv": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                           _c.c_int64, _c.c_int, _c.c_int, _c.c_void_p]),
    "nm_gemv_dense": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                                 _c.c_void_p]),
    "nm_spmv_group": (_c.c_int, [_c.c_int, _c.POINTER(_c.c_void_p), _c.POINTER(_c.c_void_p), _c.c_void_p,
                                 _c.POINTER(_c.c_void_p), _c.POINTER(_c.c_int64), _c.c_int64, _c.c_int, _c.c_int,
                                 _c.c_void_p]),
    "nm_spmm": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                           _c.c_int64, _c.c_int64, _c.c_int, _c.c_int, _c.c_void_p]),
    "nm_spmm_ws": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                              _c.c_int64, _c.c_int, _c.c_int, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "nm_spmm_workspace_bytes": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int]),
    "nm_spmm_noalloc": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                                   _c.c_int64, _c.c_int64, _c.c_int, _c.c_int, _c.c_void_p]),
    "nm_spmm_skinny": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                                  _c.c_int64, _c.c_int64, _c.c_int, _c.c_int, _c.c_void_p]),
    "nm_gemm_dense": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                                 _c.c_int64, _c.c_void_p]),
    "nm_spmm_prefill": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                                   _c.c_int64, _c.c_int64, _c.c_int, _c.c_int, _c.c_void_p]),
    "nm_gemm_dense_prefill": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int64,
                                         _c.c_int64, _c.c_void_p]),
    "nm_prefill_variant": (_c.c_char_p, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "nm_spmm_variant": (_c.c_char_p, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int]),
    "nm_spmm_ws_variant": (_c.c_char_p, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_int]),
    "nm_status_string": (_c.c_char_p, [_c.c_int]),
    "nm_spmv_variant": (_c.c_char_p, [_c.c_int64, _c.c_int64, _c.c_int, _c.c_int]),
    "nm_last_hip_error": (_c.c_int, []),
    "nm_spmv_launch_shape": (_c.c_int, [_c.c_int64, _c.c_int64, _c.c_int, _c.c_int,
                                        _c.POINTER(_c.c_int64)]),
    "nm_probe_read": (_c.c_int, [_c.c_void_p, _c.c_size_t, _c.c_void_p, _c.c_uint32, _c.c_void_p]),
    "nm_probe_read_shaped": (_c.c_int, [_c.c_void_p, _c.c_size_t, _c.c_void_p, _c.c_uint32, _c.c_int, _c.c_int,
                                        _c.c_int, _c.c_int, _c.c_void_p]),
    "nm_probe_copy": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
}

_lib = None
_lock = threading.Lock()


class NMError(RuntimeError):
    """A libnmsparse call returned a non-zero status."""

    def __init__(self, fn: str, status: int, hip_error: int | None = None):
        msg = f"{fn}: {status_string(status)} (status {status})"
        if hip_error is not None:
            msg += f", hipError {hip_error}"
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


class NMArgumentError(NMError, ValueError):
    """Invalid arguments rejected before any HIP call."""


def lib() -> ctypes.CDLL:
    """The loaded library, with argtypes set. Raises if it is not built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is not built: run `python -m semi_structured_sparse_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().nm_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status == NM_OK:
        return
    if status == NM_ERR_HIP:
        raise NMError(fn, status, lib().nm_last_hip_error())
    raise NMArgumentError(fn, status)


def values_count(rows: int, cols: int, N: int, M: int) -> int:
    return int(lib().nm_values_count(rows, cols, N, M))


def masks_count(rows: int, cols: int) -> int:
    return int(lib().nm_masks_count(rows, cols))


def max_cols() -> int:
    return int(lib().nm_max_cols())


def spmv_variant(rows: int, cols: int, N: int, M: int) -> str:
    """Kernel configuration nm_spmv launches for this shape on the current device."""
    return lib().nm_spmv_variant(rows, cols, N, M).decode()


def spmv_launch_shape(rows: int, cols: int, N: int, M: int) -> dict:
    """Workgroup shape nm_spmv uses for this shape on the current device."""
    out = (ctypes.c_int64 * 4)()
    _check("nm_spmv_launch_shape", lib().nm_spmv_launch_shape(rows, cols, N, M, out))
    return {"rows_per_workgroup": out[0], "row_groups": out[1], "waves_per_row_group": out[2],
            "workgroups": out[3]}


# --------------------------------------------------------------------------- torch layer
def _torch():
    import torch
    return torch


def _stream_ptr(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device (no CPU path)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def nm_pack(W, N: int, M: int):
    """Encode fp16 W [rows, cols] -> (values fp16 [rows, cols*N/M], masks int32 [rows, cols/32]).

    masks hold the uint32 mask words (viewed as int32; bit j of word w = column 32w+j).
    """
    torch = _torch()
    _require(W, "W", torch.float16, 2)
    rows, cols = W.shape
    nv = values_count(rows, cols, N, M)
    if nv == 0:
        st = NM_ERR_PATTERN if (N, M) not in ALL_PATTERNS else NM_ERR_SHAPE
        raise NMArgumentError("nm_pack", st)
    values = torch.empty((rows, cols * N // M), dtype=torch.float16, device=W.device)
    masks = torch.empty((rows, cols // 32), dtype=torch.int32, device=W.device)
    with torch.cuda.device(W.device):
        st = lib().nm_pack(W.data_ptr(), values.data_ptr(), masks.data_ptr(), rows, cols, N, M,
                           _stream_ptr(W))
    _check("nm_pack", st)
    return values, masks


def nm_unpack(values, masks, N: int, M: int, out=None):
    """Dense fp16 W' [rows, cols] from the packed (values, masks): the inverse of nm_pack."""
    torch = _torch()
    _require(values, "values", torch.float16, 2)
    _require(masks, "masks", torch.int32, 2)
    rows, words = masks.shape
    cols = words * 32
    if (N, M) in ALL_PATTERNS and values.shape != (rows, cols * N // M):
        raise ValueError(f"values shape {tuple(values.shape)} != {(rows, cols * N // M)}")
    if values.device != masks.device:
        raise ValueError("values and masks must be on one device")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float16, device=values.device)
    else:
        _require(out, "out", torch.float16, 2)
        if tuple(out.shape) != (rows, cols) or out.device != values.device:
            raise ValueError("out must be fp16 [rows, cols] on the same device")
    with torch.cuda.device(values.device):
        st = lib().nm_unpack(values.data_ptr(), masks.data_ptr(), out.data_ptr(), rows, cols, N, M,
                             _stream_ptr(values))
    _check("nm_unpack", st)
    return out


def nm_spmv(values, masks, x, N: int, M: int, out=None):
    """y = W' x for the packed (values, masks); fp16 y [rows]."""
    torch = _torch()
    _require(values, "values", torch.float16, 2)
    _require(masks, "masks", torch.int32, 2)
    _require(x, "x", torch.float16, 1)
    rows, words = masks.shape
    cols = words * 32
    if x.shape[0] != cols:
        raise ValueError(f"x has {x.shape[0]} elements, masks describe {cols} columns")
    if (N, M) in ALL_PATTERNS and values.shape != (rows, cols * N // M):
        raise ValueError(f"values shape {tuple(values.shape)} != {(rows, cols * N // M)}")
    if not (values.device == masks.device == x.device):
        raise ValueError("values, masks and x must be on one device")
    if out is None:
        out = torch.empty(rows, dtype=torch.float16, device=x.device)
    else:
        _require(out, "out", torch.float16, 1)
        if out.shape[0] != rows or out.device != x.device:
            raise ValueError("out must be fp16 [rows] on the same device")
    with torch.cuda.device(x.device):
        st = lib().nm_spmv(values.data_ptr(), masks.data_ptr(), x.data_ptr(), out.data_ptr(),
                           rows, cols, N, M, _stream_ptr(x))
    _check("nm_spmv", st)
    return out


MAX_SPMV_GROUP = 8


def nm_spmv_group(values_list, masks_list, x, N: int, M: int, outs=None):
    """y_k = W'_k x for several packed matrices that share x and cols, in one launch;
    returns the list of fp16 y_k [rows_k]."""
    torch = _torch()
    count = len(values_list)
    if count != len(masks_list) or not 1 <= count <= MAX_SPMV_GROUP:
        raise ValueError(f"need 1..{MAX_SPMV_GROUP} (values, masks) pairs, got {count} and {len(masks_list)}")
    _require(x, "x", torch.float16, 1)
    cols = x.shape[0]
    rows = []
    for k, (values, masks) in enumerate(zip(values_list, masks_list)):
        _require(values, f"values[{k}]", torch.float16, 2)
        _require(masks, f"masks[{k}]", torch.int32, 2)
        r, words = masks.shape
        if words * 32 != cols:
            raise ValueError(f"masks[{k}] describe {words * 32} columns, x has {cols}")
        if (N, M) in ALL_PATTERNS and values.shape != (r, cols * N // M):
            raise ValueError(f"values[{k}] shape {tuple(values.shape)} != {(r, cols * N // M)}")
        if values.device != x.device or masks.device != x.device:
            raise ValueError("every matrix and x must be on one device")
        rows.append(r)
    if outs is None:
        outs = [torch.empty(r, dtype=torch.float16, device=x.device) for r in rows]
    else:
        if len(outs) != count:
            raise ValueError("one output per product")
        for k, (o, r) in enumerate(zip(outs, rows)):
            _require(o, f"outs[{k}]", torch.float16, 1)
            if o.shape[0] != r or o.device != x.device:
                raise ValueError(f"outs[{k}] must be fp16 [{r}] on the same device")
    vp = (ctypes.c_void_p * count)(*[v.data_ptr() for v in values_list])
    mp = (ctypes.c_void_p * count)(*[m.data_ptr() for m in masks_list])
    yp = (ctypes.c_void_p * count)(*[o.data_ptr() for o in outs])
    rp = (ctypes.c_int64 * count)(*rows)
    with torch.cuda.device(x.device):
        st = lib().nm_spmv_group(count, vp, mp, x.data_ptr(), yp, rp, cols, N, M, _stream_ptr(x))
    _check("nm_spmv_group", st)
    return outs


def nm_gemv_dense(W, x, out=None):
    """Dense baseline y = W x; fp16 W [rows, cols], fp16 x [cols] -> fp16 y [rows]."""
    torch = _torch()
    _require(W, "W", torch.float16, 2)
    _require(x, "x", torch.float16, 1)
    rows, cols = W.shape
    if x.shape[0] != cols:
        raise ValueError(f"x has {x.shape[0]} elements, W has {cols} columns")
    if W.device != x.device:
        raise ValueError("W and x must be on one device")
    if out is None:
        out = torch.empty(rows, dtype=torch.float16, device=x.device)
    else:
        _require(out, "out", torch.float16, 1)
        if out.shape[0] != rows or out.device != x.device:
            raise ValueError("out must be fp16 [rows] on the same device")
    with torch.cuda.device(x.device):
        st = lib().nm_gemv_dense(W.data_ptr(), x.data_ptr(), out.data_ptr(), rows, cols,
                                 _stream_ptr(x))
    _check("nm_gemv_dense", st)
    return out


def spmm_variant(rows: int, cols: int, batch: int, N: int, M: int) -> str:
    """Kernel nm_spmm launches for this shape, batch and pattern (the first, if several)."""
    return lib().nm_spmm_variant(rows, cols, batch, N, M).decode()


def spmm_ws_variant(rows: int, cols: int, batch: int, N: int, M: int) -> str:
    """Kernel nm_spmm_ws launches with a workspace of spmm_workspace_bytes (the first, if
    several)."""
    return lib().nm_spmm_ws_variant(rows, cols, batch, N, M).decode()


def prefill_variant(rows: int, cols: int, tokens: int, sparse: bool, split: bool = False,
                    expand: bool = False) -> str:
    """Kernel configuration nm_spmm_prefill (sparse; split: for 4:8 / 8:16; expand: for
    16:32) or nm_gemm_dense_prefill launches."""
    code = (3 if expand else 2 if split else 1) if sparse else 0
    return lib().nm_prefill_variant(rows, cols, tokens, code).decode()


def _batch_args(values, masks, X, N, M, out):
    torch = _torch()
    _require(values, "values", torch.float16, 2)
    _require(masks, "masks", torch.int32, 2)
    _require(X, "X", torch.float16, 2)
    rows, words = masks.shape
    cols = words * 32
    batch = X.shape[0]
    if X.shape[1] != cols:
        raise ValueError(f"X has {X.shape[1]} columns, masks describe {cols}")
    if (N, M) in ALL_PATTERNS and values.shape != (rows, cols * N // M):
        raise ValueError(f"values shape {tuple(values.shape)} != {(rows, cols * N // M)}")
    if not (values.device == masks.device == X.device):
        raise ValueError("values, masks and X must be on one device")
    if out is None:
        out = torch.empty((batch, rows), dtype=torch.float16, device=X.device)
    else:
        _require(out, "out", torch.float16, 2)
        if tuple(out.shape) != (batch, rows) or out.device != X.device:
            raise ValueError("out must be fp16 [batch, rows] on the same device")
    return rows, cols, batch, out


def nm_spmm(values, masks, X, N: int, M: int, out=None):
    """Y = X W'^T for a batch of activation vectors: X fp16 [batch, cols] -> Y fp16
    [batch, rows] (row b of Y is the packed matrix times row b of X)."""
    torch = _torch()
    rows, cols, batch, out = _batch_args(values, masks, X, N, M, out)
    with torch.cuda.device(X.device):
        st = lib().nm_spmm(values.data_ptr(), masks.data_ptr(), X.data_ptr(), out.data_ptr(),
                           rows, cols, batch, N, M, _stream_ptr(X))
    _check("nm_spmm", st)
    return out


def spmm_workspace_bytes(rows: int, cols: int, batch: int, N: int, M: int) -> int:
    """Workspace bytes nm_spmm_ws can use for this shape (0: no column split)."""
    return int(lib().nm_spmm_workspace_bytes(rows, cols, batch, N, M))


def spmm_workspace(rows: int, cols: int, batch: int, N: int, M: int, device=None):
    """A zeroed uint8 workspace for nm_spmm_ws of this shape (None when it takes none)."""
    torch = _torch()
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.device(dev):
        n = spmm_workspace_bytes(rows, cols, batch, N, M)
    return torch.zeros(n, dtype=torch.uint8, device=dev) if n > 0 else None


def nm_spmm_ws(values, masks, X, N: int, M: int, workspace=None, out=None):
    """nm_spmm with a caller-owned workspace (a uint8 device tensor whose counters start at
    zero, e.g. from spmm_workspace; None runs nm_spmm's kernels): short layers split their
    columns over several workgroups. Calls sharing a workspace must be stream-ordered."""
    torch = _torch()
    rows, cols, batch, out = _batch_args(values, masks, X, N, M, out)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _require(workspace, "workspace", torch.uint8, 1)
        if workspace.device != X.device:
            raise ValueError("workspace must be on X's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    with torch.cuda.device(X.device):
        st = lib().nm_spmm_ws(values.data_ptr(), masks.data_ptr(), X.data_ptr(), out.data_ptr(),
                              rows, cols, batch, N, M, ws_ptr, ws_bytes, _stream_ptr(X))
    _check("nm_spmm_ws", st)
    return out


def nm_spmm_noalloc(values, masks, X, N: int, M: int, out=None):
    """nm_spmm_ws with the library's static per-GPU scratch as the workspace (for callers
    that cannot allocate; calls overlapping on one GPU race). out=None allocates Y here in
    the binding, not in the library: pass `out` to allocate nothing."""
    torch = _torch()
    rows, cols, batch, out = _batch_args(values, masks, X, N, M, out)
    with torch.cuda.device(X.device):
        st = lib().nm_spmm_noalloc(values.data_ptr(), masks.data_ptr(), X.data_ptr(), out.data_ptr(),
                                   rows, cols, batch, N, M, _stream_ptr(X))
    _check("nm_spmm_noalloc", st)
    return out


def nm_spmm_skinny(values, masks, X, N: int, M: int, out=None):
    """nm_spmm's batch product on the matrix instructions for any batch and 50% pattern,
    whatever nm_spmm would pick: X fp16 [batch, cols] -> Y fp16 [batch, rows]."""
    torch = _torch()
    rows, cols, batch, out = _batch_args(values, masks, X, N, M, out)
    with torch.cuda.device(X.device):
        st = lib().nm_spmm_skinny(values.data_ptr(), masks.data_ptr(), X.data_ptr(), out.data_ptr(),
                                  rows, cols, batch, N, M, _stream_ptr(X))
    _check("nm_spmm_skinny", st)
    return out


def nm_spmm_prefill(values, masks, X, N: int = 2, M: int = 4, out=None):
    """Prefill product Y = X W'^T of a 50% packed matrix (2:4, 4:8, 8:16 or 16:32) on the
    matrix cores: X fp16 [tokens, cols] -> Y fp16 [tokens, rows]."""
    torch = _torch()
    rows, cols, tokens, out = _batch_args(values, masks, X, N, M, out)
    with torch.cuda.device(X.device):
        st = lib().nm_spmm_prefill(values.data_ptr(), masks.data_ptr(), X.data_ptr(), out.data_ptr(),
                                   rows, cols, tokens, N, M, _stream_ptr(X))
    _check("nm_spmm_prefill", st)
    return out


def _dense_args(W, X, out):
    torch = _torch()
    _require(W, "W", torch.float16, 2)
    _require(X, "X", torch.float16, 2)
    rows, cols = W.shape
    batch = X.shape[0]
    if X.shape[1] != cols:
        raise ValueError(f"X has {X.shape[1]} columns, W has {cols}")
    if W.device != X.device:
        raise ValueError("W and X must be on one device")
    if out is None:
        out = torch.empty((batch, rows), dtype=torch.float16, device=X.device)
    else:
        _require(out, "out", torch.float16, 2)
        if tuple(out.shape) != (batch, rows) or out.device != X.device:
            raise ValueError("out must be fp16 [batch, rows] on the same device")
    return rows, cols, batch, out


def nm_gemm_dense(W, X, out=None):
    """Dense baseline Y = X W^T: fp16 W [rows, cols], X [batch, cols] -> Y [batch, rows]."""
    torch = _torch()
    rows, cols, batch, out = _dense_args(W, X, out)
    with torch.cuda.device(X.device):
        st = lib().nm_gemm_dense(W.data_ptr(), X.data_ptr(), out.data_ptr(), rows, cols, batch,
                                 _stream_ptr(X))
    _check("nm_gemm_dense", st)
    return out


def nm_gemm_dense_prefill(W, X, out=None):
    """Dense prefill baseline Y = X W^T on the dense matrix cores: fp16 W [rows, cols],
    X [tokens, cols] -> Y [tokens, rows]."""
    torch = _torch()
    rows, cols, tokens, out = _dense_args(W, X, out)
    with torch.cuda.device(X.device):
        st = lib().nm_gemm_dense_prefill(W.data_ptr(), X.data_ptr(), out.data_ptr(), rows, cols, tokens,
                                         _stream_ptr(X))
    _check("nm_gemm_dense_prefill", st)
    return out


def nm_probe_read(buf, sink, magic: int = 0x9E3779B9):
    """Stream every byte of the contiguous device tensor `buf` (read-bandwidth probe)."""
    torch = _torch()
    nbytes = buf.numel() * buf.element_size()
    with torch.cuda.device(buf.device):
        st = lib().nm_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), magic, _stream_ptr(buf))
    _check("nm_probe_read", st)


def nm_probe_copy(dst, src):
    """Copy the contiguous device tensor src into dst (known-traffic kernel)."""
    torch = _torch()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    with torch.cuda.device(src.device):
        st = lib().nm_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream_ptr(src))
    _check("nm_probe_copy", st)
