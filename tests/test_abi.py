"""CPU tests of the C-ABI boundary: the library loads, exports every symbol the public
headers declare, and rejects bad arguments before any HIP call (so no GPU is needed)."""
import ctypes
import glob
import os
import re

import pytest

import semi_structured_sparse_amd as nm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A16 = 0x10000  # a 16-byte-aligned fake device address: validation never dereferences it


def declared_functions():
    names = []
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(nm_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_builds_and_loads():
    assert os.path.exists(nm.LIB_PATH), "build libnmsparse.so first"
    assert nm.lib() is not None


def test_every_declared_symbol_is_exported():
    decl = declared_functions()
    assert {"nm_pack", "nm_spmv", "nm_gemv_dense", "nm_values_count", "nm_masks_count",
            "nm_max_cols", "nm_status_string", "nm_last_hip_error", "nm_probe_read",
            "nm_probe_copy"} <= set(decl)
    handle = ctypes.CDLL(nm.LIB_PATH)
    for name in decl:
        assert hasattr(handle, name), name
    assert set(decl) == set(nm.SIGNATURES), "binding and headers disagree"


def test_status_strings():
    for s in range(8):
        assert nm.status_string(s)
    assert "scratch" in nm.status_string(nm.NM_ERR_SCRATCH)
    assert nm.status_string(99) == "unknown status"
    assert nm.status_string(0) == "ok"


@pytest.mark.parametrize("rows,cols,N,M,want", [
    (4096, 4096, 2, 4, 4096 * 2048), (1, 32, 16, 32, 16), (3, 96, 4, 8, 144),
    (0, 32, 2, 4, 0), (1, 0, 2, 4, 0), (1, 48, 2, 4, 0), (1, 32, 3, 4, 0), (1, 32, 1, 2, 0),
    (-1, 32, 2, 4, 0), (1, 16, 8, 16, 0),
    (1, 32, 1, 4, 8), (5, 256, 2, 8, 320), (2, 64, 4, 16, 32), (1, 32, 8, 32, 8),   # 25%
])
def test_values_count(rows, cols, N, M, want):
    assert nm.values_count(rows, cols, N, M) == want


def test_masks_count():
    assert nm.masks_count(7, 96) == 21
    assert nm.masks_count(7, 100) == 0
    assert nm.masks_count(1 << 40, 1 << 30) == 0  # overflow


def _spmv(**kw):
    a = dict(values=A16, masks=A16, x=A16, y=A16, rows=16, cols=64, N=2, M=4, stream=None)
    a.update(kw)
    return nm.lib().nm_spmv(a["values"], a["masks"], a["x"], a["y"], a["rows"], a["cols"],
                            a["N"], a["M"], a["stream"])


def _pack(**kw):
    a = dict(W=A16, values=A16, masks=A16, rows=16, cols=64, N=2, M=4, stream=None)
    a.update(kw)
    return nm.lib().nm_pack(a["W"], a["values"], a["masks"], a["rows"], a["cols"], a["N"],
                            a["M"], a["stream"])


def _gemv(**kw):
    a = dict(W=A16, x=A16, y=A16, rows=16, cols=64, stream=None)
    a.update(kw)
    return nm.lib().nm_gemv_dense(a["W"], a["x"], a["y"], a["rows"], a["cols"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(values=None), nm.NM_ERR_NULL), (dict(masks=None), nm.NM_ERR_NULL),
    (dict(x=None), nm.NM_ERR_NULL), (dict(y=None), nm.NM_ERR_NULL),
    (dict(rows=0), nm.NM_ERR_SHAPE), (dict(rows=-5), nm.NM_ERR_SHAPE),
    (dict(cols=0), nm.NM_ERR_SHAPE), (dict(cols=16), nm.NM_ERR_SHAPE), (dict(cols=80), nm.NM_ERR_SHAPE),
    (dict(rows=1 << 40), nm.NM_ERR_SHAPE),
    (dict(N=3, M=4), nm.NM_ERR_PATTERN), (dict(N=1, M=2), nm.NM_ERR_PATTERN),
    (dict(N=4, M=32), nm.NM_ERR_PATTERN), (dict(N=32, M=64), nm.NM_ERR_PATTERN),
    (dict(values=A16 + 8), nm.NM_ERR_ALIGN), (dict(masks=A16 + 2), nm.NM_ERR_ALIGN),
    (dict(x=A16 + 4), nm.NM_ERR_ALIGN), (dict(y=A16 + 1), nm.NM_ERR_ALIGN),
])
def test_spmv_validation(kw, want):
    assert _spmv(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(values=None), nm.NM_ERR_NULL), (dict(masks=None), nm.NM_ERR_NULL), (dict(W=None), nm.NM_ERR_NULL),
    (dict(rows=0), nm.NM_ERR_SHAPE), (dict(cols=48), nm.NM_ERR_SHAPE),
    (dict(N=3, M=4), nm.NM_ERR_PATTERN),
    (dict(values=A16 + 8), nm.NM_ERR_ALIGN), (dict(masks=A16 + 2), nm.NM_ERR_ALIGN), (dict(W=A16 + 4), nm.NM_ERR_ALIGN),
])
def test_unpack_validation(kw, want):
    a = dict(values=A16, masks=A16, W=A16, rows=16, cols=64, N=2, M=4)
    a.update(kw)
    assert nm.lib().nm_unpack(a["values"], a["masks"], a["W"], a["rows"], a["cols"], a["N"], a["M"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(W=None), nm.NM_ERR_NULL), (dict(values=None), nm.NM_ERR_NULL), (dict(masks=None), nm.NM_ERR_NULL),
    (dict(rows=0), nm.NM_ERR_SHAPE), (dict(cols=33), nm.NM_ERR_SHAPE),
    (dict(N=4, M=4), nm.NM_ERR_PATTERN),
    (dict(W=A16 + 2), nm.NM_ERR_ALIGN), (dict(values=A16 + 4), nm.NM_ERR_ALIGN),
    (dict(masks=A16 + 1), nm.NM_ERR_ALIGN),
])
def test_pack_validation(kw, want):
    assert _pack(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(W=None), nm.NM_ERR_NULL), (dict(x=None), nm.NM_ERR_NULL), (dict(y=None), nm.NM_ERR_NULL),
    (dict(rows=0), nm.NM_ERR_SHAPE), (dict(cols=31), nm.NM_ERR_SHAPE),
    (dict(W=A16 + 8), nm.NM_ERR_ALIGN), (dict(x=A16 + 2), nm.NM_ERR_ALIGN), (dict(y=A16 + 1), nm.NM_ERR_ALIGN),
])
def test_gemv_validation(kw, want):
    assert _gemv(**kw) == want


def _group(count=3, values=None, masks=None, x=A16, y=None, rows=None, cols=64, N=2, M=4, nulls=False):
    n = max(count, 1)
    P = ctypes.c_void_p * n
    vals = P(*([A16] * n)) if values is None else P(*values)
    msks = P(*([A16] * n)) if masks is None else P(*masks)
    outs = P(*([A16] * n)) if y is None else P(*y)
    rws = (ctypes.c_int64 * n)(*([16] * n if rows is None else rows))
    if nulls:
        return nm.lib().nm_spmv_group(count, None, msks, x, outs, rws, cols, N, M, None)
    return nm.lib().nm_spmv_group(count, vals, msks, x, outs, rws, cols, N, M, None)


def test_spmv_group_validation():
    """nm_spmv_group validates every product before any HIP call."""
    assert _group(nulls=True) == nm.NM_ERR_NULL
    assert _group(x=None) == nm.NM_ERR_NULL
    assert _group(values=[A16, 0, A16]) == nm.NM_ERR_NULL
    assert _group(y=[A16, A16, 0]) == nm.NM_ERR_NULL
    assert _group(count=0) == nm.NM_ERR_SHAPE
    assert _group(count=9) == nm.NM_ERR_SHAPE
    assert _group(rows=[16, 0, 16]) == nm.NM_ERR_SHAPE
    assert _group(cols=48) == nm.NM_ERR_SHAPE
    assert _group(N=3) == nm.NM_ERR_PATTERN
    assert _group(x=A16 + 2) == nm.NM_ERR_ALIGN
    assert _group(values=[A16, A16 + 8, A16]) == nm.NM_ERR_ALIGN
    assert _group(masks=[A16, A16, A16 + 2]) == nm.NM_ERR_ALIGN
    assert _group(y=[A16 + 1, A16, A16]) == nm.NM_ERR_ALIGN


def test_probe_validation():
    L = nm.lib()
    assert L.nm_probe_read(None, 16, A16, 0, None) == nm.NM_ERR_NULL
    assert L.nm_probe_read(A16, 0, A16, 0, None) == nm.NM_ERR_SHAPE
    assert L.nm_probe_read(A16, 24, A16, 0, None) == nm.NM_ERR_SHAPE
    assert L.nm_probe_read(A16 + 8, 16, A16, 0, None) == nm.NM_ERR_ALIGN
    assert L.nm_probe_copy(A16, None, 16, None) == nm.NM_ERR_NULL
    assert L.nm_probe_copy(A16 + 4, A16, 16, None) == nm.NM_ERR_ALIGN
    # the shaped read: every launch-shape argument outside its range is rejected
    rs = L.nm_probe_read_shaped
    assert rs(None, 16, A16, 0, 256, 512, 4, 0, None) == nm.NM_ERR_NULL
    assert rs(A16, 0, A16, 0, 256, 512, 4, 0, None) == nm.NM_ERR_SHAPE
    assert rs(A16 + 8, 16, A16, 0, 256, 512, 4, 0, None) == nm.NM_ERR_ALIGN
    for blocks, threads, unroll, blocked in ((0, 512, 4, 0), ((1 << 20) + 1, 512, 4, 0), (256, 32, 4, 0),
                                             (256, 1088, 4, 0), (256, 500, 4, 0), (256, 512, 3, 0),
                                             (256, 512, 16, 0), (256, 512, 4, 2), (256, 512, 4, -1)):
        assert rs(A16, 16, A16, 0, blocks, threads, unroll, blocked, None) == nm.NM_ERR_SHAPE


@pytest.mark.parametrize("kw,want", [
    (dict(values=None), nm.NM_ERR_NULL), (dict(X=None), nm.NM_ERR_NULL), (dict(Y=None), nm.NM_ERR_NULL),
    (dict(batch=0), nm.NM_ERR_SHAPE), (dict(batch=(1 << 24) + 1), nm.NM_ERR_SHAPE), (dict(cols=48), nm.NM_ERR_SHAPE),
    (dict(N=2, M=8), nm.NM_ERR_PATTERN), (dict(N=1, M=4, batch=9), nm.NM_ERR_PATTERN),
    (dict(batch=9, X=A16 + 8), nm.NM_ERR_ALIGN), (dict(batch=40, X=A16 + 8), nm.NM_ERR_ALIGN),
    (dict(batch=40, cols=(1 << 21) + 32), nm.NM_ERR_SHAPE),
    (dict(X=A16 + 8), nm.NM_ERR_ALIGN), (dict(Y=A16 + 1), nm.NM_ERR_ALIGN), (dict(masks=A16 + 2), nm.NM_ERR_ALIGN),
])
def test_spmm_validation(kw, want):
    a = dict(values=A16, masks=A16, X=A16, Y=A16, rows=64, cols=128, batch=4, N=2, M=4)
    a.update(kw)
    assert nm.lib().nm_spmm(a["values"], a["masks"], a["X"], a["Y"], a["rows"], a["cols"], a["batch"],
                            a["N"], a["M"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(values=None), nm.NM_ERR_NULL), (dict(masks=None), nm.NM_ERR_NULL), (dict(X=None), nm.NM_ERR_NULL),
    (dict(Y=None), nm.NM_ERR_NULL),
    (dict(batch=0), nm.NM_ERR_SHAPE), (dict(batch=(1 << 24) + 1), nm.NM_ERR_SHAPE), (dict(rows=0), nm.NM_ERR_SHAPE),
    (dict(cols=80), nm.NM_ERR_SHAPE), (dict(cols=(1 << 21) + 32), nm.NM_ERR_SHAPE),
    (dict(N=1, M=4), nm.NM_ERR_PATTERN), (dict(N=3, M=6), nm.NM_ERR_PATTERN), (dict(N=2, M=8), nm.NM_ERR_PATTERN),
    (dict(values=A16 + 8), nm.NM_ERR_ALIGN), (dict(masks=A16 + 2), nm.NM_ERR_ALIGN),
    (dict(X=A16 + 4), nm.NM_ERR_ALIGN), (dict(Y=A16 + 1), nm.NM_ERR_ALIGN),
    # every 50% pattern passes the pattern check and reaches the alignment check
    (dict(N=4, M=8, values=A16 + 8), nm.NM_ERR_ALIGN), (dict(N=8, M=16, X=A16 + 4), nm.NM_ERR_ALIGN),
    (dict(N=16, M=32, Y=A16 + 1), nm.NM_ERR_ALIGN),
])
def test_spmm_skinny_validation(kw, want):
    a = dict(values=A16, masks=A16, X=A16, Y=A16, rows=64, cols=128, batch=7, N=2, M=4)
    a.update(kw)
    assert nm.lib().nm_spmm_skinny(a["values"], a["masks"], a["X"], a["Y"], a["rows"], a["cols"], a["batch"],
                                   a["N"], a["M"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(W=None), nm.NM_ERR_NULL), (dict(batch=0), nm.NM_ERR_SHAPE), (dict(batch=(1 << 24) + 1), nm.NM_ERR_SHAPE),
    (dict(X=A16 + 2), nm.NM_ERR_ALIGN), (dict(batch=9, Y=A16 + 1), nm.NM_ERR_ALIGN),
    (dict(batch=40, Y=A16 + 1), nm.NM_ERR_ALIGN), (dict(batch=40, cols=(1 << 21) + 32), nm.NM_ERR_SHAPE),
])
def test_gemm_validation(kw, want):
    a = dict(W=A16, X=A16, Y=A16, rows=64, cols=128, batch=2)
    a.update(kw)
    assert nm.lib().nm_gemm_dense(a["W"], a["X"], a["Y"], a["rows"], a["cols"], a["batch"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(values=None), nm.NM_ERR_NULL), (dict(Y=None), nm.NM_ERR_NULL), (dict(batch=0), nm.NM_ERR_SHAPE),
    (dict(cols=48), nm.NM_ERR_SHAPE), (dict(N=2, M=8, batch=9), nm.NM_ERR_PATTERN),
    (dict(X=A16 + 8), nm.NM_ERR_ALIGN), (dict(Y=A16 + 1), nm.NM_ERR_ALIGN),
    # the workspace must be 16-byte aligned whatever kernel the shape takes
    (dict(ws=A16 + 8), nm.NM_ERR_ALIGN), (dict(ws=A16 + 4, batch=40), nm.NM_ERR_ALIGN),
    (dict(ws=A16 + 8, batch=1), nm.NM_ERR_ALIGN),
])
def test_spmm_ws_validation(kw, want):
    """nm_spmm_ws: nm_spmm's checks, plus the workspace's alignment, before any HIP call."""
    a = dict(values=A16, masks=A16, X=A16, Y=A16, rows=1024, cols=4096, batch=8, N=2, M=4, ws=A16)
    a.update(kw)
    assert nm.lib().nm_spmm_ws(a["values"], a["masks"], a["X"], a["Y"], a["rows"], a["cols"], a["batch"],
                               a["N"], a["M"], a["ws"], 1 << 20, None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(values=None), nm.NM_ERR_NULL), (dict(X=None), nm.NM_ERR_NULL), (dict(batch=0), nm.NM_ERR_SHAPE),
    (dict(rows=0), nm.NM_ERR_SHAPE), (dict(cols=48), nm.NM_ERR_SHAPE), (dict(N=2, M=8, batch=9), nm.NM_ERR_PATTERN),
    (dict(N=3, M=4), nm.NM_ERR_PATTERN), (dict(X=A16 + 8), nm.NM_ERR_ALIGN), (dict(Y=A16 + 1), nm.NM_ERR_ALIGN),
    (dict(masks=A16 + 2, batch=40), nm.NM_ERR_ALIGN),
])
def test_spmm_noalloc_validation(kw, want):
    """nm_spmm_noalloc: nm_spmm's checks before any HIP call (so before the scratch lookup)."""
    a = dict(values=A16, masks=A16, X=A16, Y=A16, rows=1024, cols=8192, batch=8, N=2, M=4)
    a.update(kw)
    assert nm.lib().nm_spmm_noalloc(a["values"], a["masks"], a["X"], a["Y"], a["rows"], a["cols"], a["batch"],
                                    a["N"], a["M"], None) == want


def test_noalloc_scratch_is_static_and_bounded():
    """The scratch array is a file-scope static device array of the declared size, reached
    through hipGetSymbolAddress; the entry point's source calls no allocator."""
    src = open(os.path.join(ROOT, "semi_structured_sparse_amd", "csrc", "nm_noalloc.hip")).read()
    code = re.sub(r"//[^\n]*", "", src)
    assert re.search(r"static __device__ __align__\(256\) unsigned char scratch\[kScratchBytes\]", code)
    assert "hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))" in code
    for alloc in ("hipMalloc", "hipFree", "hipMemset", "hipExtMalloc", "hipHostMalloc", "malloc(", "new "):
        assert alloc not in code, alloc
    hdr = open(os.path.join(ROOT, "include", "nm_sparse.h")).read()
    # 32 MiB of partial tiles (the largest split on a 256-CU part: 256 workgroups x 128 KiB
    # of a 256 x 128 tile) and room for the counters
    m = re.search(r"#define NM_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u \+ (\d+)u\)", hdr)
    assert m and int(m.group(1)) * int(m.group(2)) * int(m.group(3)) + int(m.group(4)) == 32 * 1024 * 1024 + 4096


def test_spmm_workspace_bytes_invalid_arguments():
    """Invalid shapes and patterns need no workspace (0, no HIP call)."""
    ws = nm.lib().nm_spmm_workspace_bytes
    assert ws(0, 4096, 8, 2, 4) == 0
    assert ws(1024, 48, 8, 2, 4) == 0
    assert ws(1024, 4096, 0, 2, 4) == 0
    assert ws(1024, 4096, 8, 3, 4) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(values=None), nm.NM_ERR_NULL), (dict(masks=None), nm.NM_ERR_NULL), (dict(X=None), nm.NM_ERR_NULL),
    (dict(Y=None), nm.NM_ERR_NULL),
    (dict(tokens=0), nm.NM_ERR_SHAPE), (dict(tokens=(1 << 24) + 1), nm.NM_ERR_SHAPE), (dict(rows=0), nm.NM_ERR_SHAPE),
    (dict(cols=80), nm.NM_ERR_SHAPE), (dict(cols=(1 << 21) + 32), nm.NM_ERR_SHAPE),
    (dict(N=1, M=4), nm.NM_ERR_PATTERN), (dict(N=3, M=4), nm.NM_ERR_PATTERN), (dict(N=8, M=32), nm.NM_ERR_PATTERN),
    (dict(N=2, M=8), nm.NM_ERR_PATTERN),
    (dict(values=A16 + 8), nm.NM_ERR_ALIGN), (dict(masks=A16 + 2), nm.NM_ERR_ALIGN),
    (dict(X=A16 + 4), nm.NM_ERR_ALIGN), (dict(Y=A16 + 1), nm.NM_ERR_ALIGN),
    # 4:8, 8:16 (the split operands) and 16:32 (expanded fragments) pass the pattern check and
    # reach the alignment check
    (dict(N=4, M=8, values=A16 + 8), nm.NM_ERR_ALIGN), (dict(N=8, M=16, X=A16 + 4), nm.NM_ERR_ALIGN),
    (dict(N=16, M=32, masks=A16 + 2), nm.NM_ERR_ALIGN),
])
def test_spmm_prefill_validation(kw, want):
    a = dict(values=A16, masks=A16, X=A16, Y=A16, rows=64, cols=128, tokens=300, N=2, M=4)
    a.update(kw)
    assert nm.lib().nm_spmm_prefill(a["values"], a["masks"], a["X"], a["Y"], a["rows"], a["cols"], a["tokens"],
                                    a["N"], a["M"], None) == want


@pytest.mark.parametrize("kw,want", [
    (dict(W=None), nm.NM_ERR_NULL), (dict(X=None), nm.NM_ERR_NULL), (dict(Y=None), nm.NM_ERR_NULL),
    (dict(tokens=0), nm.NM_ERR_SHAPE), (dict(cols=33), nm.NM_ERR_SHAPE), (dict(cols=(1 << 21) + 32), nm.NM_ERR_SHAPE),
    (dict(W=A16 + 2), nm.NM_ERR_ALIGN), (dict(X=A16 + 8), nm.NM_ERR_ALIGN), (dict(Y=A16 + 1), nm.NM_ERR_ALIGN),
])
def test_gemm_prefill_validation(kw, want):
    a = dict(W=A16, X=A16, Y=A16, rows=64, cols=128, tokens=300)
    a.update(kw)
    assert nm.lib().nm_gemm_dense_prefill(a["W"], a["X"], a["Y"], a["rows"], a["cols"], a["tokens"], None) == want


def test_spmm_variant_validation():
    """Invalid arguments give the empty name before any HIP call."""
    L = nm.lib()
    assert L.nm_spmm_variant(0, 128, 4, 2, 4) == b""
    assert L.nm_spmm_variant(64, 80, 4, 2, 4) == b""
    assert L.nm_spmm_variant(64, 128, 0, 2, 4) == b""
    assert L.nm_spmm_variant(64, 128, 4, 3, 4) == b""
    assert L.nm_spmm_variant(64, 128, 4, 1, 4) == b""   # 25% patterns: one vector only


def test_prefill_variant_validation():
    """Invalid shapes give the empty name before any HIP call."""
    L = nm.lib()
    assert L.nm_prefill_variant(0, 128, 16, 1) == b""
    assert L.nm_prefill_variant(64, 80, 16, 1) == b""
    assert L.nm_prefill_variant(64, 128, 0, 0) == b""


def test_launch_shape_validation():
    """nm_spmv_launch_shape validates like nm_spmv, before any HIP call."""
    L = nm.lib()
    buf = (ctypes.c_int64 * 4)()
    assert L.nm_spmv_launch_shape(64, 128, 2, 4, None) == nm.NM_ERR_NULL
    assert L.nm_spmv_launch_shape(0, 128, 2, 4, buf) == nm.NM_ERR_SHAPE
    assert L.nm_spmv_launch_shape(64, 80, 2, 4, buf) == nm.NM_ERR_SHAPE
    assert L.nm_spmv_launch_shape(64, 128, 3, 4, buf) == nm.NM_ERR_PATTERN


def test_python_layer_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    W = torch.zeros(16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        nm.nm_pack(W, 2, 4)
    with pytest.raises(ValueError):
        nm.nm_gemv_dense(W, torch.zeros(64, dtype=torch.float16))
    v = torch.zeros(16, 32, dtype=torch.float16)
    m = torch.zeros(16, 2, dtype=torch.int32)
    with pytest.raises(ValueError):
        nm.nm_spmv_group([v], [m], torch.zeros(64, dtype=torch.float16), 2, 4)
    with pytest.raises(ValueError):   # no products, or more than the group holds
        nm.nm_spmv_group([], [], torch.zeros(64, dtype=torch.float16), 2, 4)
