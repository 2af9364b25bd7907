"""Helpers shared by the GPU tests: device transfer, sampled-row parity checks."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import semi_structured_sparse_amd as nm


def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def up_f16(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(device())


def up_u32(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(device())


def down_bits16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def down_u32(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def down_f16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.float16)


def sample_rows(rows: int, k: int = 48, seed: int = 0, rpb: int | None = None) -> np.ndarray:
    """First, last, the rows on both sides of the first and last workgroup edges (rpb rows
    per workgroup; 16 if not given), and k random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    t = rpb or 16
    last0 = (rows - 1) // t * t                   # first row of the last workgroup
    pick = {0, rows - 1, rows // 2, t - 1, t, last0 - 1, last0, last0 + 7, last0 + 8}
    pick |= set(rng.integers(0, rows, size=min(k, rows)).tolist())
    return np.array(sorted(p for p in pick if 0 <= p < rows), dtype=np.int64)


def check_launch_shape(rows: int, cols: int, N: int, M: int) -> dict:
    """The workgroup shape nm_spmv reports covers every row exactly once and fits a
    workgroup (at most 16 waves)."""
    s = nm.spmv_launch_shape(rows, cols, N, M)
    rpb, rg, cs, g = s["rows_per_workgroup"], s["row_groups"], s["waves_per_row_group"], s["workgroups"]
    assert rpb >= 1 and cs >= 1, s
    assert rg == -(-rpb // 8), s
    assert rg * cs <= 16, s
    assert g == -(-rows // rpb), s
    return s


def check_full_layer(W_host: np.ndarray, x_host: np.ndarray, N: int, M: int, tag: str,
                     check_dense: bool = True) -> dict:
    """Pack on the GPU, run the sparse (and dense) product, and compare sampled rows with
    the oracle: pack bit-exact, y within tolerance. Returns the parity figures."""
    rows, cols = W_host.shape
    shape = check_launch_shape(rows, cols, N, M)
    Wd = up_f16(W_host)
    xd = up_f16(x_host)
    values, masks = nm.nm_pack(Wd, N, M)
    y = nm.nm_spmv(values, masks, xd, N, M)
    yd = nm.nm_gemv_dense(Wd, xd) if check_dense else None
    torch.cuda.synchronize()
    idx = sample_rows(rows, rpb=shape["rows_per_workgroup"])
    it = torch.from_numpy(idx).to(device())
    gv = down_bits16(values.index_select(0, it))
    gm = down_u32(masks.index_select(0, it))
    rv, rm = oracle.pack_ref(W_host[idx], N, M)
    assert np.array_equal(gm, rm), f"{tag}: masks differ from the oracle"
    assert np.array_equal(gv, rv), f"{tag}: values differ from the oracle"
    ref = oracle.spmv_ref(rv, rm, x_host, cols, N, M)
    rep = oracle.y_tolerance_report(down_f16(y)[idx], ref)
    assert rep["ok"], f"{tag}: spmv {rep}"
    out = {"spmv": rep}
    if check_dense:
        dref = oracle.gemv_ref(W_host[idx], x_host)
        drep = oracle.y_tolerance_report(down_f16(yd)[idx], dref)
        assert drep["ok"], f"{tag}: dense {drep}"
        out["dense"] = drep
    del Wd, values, masks, y, yd
    return out


def check_all_rows(W_host: np.ndarray, x_host: np.ndarray, N: int, M: int, tag: str, chunk: int = 512) -> dict:
    """Pack on the GPU and run the sparse product, then compare EVERY row with the oracle:
    values and masks bit-exact, y within tolerance. The oracle runs on chunks of rows over a
    pool of host threads (numpy releases the interpreter lock in its array operations)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    rows, cols = W_host.shape
    Wd = up_f16(W_host)
    values, masks = nm.nm_pack(Wd, N, M)
    y = nm.nm_spmv(values, masks, up_f16(x_host), N, M)
    torch.cuda.synchronize()
    del Wd
    gv, gm, gy = down_bits16(values), down_u32(masks), down_f16(y)
    del values, masks, y

    def one(a):
        b = min(rows, a + chunk)
        rv, rm = oracle.pack_ref(W_host[a:b], N, M)
        bad = int(np.count_nonzero(gv[a:b] != rv)) + int(np.count_nonzero(gm[a:b] != rm))
        return a, bad, oracle.spmv_ref(rv, rm, x_host, cols, N, M)

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    ref = np.empty(rows, np.float64)
    mismatches = 0
    with ThreadPoolExecutor(max(1, min(16, cores))) as ex:
        for a, bad, r in ex.map(one, range(0, rows, chunk)):
            mismatches += bad
            ref[a:a + r.shape[0]] = r
    assert mismatches == 0, f"{tag}: {mismatches} packed words/values differ from the oracle"
    rep = oracle.y_tolerance_report(gy, ref)
    assert rep["ok"], f"{tag}: spmv {rep}"
    return rep
