"""GPU test of nm_spmm_noalloc, the batch product for callers that cannot allocate (its
column-split workspace is the library's static per-GPU scratch), through the C ABI: calls in
a row, each followed by a smaller one, give Y bit-identical to nm_spmm_ws with a fresh
workspace of its own (the same kernels, splits and summation order) and within the oracle's
tolerance on sampled rows; shapes without a split and the prefill route match nm_spmm."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import device, down_bits16, down_f16, sample_rows, say, up_f16

pytestmark = pytest.mark.gpu


def _inputs(N, M, R, C, T, seed):
    W = synth.weight(R, C, seed)
    X = synth.activations(T, C, seed + 1)
    v, m = nm.nm_pack(up_f16(W), N, M)
    return W, X, v, m, up_f16(X)


def _noalloc(v, m, x, N, M, R, T):
    out = torch.full((T, R), float("nan"), dtype=torch.float16, device=device())
    return nm.nm_spmm_noalloc(v, m, x, N, M, out=out)


def _oracle_ok(W, X, Y, N, M):
    R, C = W.shape
    idx = sample_rows(R, k=24, rpb=16)
    rv, rm = oracle.pack_ref(W[idx], N, M)
    rep = oracle.y_tolerance_report(down_f16(Y)[:, idx], oracle.spmm_ref(rv, rm, X, C, N, M))
    assert rep["ok"], rep


# pairs of calls in a row, the second smaller: (pattern, rows, cols, vectors) each
PAIRS = [
    (((2, 4), 2048, 14336, 16), ((2, 4), 1024, 8192, 8)),     # 2 splits x 128 tiles, then 4 x 64
    (((8, 16), 1024, 4096, 12), ((4, 8), 512, 4096, 9)),      # the split patterns: 4 x 64, then 8 x 32
    (((2, 4), 1000, 8192, 17), ((2, 4), 300, 8224, 6)),       # column-split prefill kernel; skinny, ragged
    (((4, 8), 4096, 14336, 40), ((2, 4), 1024, 4096, 20)),    # column-split prefill: 7 x 64 tiles, then 8 x 16
    (((2, 4), 4000, 14304, 300), ((8, 16), 2050, 10240, 260)),  # taller splits: 4 x 48 tiles of 256 x 128, then 4 x 51 of 128 x 128
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_entry_point(first, second):
    for k, ((N, M), R, C, T) in enumerate((first, second)):
        assert nm.spmm_workspace_bytes(R, C, T, N, M) > 0, (R, C, T)
        say(f"noalloc call {k}: {N}:{M} {R}x{C} vectors={T}")
        W, X, v, m, x = _inputs(N, M, R, C, T, 5000 + 7 * k + R % 97 + C % 89 + T)
        got = _noalloc(v, m, x, N, M, R, T)
        want = nm.nm_spmm_ws(v, m, x, N, M, nm.spmm_workspace(R, C, T, N, M))
        assert np.array_equal(down_bits16(got), down_bits16(want)), ((N, M), R, C, T)
        _oracle_ok(W, X, got, N, M)


def test_noalloc_repeated_calls_are_identical():
    """The scratch keeps the last call's contents: the counters it leaves at zero let the
    next call split again, with the same bits."""
    N, M, R, C, T = 2, 4, 1024, 14336, 8
    _, _, v, m, x = _inputs(N, M, R, C, T, 5100)
    Y0 = down_bits16(_noalloc(v, m, x, N, M, R, T))
    for _ in range(5):
        assert np.array_equal(down_bits16(_noalloc(v, m, x, N, M, R, T)), Y0)


@pytest.mark.parametrize("pat,R,C,T", [((2, 4), 4096, 4096, 8), ((16, 32), 4096, 4096, 12), ((2, 4), 1024, 4096, 4),
                                       ((8, 16), 4096, 4096, 1024), ((2, 4), 2048, 2048, 1)])
def test_noalloc_unsplit_routes_match_nm_spmm(pat, R, C, T):
    """Shapes that take no column split (large layers, 16:32, fewer than 5 vectors, prefill
    sizes, one vector) run nm_spmm's kernels: bit-identical Y."""
    N, M = pat
    assert nm.spmm_workspace_bytes(R, C, T, N, M) == 0
    say(f"noalloc unsplit {N}:{M} {R}x{C} vectors={T}")
    _, _, v, m, x = _inputs(N, M, R, C, T, 5200 + T)
    assert np.array_equal(down_bits16(_noalloc(v, m, x, N, M, R, T)), down_bits16(nm.nm_spmm(v, m, x, N, M)))
