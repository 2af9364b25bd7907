"""GPU parity tests of the small-batch products (nm_spmm, nm_gemm_dense) through the C ABI,
against the CPU oracle (spmm_ref, gemm_ref).

Bars: y within |y - ref| <= 2e-3 + 1e-2*|ref| per element and relative L2 <= 1e-3 over
the whole [batch, rows] output (fp32 accumulation, fp16 output, fp64 oracle); structural
properties (row permutation, determinism, batch 1 = the single-vector kernel) bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import device, down_bits16, down_f16, sample_rows, say, up_f16, up_u32

pytestmark = pytest.mark.gpu
PATTERNS = synth.PATTERNS
BATCHES = (1, 2, 3, 4, 5, 8)

# ragged rows and columns (1..3 mask words in the last step), several workgroups
SMALL = [(1, 32), (3, 64), (17, 96), (5, 160), (37, 544), (16, 4096), (100, 2080), (33, 1056),
         (2100, 96)]


def batch_x(B: int, C: int, seed: int) -> np.ndarray:
    """B seeded activation vectors ~N(0,1) fp16, one per row."""
    return np.stack([synth.activation(C, seed + 7919 * b) for b in range(B)])


def check_spmm(W, X, N, M, tag, rows_idx=None, dense=False):
    """Run nm_spmm (and optionally nm_gemm_dense) and compare with the oracle: on all rows
    with the oracle's packing as input, or, given a sample of rows, with the GPU's packing
    (bit-exact to the oracle's, checked on those rows) on the sampled rows."""
    R, C = W.shape
    if rows_idx is None:
        idx = np.arange(R)
        rv, rm = oracle.pack_ref(W, N, M)          # the oracle's packing of every row
        Y = down_f16(nm.nm_spmm(up_f16(rv), up_u32(rm), up_f16(X), N, M))
    else:
        idx = rows_idx
        values, masks = nm.nm_pack(up_f16(W), N, M)
        Y = down_f16(nm.nm_spmm(values, masks, up_f16(X), N, M))
        rv, rm = oracle.pack_ref(W[idx], N, M)     # the oracle's packing of the sampled rows
        it = torch.from_numpy(idx).to(device())
        assert np.array_equal(down_bits16(values.index_select(0, it)), rv.view(np.uint16)), tag
        del values, masks
    assert Y.shape == (X.shape[0], R)
    ref = oracle.spmm_ref(rv, rm, X, C, N, M)     # rows idx of the product
    rep = oracle.y_tolerance_report(Y[:, idx], ref)
    assert rep["ok"], (tag, rep)
    if dense:
        Yd = down_f16(nm.nm_gemm_dense(up_f16(W), up_f16(X)))
        drep = oracle.y_tolerance_report(Yd[:, idx], oracle.gemm_ref(W[idx], X))
        assert drep["ok"], (tag, "dense", drep)
    return rep


@pytest.mark.parametrize("N,M", PATTERNS)
def test_spmm_small(N, M):
    for i, (R, C) in enumerate(SMALL):
        W = synth.weight(R, C, seed=900 + i)
        for B in BATCHES:
            check_spmm(W, batch_x(B, C, 950 + i), N, M, (R, C, B))


def test_gemm_small():
    for i, (R, C) in enumerate(SMALL):
        W = synth.weight(R, C, seed=1000 + i)
        for B in BATCHES:
            X = batch_x(B, C, 1050 + i)
            Y = down_f16(nm.nm_gemm_dense(up_f16(W), up_f16(X)))
            rep = oracle.y_tolerance_report(Y, oracle.gemm_ref(W, X))
            assert rep["ok"], ((R, C, B), rep)


# widths that need two or more column phases at the interleave stride of the batch
# (x of B vectors does not fit one workgroup's LDS at once), and batch 1 beyond the
# single-vector kernel's widest x
PHASED = [(8, 37, 14336), (5, 19, 14336), (4, 23, 20000 // 32 * 32), (2, 11, 40064), (3, 7, 20000 // 32 * 32),
          (1, 3, 82048)]


@pytest.mark.parametrize("B,R,C", PHASED)
def test_spmm_column_phases(B, R, C):
    W = synth.weight(R, C, seed=1100 + B)
    X = batch_x(B, C, 1150 + B)
    for N, M in PATTERNS:
        say(f"phased spmm B={B} {R}x{C} {N}:{M}")
        check_spmm(W, X, N, M, (B, R, C, N), dense=(N == 2))


# one shape per regime of the workgroup-shape rule, sampled rows at full size
REGIMES = [(1024, 4096), (4096, 4096), (14336, 4096), (4096, 14336), (777, 16416), (10241, 8320)]


@pytest.mark.parametrize("B", (2, 8))
def test_spmm_regimes(B):
    for i, (R, C) in enumerate(REGIMES):
        W = synth.weight(R, C, seed=1200 + i)
        X = batch_x(B, C, 1250 + i)
        for N, M in PATTERNS:
            say(f"regime spmm B={B} {R}x{C} {N}:{M}")
            check_spmm(W, X, N, M, (B, R, C, N), rows_idx=sample_rows(R), dense=(N == 2))


@pytest.mark.parametrize("N,M", PATTERNS)
def test_spmm_narrow_layers_all_rows(N, M):
    """Every row of narrow layers (at most 4 rows per workgroup) at several batches, against
    the oracle: 1023 x 2048 (4 rows per workgroup, the last one 3; too few steps per wave for
    column parts, so spare lanes repeat the last row), 1000 x 8192 (each row on 2 parts of a
    wave's lanes) and 300 x 16416 (2 rows per workgroup on 4 parts, a one-word tail step)."""
    for i, (R, C, ci) in enumerate(((1023, 2048, 1), (1000, 8192, 2), (300, 16416, 4))):
        W = synth.weight(R, C, seed=1600 + i)
        for B in (2, 3, 5, 8):
            name = nm.spmm_variant(R, C, B, N, M)
            say(f"narrow spmm B={B} {R}x{C} {N}:{M} {name}")
            if not name.startswith("skinny"):
                want = f"spmm_narrow_kernel<{N}, {B}, " if ci > 1 else f"spmm_kernel<{N}, {B}, "
                assert name.startswith(want) and (ci == 1 or name.endswith(f", {ci}>")), name
            check_spmm(W, batch_x(B, C, 1650 + 10 * i + B), N, M, (B, R, C, N))


@pytest.mark.parametrize("N,M", PATTERNS)
def test_spmm_rows_of_x_are_independent(N, M):
    """Permuting the rows of X permutes the rows of Y bit-exactly (each output row is
    computed alone, in a fixed order), and repeated calls give the same bits."""
    R, C, B = 300, 4096, 8
    W = synth.weight(R, C, seed=1300)
    X = batch_x(B, C, 1301)
    rv, rm = oracle.pack_ref(W, N, M)
    v, m = up_f16(rv), up_u32(rm)
    Y = down_bits16(nm.nm_spmm(v, m, up_f16(X), N, M))
    perm = np.array([3, 7, 0, 5, 1, 6, 2, 4])
    Yp = down_bits16(nm.nm_spmm(v, m, up_f16(X[perm]), N, M))
    assert np.array_equal(Yp, Y[perm])
    for _ in range(20):
        assert np.array_equal(down_bits16(nm.nm_spmm(v, m, up_f16(X), N, M)), Y)


@pytest.mark.parametrize("N,M", PATTERNS)
def test_spmm_batch1_is_the_spmv_kernel(N, M):
    """A batch of one vector takes the single-vector kernel: bit-identical to nm_spmv."""
    R, C = 513, 4096
    W = synth.weight(R, C, seed=1400)
    x = synth.activation(C, seed=1401)
    rv, rm = oracle.pack_ref(W, N, M)
    v, m = up_f16(rv), up_u32(rm)
    y = down_bits16(nm.nm_spmv(v, m, up_f16(x), N, M))
    Y = down_bits16(nm.nm_spmm(v, m, up_f16(x[None, :]), N, M))
    assert np.array_equal(Y[0], y)


def test_spmm_malformed_masks_stay_in_bounds():
    """Masks with the wrong number of set bits give an unspecified Y but the kernel runs to
    completion (every x read stays inside the padded LDS buffer)."""
    for R, C, B in ((64, 1024, 8), (1024, 1024, 8)):
        v = up_f16(synth.weight(R, C // 2, seed=1500))
        X = up_f16(batch_x(B, C, 1501))
        for N, M in PATTERNS:
            for word in (0, 1, 0x80000000, 0xFFFFFFFF):
                m = torch.full((R, C // 32), np.uint32(word).view(np.int32).item(), dtype=torch.int32,
                               device=device())
                Y = nm.nm_spmm(v, m, X, N, M)
                torch.cuda.synchronize()
                assert Y.shape == (B, R)


def test_spmm_argument_errors():
    v = torch.zeros((4, 64), dtype=torch.float16, device=device())
    m = torch.zeros((4, 4), dtype=torch.int32, device=device())
    X = torch.zeros((2, 128), dtype=torch.float16, device=device())
    Y = torch.zeros((2, 4), dtype=torch.float16, device=device())
    assert nm.lib().nm_spmm(v.data_ptr(), m.data_ptr(), X.data_ptr(), Y.data_ptr(), 4, 128, 0, 2, 4,
                            None) == nm.NM_ERR_SHAPE
    with pytest.raises(ValueError):
        nm.nm_spmm(v, m, torch.zeros((2, 96), dtype=torch.float16, device=device()), 2, 4)
