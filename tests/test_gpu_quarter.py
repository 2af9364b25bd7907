"""GPU parity tests of the 25% N:M patterns (1:4, 2:8, 4:16, 8:32; 8 kept values per mask
word) through the C ABI, against the CPU oracle.

Bars as for the 50% patterns: nm_pack bit-exact; y within |y - ref| <= 2e-3 + 1e-2*|ref|
per element and relative L2 <= 1e-3; exact special cases bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import (check_full_layer, device, down_bits16, down_f16, down_u32, say,
                               up_f16, up_u32)

pytestmark = pytest.mark.gpu
QUARTER = synth.PATTERNS_QUARTER

# 1..7 mask words in the last step of 256 columns, several steps and workgroups, both
# sides of 8 rows per CU
SMALL = [(1, 32), (3, 64), (17, 96), (5, 224), (9, 288), (7, 480), (37, 544), (16, 4096),
         (100, 2080), (256, 512), (33, 1056), (2100, 96), (2064, 160)]


@pytest.mark.parametrize("N,M", QUARTER)
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_quarter_pack_bit_exact(N, M, kind):
    for i, (R, C) in enumerate(SMALL):
        W = synth.weight(R, C, seed=1600 + i) if kind == "normal" else synth.tie_heavy_weight(R, C, seed=1650 + i)
        values, masks = nm.nm_pack(up_f16(W), N, M)
        rv, rm = oracle.pack_ref(W, N, M)
        assert np.array_equal(down_u32(masks), rm), (R, C)
        assert np.array_equal(down_bits16(values), rv), (R, C)


@pytest.mark.parametrize("N,M", QUARTER)
def test_quarter_spmv_small(N, M):
    for i, (R, C) in enumerate(SMALL):
        W = synth.weight(R, C, seed=1700 + i)
        x = synth.activation(C, seed=1750 + i)
        rv, rm = oracle.pack_ref(W, N, M)
        y = nm.nm_spmv(up_f16(rv), up_u32(rm), up_f16(x), N, M)
        rep = oracle.y_tolerance_report(down_f16(y), oracle.spmv_ref(rv, rm, x, C, N, M))
        assert rep["ok"], ((R, C), rep)
        gv, gm = nm.nm_pack(up_f16(W), N, M)
        y2 = nm.nm_spmv(gv, gm, up_f16(x), N, M)
        assert np.array_equal(down_bits16(y2), down_bits16(y)), (R, C)


REGIMES = [(255, 4096), (2048, 1024), (1500, 2080), (2049, 512), (5121, 4096), (300, 16640),
           (777, 16416), (10241, 16640)]


@pytest.mark.parametrize("N,M", QUARTER)
def test_quarter_regimes(N, M):
    for i, (R, C) in enumerate(REGIMES):
        say(f"quarter regime {R}x{C} {N}:{M} {nm.spmv_launch_shape(R, C, N, M)}")
        W = synth.weight(R, C, seed=1800 + i)
        x = synth.activation(C, seed=1850 + i)
        check_full_layer(W, x, N, M, f"quarter-{R}x{C}", check_dense=False)


@pytest.mark.parametrize("N,M", QUARTER)
def test_quarter_one_hot_and_determinism(N, M):
    """x = e_c gives column c of the pruned matrix bit-exactly; repeated calls give the
    same bits."""
    R, C = 64, 1024
    W = synth.weight(R, C, seed=1900)
    rv, rm = oracle.pack_ref(W, N, M)
    v, m = up_f16(rv), up_u32(rm)
    D = oracle.unpack_ref(rv, rm, C, N, M)
    for c in (0, 1, 255, 256, 777, C - 1):
        x = np.zeros(C, np.float16)
        x[c] = 1.0
        y = down_bits16(nm.nm_spmv(v, m, up_f16(x), N, M))
        want = D[:, c].copy()
        want[want == 0x8000] = 0  # -0 weights give +0 in the fp32 sum
        assert np.array_equal(y, want), c
    x = synth.activation(C, seed=1901)
    y0 = down_bits16(nm.nm_spmv(v, m, up_f16(x), N, M))
    for _ in range(20):
        assert np.array_equal(down_bits16(nm.nm_spmv(v, m, up_f16(x), N, M)), y0)


def test_quarter_widest_and_malformed():
    mc = nm.max_cols()
    W = synth.weight(3, mc, seed=1950)
    x = synth.activation(mc, seed=1951)
    for N, M in QUARTER:
        rv, rm = oracle.pack_ref(W, N, M)
        y = nm.nm_spmv(up_f16(rv), up_u32(rm), up_f16(x), N, M)
        assert oracle.y_tolerance_report(down_f16(y), oracle.spmv_ref(rv, rm, x, mc, N, M))["ok"], (N, M)
    R, C = 64, 1024
    v = up_f16(synth.weight(R, C // 4, seed=1952))
    xd = up_f16(synth.activation(C, seed=1953))
    for N, M in QUARTER:
        for word in (0, 1, 0x80000000, 0xFFFFFFFF):
            m = torch.full((R, C // 32), np.uint32(word).view(np.int32).item(), dtype=torch.int32, device=device())
            y = nm.nm_spmv(v, m, xd, N, M)
            torch.cuda.synchronize()
            assert y.shape == (R,)


def test_quarter_through_the_batch_entry_point():
    """nm_spmm accepts the 25% patterns for one vector (the single-vector kernel, same bits)
    and rejects them for larger batches."""
    R, C = 300, 4096
    W = synth.weight(R, C, seed=1960)
    x = synth.activation(C, seed=1961)
    for N, M in QUARTER:
        rv, rm = oracle.pack_ref(W, N, M)
        v, m = up_f16(rv), up_u32(rm)
        y = down_bits16(nm.nm_spmv(v, m, up_f16(x), N, M))
        Y = down_bits16(nm.nm_spmm(v, m, up_f16(x[None, :]), N, M))
        assert np.array_equal(Y[0], y)
        with pytest.raises(nm.NMArgumentError) as e:
            nm.nm_spmm(v, m, up_f16(np.stack([x, x])), N, M)
        assert e.value.status == nm.NM_ERR_PATTERN


def _full_size_cases():
    return [pytest.param(name, R, C, p, id=f"{name}-{R}x{C}-{p[0]}:{p[1]}")
            for name, R, C in synth.LLAMA31_8B for p in QUARTER]


@pytest.mark.slow
@pytest.mark.parametrize("name,R,C,pat", _full_size_cases())
def test_quarter_full_size(name, R, C, pat):
    """The Llama-3.1-8B projection shapes at full size for every 25% pattern: pack
    bit-exact and y within tolerance on sampled rows."""
    N, M = pat
    say(f"quarter full-size {name} {R}x{C} {N}:{M}")
    W = synth.weight(R, C, synth.weight_seed(2, [l[0] for l in synth.LLAMA31_8B].index(name), pat))
    x = synth.activation(C, synth.x_seed(2, 0, pat))
    check_full_layer(W, x, N, M, f"quarter-{name}", check_dense=False)
