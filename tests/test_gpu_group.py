"""GPU parity of nm_spmv_group: several packed matrices that share x, in one launch
(q, k, v or gate, up stored as separate matrices). Each output is checked against the
CPU oracle, and against nm_spmv bit for bit where both run spmv_kernel with the same
workgroup shape; shapes outside the one-launch path (long rows, 25% patterns) take one
nm_spmv launch per product and must equal it bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import down_bits16, down_f16, sample_rows, say, up_f16, up_u32
from tests.test_gpu_graph import _replay_and_check

pytestmark = pytest.mark.gpu


def _packed(rows, C, N, M, seed):
    out = []
    for k, R in enumerate(rows):
        W = synth.weight(R, C, seed + k)
        rv, rm = oracle.pack_ref(W, N, M)
        out.append((W, rv, rm, up_f16(rv), up_u32(rm)))
    return out


def _check(rows, C, N, M, seed, all_rows=True, bitwise=True):
    mats = _packed(rows, C, N, M, seed)
    x = synth.activation(C, seed + 99)
    xd = up_f16(x)
    ys = nm.nm_spmv_group([m[3] for m in mats], [m[4] for m in mats], xd, N, M)
    torch.cuda.synchronize()
    for k, (W, rv, rm, v, m) in enumerate(mats):
        R = rows[k]
        idx = np.arange(R) if all_rows else sample_rows(R)
        y = down_f16(ys[k])
        rep = oracle.y_tolerance_report(y[idx], oracle.spmv_ref(rv[idx], rm[idx], x, C, N, M))
        assert rep["ok"], (k, R, C, N, rep)
        single = nm.spmv_variant(R, C, N, M)
        separate = M == 4 * N or C > 8192           # one nm_spmv launch per product
        if separate or (bitwise and single.startswith("spmv_kernel")):
            assert np.array_equal(down_bits16(ys[k]), down_bits16(nm.nm_spmv(v, m, xd, N, M))), (k, R, single)
    return ys


@pytest.mark.parametrize("N,M", synth.PATTERNS)
def test_group_qkv_shapes(N, M):
    """q, k, v of a Llama-3.1-8B block (4096, 1024, 1024 rows x 4096 columns)."""
    say(f"group qkv {N}:{M}")
    _check((4096, 1024, 1024), 4096, N, M, seed=6000 + N)


@pytest.mark.parametrize("N,M", synth.PATTERNS)
def test_group_ragged(N, M):
    """Ragged rows (1, 7, 300, 2049: workgroups of fewer rows than their lanes cover) and a
    ragged last step (2080 columns), every row against the oracle."""
    say(f"group ragged {N}:{M}")
    _check((1, 7, 300, 2049), 2080, N, M, seed=6100 + N, bitwise=False)


@pytest.mark.parametrize("N,M", synth.PATTERNS)
def test_group_tiny(N, M):
    """Rows of 1..3 at 32 and 96 columns (one and three mask words: only a partial step)."""
    for C in (32, 96):
        say(f"group tiny {N}:{M} x{C}")
        _check((1, 2, 3), C, N, M, seed=6700 + C + N, bitwise=False)


def test_group_gate_up_and_eight_products():
    """gate and up (14336 rows each, 4096 columns) on sampled rows; eight products of
    mixed rows (the largest group) on every row."""
    say("group gate/up 2:4")
    _check((14336, 14336), 4096, 2, 4, seed=6200, all_rows=False)
    say("group of eight 8:16")
    _check((64, 512, 1024, 96, 2048, 33, 700, 4096), 1024, 8, 16, seed=6300, bitwise=False)


@pytest.mark.parametrize("N,M,C", [(2, 4, 14336), (16, 32, 9216), (1, 4, 4096), (8, 32, 2048)])
def test_group_separate_launch_path(N, M, C):
    """Long rows (more than 64 steps of 128 columns) and 25% patterns take one nm_spmv
    launch per product: bit-identical to nm_spmv."""
    say(f"group separate launches {N}:{M} x{C}")
    _check((1024, 513), C, N, M, seed=6400 + N, all_rows=False)


def test_group_graph_replays():
    """A captured group call replays with the eager call's bits, new x between replays."""
    C, rows = 4096, (4096, 1024, 1024)
    mats = _packed(rows, C, 2, 4, seed=6500)
    xd = up_f16(synth.activation(C, 6599))
    outs = [torch.empty(R, dtype=torch.float16, device=xd.device) for R in rows]
    cat = torch.empty(sum(rows), dtype=torch.float16, device=xd.device)

    def run():
        nm.nm_spmv_group([m[3] for m in mats], [m[4] for m in mats], xd, 2, 4, outs=outs)
        torch.cat(outs, out=cat)

    _replay_and_check(run, [xd], cat, lambda i: xd.copy_(up_f16(synth.activation(C, 6600 + i))))


def test_group_argument_errors():
    v, m = up_f16(np.zeros((8, 32), np.float16)), up_u32(np.zeros((8, 2), np.uint32))
    x = up_f16(np.zeros(64, np.float16))
    with pytest.raises(ValueError):
        nm.nm_spmv_group([], [], x, 2, 4)
    with pytest.raises(ValueError):
        nm.nm_spmv_group([v] * 9, [m] * 9, x, 2, 4)
    with pytest.raises(ValueError):
        nm.nm_spmv_group([v], [m], up_f16(np.zeros(96, np.float16)), 2, 4)   # cols disagree
