"""GPU tests of nm_unpack (the decoder, inverse of nm_pack) through the C ABI, against the
CPU oracle (unpack_ref): bit-exact, every pattern, ragged shapes; and the route it opens for
prefill-sized products of the patterns without a sparse matrix path (decode once, then the
dense matrix-core product)."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import device, down_bits16, down_f16, say, up_f16, up_u32

pytestmark = pytest.mark.gpu
SHAPES = [(1, 32), (3, 64), (17, 96), (37, 544), (256, 4096), (1000, 2080), (4100, 1056)]


@pytest.mark.parametrize("N,M", synth.PATTERNS + synth.PATTERNS_QUARTER)
def test_unpack_bit_exact(N, M):
    for i, (R, C) in enumerate(SHAPES):
        W = synth.weight(R, C, 3300 + i) if i % 2 == 0 else synth.tie_heavy_weight(R, C, 3350 + i)
        rv, rm = oracle.pack_ref(W, N, M)
        D = down_bits16(nm.nm_unpack(up_f16(rv), up_u32(rm), N, M))
        assert np.array_equal(D, oracle.unpack_ref(rv, rm, C, N, M)), (R, C)
        values, masks = nm.nm_pack(up_f16(W), N, M)          # GPU round trip
        assert np.array_equal(down_bits16(nm.nm_unpack(values, masks, N, M)), D), (R, C)


def test_unpack_malformed_masks_stay_in_bounds():
    R, C = 64, 1024
    v = up_f16(synth.weight(R, C // 2, 3400))
    for word in (0, 1, 0xFFFFFFFF, 0x12345678):
        m = torch.full((R, C // 32), np.uint32(word).view(np.int32).item(), dtype=torch.int32, device=device())
        D = nm.nm_unpack(v, m, 2, 4)
        torch.cuda.synchronize()
        assert D.shape == (R, C)


@pytest.mark.parametrize("N,M", ((4, 8), (16, 32)))
def test_unpack_then_dense_prefill(N, M):
    """A prefill-sized batch of a 4:8 / 16:32 matrix: decode once, then the dense
    matrix-core product, within tolerance of the oracle's sparse product."""
    R, C, T = 1000, 2080, 300
    W = synth.weight(R, C, 3500 + N)
    X = synth.activations(T, C, 3501 + N)
    say(f"unpack + dense prefill {N}:{M} {R}x{C} tokens={T}")
    values, masks = nm.nm_pack(up_f16(W), N, M)
    Y = down_f16(nm.nm_gemm_dense_prefill(nm.nm_unpack(values, masks, N, M), up_f16(X)))
    rv, rm = oracle.pack_ref(W, N, M)
    rep = oracle.y_tolerance_report(Y, oracle.spmm_ref(rv, rm, X, C, N, M))
    assert rep["ok"], rep
