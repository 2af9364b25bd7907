"""GPU parity tests of the small-batch 50% products on the matrix instructions, through the
C ABI, against the CPU oracle (spmm_ref): nm_spmm_skinny for every 50% pattern (2:4 direct;
4:8 and 8:16 split into two 2:4 operands; 16:32 expanded to dense fragments) on ragged
shapes, and nm_spmm where its routing picks them (5..31 vectors: 2:4 on layers of at least
256 rows; 4:8 and 8:16 on layers of at least 2048 rows, and on smaller ones from 9 or 12
vectors; 16:32 per launch of up to 16 vectors, from 14 vectors on layers of >= 2048 rows
(>= 4096 rows if wider than 4096 columns) and from 12 on >= 4096 rows of <= 4096 columns,
the small-batch kernel for the other launches).

Bars: Y within |y - ref| <= 2e-3 + 1e-2*|ref| per element and relative L2 <= 1e-3 (fp32
accumulation in the matrix instruction, fp16 output, fp64 oracle); exact special cases
(one-hot X) and determinism bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import device, down_bits16, down_f16, down_u32, sample_rows, say, up_f16, up_u32

pytestmark = pytest.mark.gpu
SKINNY = {2: "skinny_spmm_kernel<1, false>", 4: "skinny_spmm_kernel<1, true>", 8: "skinny_spmm_kernel<1, true>",
          16: "skinny_expand_kernel<1>"}
PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]

# (rows, cols, vectors): ragged rows (16-row tiles, row groups of 1..4 tiles), a 32-column
# tail step, steps split over 16 / 8 / 4 waves, X in several column phases (16 vectors x
# 14336 columns > 128 KiB), more than 16 vectors (two launches), 5..31 vectors
CASES = [(2048, 96, 5), (2049, 1056, 8), (2100, 4064, 16), (4100, 1024, 11), (4096, 14336, 16),
         (4100, 14368, 13), (9000, 2080, 17), (14336, 4096, 8), (2600, 544, 31), (16400, 288, 6)]


def check(R, C, T, seed, N=2, M=4, rows_idx=None, fn=nm.nm_spmm):
    W = synth.weight(R, C, seed)
    X = synth.activations(T, C, seed + 1)
    values, masks = nm.nm_pack(up_f16(W), N, M)
    Y = down_f16(fn(values, masks, up_f16(X), N, M))
    idx = np.arange(R) if rows_idx is None else rows_idx
    it = torch.from_numpy(idx).to(device())
    rv, rm = oracle.pack_ref(W[idx], N, M)
    assert np.array_equal(down_u32(masks.index_select(0, it)), rm)
    assert np.array_equal(down_bits16(values.index_select(0, it)), rv)
    rep = oracle.y_tolerance_report(Y[:, idx], oracle.spmm_ref(rv, rm, X, C, N, M))
    assert rep["ok"], ((R, C, T, N, M), rep)
    return rep


@pytest.mark.parametrize("N,M", PATTERNS)
@pytest.mark.parametrize("R,C,T", CASES)
def test_skinny_parity(R, C, T, N, M):
    say(f"skinny {N}:{M} {R}x{C} vectors={T}")
    check(R, C, T, 3000 + R % 97 + C % 89 + T + N, N, M, sample_rows(R, k=32, rpb=16), fn=nm.nm_spmm_skinny)


# nm_spmm's routing to the skinny kernels, 16:32 included (ragged rows, two launches)
# (16:32 at 20 and 24 vectors: an expansion launch of 16, then the small-batch kernel for the
# rest; 31 on 2050 rows: two expansion launches, 16 and 15)
ROUTED_CASES = [((2, 4), 4100, 1024, 11), ((8, 16), 2100, 4064, 16), ((16, 32), 4096, 4096, 12),
                ((16, 32), 4100, 4064, 16), ((16, 32), 14336, 4096, 20), ((16, 32), 4096, 14336, 24),
                ((16, 32), 2050, 4096, 31), ((16, 32), 4100, 8192, 40)]


@pytest.mark.parametrize("pat,R,C,T", ROUTED_CASES)
def test_skinny_routed(pat, R, C, T):
    N, M = pat
    assert nm.spmm_variant(R, C, T, N, M) == SKINNY[N]
    say(f"skinny routed {N}:{M} {R}x{C} vectors={T}")
    check(R, C, T, 3300 + R % 97 + C % 89 + T + N, N, M, sample_rows(R, k=32, rpb=16))


# smaller layers (fewer than 2048 rows): ragged rows, a 32-column tail, one and two launches
SMALL_CASES = [((2, 4), 256, 4096, 5), ((2, 4), 1024, 4096, 8), ((2, 4), 300, 1056, 6), ((2, 4), 1000, 8192, 17),
               ((4, 8), 1024, 4096, 9), ((8, 16), 1030, 5120, 16), ((8, 16), 512, 8192, 12), ((4, 8), 777, 2080, 20)]


@pytest.mark.parametrize("pat,R,C,T", SMALL_CASES)
def test_skinny_small_layers(pat, R, C, T):
    N, M = pat
    assert nm.spmm_variant(R, C, T, N, M) == SKINNY[N]
    say(f"skinny small {N}:{M} {R}x{C} vectors={T}")
    check(R, C, T, 3100 + R % 97 + C % 89 + T + N, N, M)


@pytest.mark.parametrize("N,M", [(4, 8), (8, 16)])
def test_skinny_split_two_launches(N, M):
    """4:8 and 8:16 at 20 vectors: a launch of 16 on the split kernel, then the last 4 on the
    small-batch kernel (a launch too small for the matrix instructions)."""
    R, C, T = 2064, 1024, 20
    assert nm.spmm_variant(R, C, T, N, M) == SKINNY[N]
    say(f"skinny {N}:{M} {R}x{C} vectors={T}")
    check(R, C, T, 3050 + N, N, M, sample_rows(R, k=32, rpb=16))


def test_skinny_routing():
    """Which kernel nm_spmm picks: the sparse matrix instruction at 5..31 vectors for 2:4 on
    layers of >= 256 rows and for 4:8 and 8:16 on layers of >= 2048 rows (on smaller ones from
    9 vectors up to 5120 columns, else from 12); for 16:32, per launch of up to 16 vectors,
    the expansion kernel from 14 vectors on >= 2048 rows (>= 4096 if wider than 4096
    columns) and from 12 on >= 4096 rows of <= 4096 columns; the small-batch kernel below 5
    vectors, on smaller layers and for the other 16:32 launches; the prefill kernels from 32
    vectors on (16:32, which has none, keeps its per-launch routing at any batch)."""
    assert nm.spmm_variant(4096, 4096, 4, 2, 4) == "spmm_kernel<2, 4, 2>"
    assert nm.spmm_variant(2047, 4096, 8, 2, 4) == SKINNY[2]
    assert nm.spmm_variant(1024, 4096, 5, 2, 4) == SKINNY[2]
    assert nm.spmm_variant(256, 8192, 8, 2, 4) == SKINNY[2]
    assert nm.spmm_variant(255, 4096, 8, 2, 4) == "spmm_kernel<2, 8, 2>"
    assert nm.spmm_variant(2047, 4096, 8, 4, 8) == "spmm_kernel<4, 8, 2>"
    assert nm.spmm_variant(1024, 4096, 9, 4, 8) == SKINNY[4]
    assert nm.spmm_variant(1024, 5120, 9, 8, 16) == SKINNY[8]
    assert nm.spmm_variant(1024, 8192, 9, 8, 16) == "spmm_narrow_kernel<8, 8, 2, 2>"
    assert nm.spmm_variant(1024, 8192, 12, 8, 16) == SKINNY[8]
    assert nm.spmm_variant(4096, 4096, 12, 16, 32) == SKINNY[16]
    assert nm.spmm_variant(14336, 4096, 31, 16, 32) == SKINNY[16]
    assert nm.spmm_variant(4096, 4096, 11, 16, 32) == "spmm_kernel<16, 8, 0>"
    assert nm.spmm_variant(4095, 4096, 16, 16, 32) == SKINNY[16]
    assert nm.spmm_variant(4095, 4096, 13, 16, 32) == "spmm_kernel<16, 8, 0>"
    assert nm.spmm_variant(4096, 4128, 16, 16, 32) == SKINNY[16]
    assert nm.spmm_variant(4096, 14336, 12, 16, 32) == "spmm_kernel<16, 8, 0>"
    assert nm.spmm_variant(4096, 14336, 14, 16, 32) == SKINNY[16]
    assert nm.spmm_variant(2048, 4096, 15, 16, 32) == SKINNY[16]
    assert nm.spmm_variant(2048, 8192, 16, 16, 32) == "spmm_kernel<16, 8, 0>"
    assert nm.spmm_variant(2047, 4096, 16, 16, 32) == "spmm_kernel<16, 8, 0>"
    assert nm.spmm_variant(1024, 4096, 16, 16, 32) == "spmm_kernel<16, 8, 0>"
    assert nm.spmm_variant(4096, 4096, 5, 16, 32) == "spmm_kernel<16, 5, 0>"
    assert nm.spmm_variant(4096, 4096, 4, 8, 16) == "spmm_kernel<8, 4, 2>"
    for N, M in PATTERNS[:3]:
        assert nm.spmm_variant(4096, 4096, 5, N, M) == SKINNY[N]
        assert nm.spmm_variant(4096, 4096, 31, N, M) == SKINNY[N]
    # 32..48 vectors stay on 16-vector launches on <= 4096 rows (32 on <= 8192 rows), where
    # the skinny kernels take the layer; the prefill kernels beyond
    assert nm.spmm_variant(4096, 4096, 32, 4, 8) == SKINNY[4]
    assert nm.spmm_variant(4096, 14336, 48, 2, 4) == SKINNY[2]
    assert nm.spmm_variant(4096, 4096, 49, 2, 4).startswith("prefill_spmm_kernel")
    assert nm.spmm_variant(8192, 8192, 32, 2, 4) == SKINNY[2]
    assert nm.spmm_variant(8192, 8192, 33, 2, 4).startswith("prefill_spmm_kernel")
    assert nm.spmm_variant(14336, 4096, 32, 2, 4).startswith("prefill_spmm_kernel")
    assert nm.spmm_variant(4096, 4096, 64, 4, 8).startswith("prefill_split_kernel")
    assert nm.spmm_variant(200, 1024, 40, 2, 4).startswith("prefill_spmm_kernel")   # no skinny below 256 rows
    if torch.cuda.get_device_properties(device()).multi_processor_count == 256:   # the tile model's pick
        assert nm.spmm_variant(4096, 4096, 2048, 8, 16) == "prefill_split_kernel<2, 16, 64, 2>"
    # 16:32: 16-vector launches up to 63 vectors, the expansion prefill kernels from 64
    assert nm.spmm_variant(4096, 4096, 40, 16, 32) == SKINNY[16]
    assert nm.spmm_variant(4096, 4096, 63, 16, 32) == SKINNY[16]
    assert nm.spmm_variant(4096, 4096, 64, 16, 32).startswith("prefill_expand_kernel")
    assert nm.spmm_variant(4096, 4096, 64, 2, 4).startswith("prefill_spmm_kernel")
    assert nm.spmm_variant(4096, 4096, 1, 2, 4).startswith("spmv_kernel")


@pytest.mark.parametrize("N,M", PATTERNS)
def test_skinny_one_hot_and_determinism(N, M):
    """X = 16 rows of the identity (columns 0, 37, ..., spread over the row): token t gives
    column c_t of the pruned matrix bit-exactly; repeated calls give the same bits."""
    R, C = 2080, 4096
    W = synth.weight(R, C, 3100 + N)
    rv, rm = oracle.pack_ref(W, N, M)
    D = oracle.unpack_ref(rv, rm, C, N, M)
    cols = [0, 37, 255, 256, 1000, 2047, 2048, 3001, 4000, 4095, 63, 64, 1, 2, 3, 4094]
    X = np.zeros((16, C), np.float16)
    for t, c in enumerate(cols):
        X[t, c] = 1.0
    v, m = up_f16(rv), up_u32(rm)
    Y = down_bits16(nm.nm_spmm_skinny(v, m, up_f16(X), N, M))
    want = D[:, cols].T.copy()
    want[want == 0x8000] = 0
    assert np.array_equal(Y, want)
    Xr = up_f16(synth.activations(16, C, 3101))
    Y0 = down_bits16(nm.nm_spmm_skinny(v, m, Xr, N, M))
    for _ in range(10):
        assert np.array_equal(down_bits16(nm.nm_spmm_skinny(v, m, Xr, N, M)), Y0)


@pytest.mark.parametrize("N,M", PATTERNS)
def test_skinny_malformed_masks_stay_in_bounds(N, M):
    R, C, T = 2100, 1056, 9
    v = up_f16(synth.weight(R, C // 2, 3200))
    X = up_f16(synth.activations(T, C, 3201))
    for word in (0, 1, 0x80000000, 0xFFFFFFFF, 0x12345678):
        m = torch.full((R, C // 32), np.uint32(word).view(np.int32).item(), dtype=torch.int32, device=device())
        Y = nm.nm_spmm_skinny(v, m, X, N, M)
        torch.cuda.synchronize()
        assert Y.shape == (T, R)


# Column splits (nm_spmm_ws): layers of at most half as many 16-row tiles as CUs take 2, 4 or 8
# workgroups per tile where that pays (rows of >= 64 lines of 128 columns; >= 40 lines from 8
# vectors; the split patterns from 9 vectors), each on a range of whole lines, the last to
# arrive summing the partial tiles. Ragged rows; a ragged last split (8224 columns = 64.25
# lines over 8 splits); several X phases inside one split (16 vectors x 14336 columns).
# (Batches of more than 16 vectors with a workspace of nm_spmm_workspace_bytes take the
# column-split prefill kernel; their skinny launches are covered below with a workspace sized
# for 16 vectors.)
SPLIT_CASES = [((2, 4), 1024, 8192, 8), ((2, 4), 512, 8192, 5), ((2, 4), 300, 8224, 6),
               ((2, 4), 2048, 14336, 16), ((4, 8), 1024, 4096, 9), ((8, 16), 1030, 8192, 16),
               ((8, 16), 512, 8192, 12)]


def _counter_bytes():
    """The counters' region: 4 bytes per CU, rounded up to 256."""
    cus = torch.cuda.get_device_properties(device()).multi_processor_count
    return -(-(4 * cus) // 256) * 256


@pytest.mark.parametrize("pat,R,C,T", SPLIT_CASES)
def test_skinny_column_split(pat, R, C, T):
    N, M = pat
    need = nm.spmm_workspace_bytes(R, C, T, N, M)
    assert need > _counter_bytes(), (R, C, T, need)
    ws = nm.spmm_workspace(R, C, T, N, M)
    say(f"skinny split {N}:{M} {R}x{C} vectors={T} workspace={need}")
    check(R, C, T, 3400 + R % 97 + C % 89 + T + N, N, M,
                fn=lambda v, m, x, n, mm: nm.nm_spmm_ws(v, m, x, n, mm, ws))
    # every call leaves the counters at zero, and repeated calls give the same bits
    assert int(ws[:_counter_bytes()].count_nonzero()) == 0
    W = synth.weight(R, C, 3400 + R % 97 + C % 89 + T + N)
    v, m = nm.nm_pack(up_f16(W), N, M)
    X = up_f16(synth.activations(T, C, 3401 + R % 97 + C % 89 + T + N))
    Y0 = down_bits16(nm.nm_spmm_ws(v, m, X, N, M, ws))
    for _ in range(5):
        assert np.array_equal(down_bits16(nm.nm_spmm_ws(v, m, X, N, M, ws)), Y0)
    assert int(ws[:_counter_bytes()].count_nonzero()) == 0


# two skinny launches on one workspace, both split (31 vectors), or the second on the
# small-batch kernel (17 and 20 vectors: the last 1 or 4), with a workspace sized for 16
# vectors (enough for every skinny launch of the shape, too small for the column-split
# prefill kernel); a ragged last split (2080 columns = 16.25 lines over 4)
MULTI_CASES = [((2, 4), 1000, 8192, 17), ((4, 8), 777, 2080, 31), ((2, 4), 256, 5120, 31), ((2, 4), 1024, 5120, 20)]


@pytest.mark.parametrize("pat,R,C,T", MULTI_CASES)
def test_skinny_column_split_several_launches(pat, R, C, T):
    N, M = pat
    ws = nm.spmm_workspace(R, C, 16, N, M)
    assert ws is not None and ws.numel() < nm.spmm_workspace_bytes(R, C, T, N, M), (R, C, T)
    say(f"skinny split launches {N}:{M} {R}x{C} vectors={T} workspace={ws.numel()}")
    check(R, C, T, 3450 + R % 97 + C % 89 + T + N, N, M,
          fn=lambda v, m, x, n, mm: nm.nm_spmm_ws(v, m, x, n, mm, ws))
    assert int(ws[:_counter_bytes()].count_nonzero()) == 0


def test_skinny_column_split_small_workspace_runs_unsplit():
    """A workspace smaller than nm_spmm_workspace_bytes (or none) runs nm_spmm's kernels:
    bit-identical to nm_spmm; shapes without a split need no workspace."""
    N, M, R, C, T = 2, 4, 1024, 8192, 8
    W = synth.weight(R, C, 3500)
    v, m = nm.nm_pack(up_f16(W), N, M)
    X = up_f16(synth.activations(T, C, 3501))
    want = down_bits16(nm.nm_spmm(v, m, X, N, M))
    need = nm.spmm_workspace_bytes(R, C, T, N, M)
    assert need > 0
    small = torch.zeros(need - 16, dtype=torch.uint8, device=device())
    assert np.array_equal(down_bits16(nm.nm_spmm_ws(v, m, X, N, M, small)), want)
    assert np.array_equal(down_bits16(nm.nm_spmm_ws(v, m, X, N, M, None)), want)
    assert int(small.count_nonzero()) == 0
    # no split: 16:32 up to 16 vectors (expanded fragments), fewer than 5 vectors, layers
    # that fill the GPU, prompts whose prefill grid fills it, and where the hand-off costs
    # more than it saves (2:4 rows of 32 lines)
    assert nm.spmm_workspace_bytes(4096, 4096, 16, 16, 32) == 0
    assert nm.spmm_workspace_bytes(1024, 8192, 4, 2, 4) == 0
    assert nm.spmm_workspace_bytes(4096, 8192, 8, 2, 4) == 0
    assert nm.spmm_workspace_bytes(4096, 4096, 2048, 2, 4) == 0
    assert nm.spmm_workspace_bytes(1024, 4096, 16, 2, 4) == 0
    assert nm.spmm_workspace_bytes(2048, 4096, 16, 4, 8) == 0
    assert nm.spmm_workspace_bytes(1024, 5120, 5, 2, 4) == 0
    # sizes: the counters (4 bytes per CU, rounded up to 256), then 1 KiB per tile and split
    c = _counter_bytes()
    if torch.cuda.get_device_properties(device()).multi_processor_count == 256:
        assert nm.spmm_workspace_bytes(1024, 8192, 8, 2, 4) == c + 64 * 4 * 1024
        assert nm.spmm_workspace_bytes(512, 4096, 12, 8, 16) == c + 32 * 8 * 1024
        assert nm.spmm_workspace_bytes(2048, 8192, 5, 2, 4) == c + 128 * 2 * 1024


def test_skinny_column_split_shared_workspace():
    """One workspace, sized for the largest shape, serves products of more and fewer tiles
    and a pattern change, in stream order (a shape of 128 tiles after ones of 32 and 64
    finds its counters at zero); each matches its own fresh-workspace result."""
    cases = [((2, 4), 1024, 8192, 16), ((8, 16), 512, 4096, 9), ((2, 4), 2048, 8192, 8), ((2, 4), 512, 8192, 5),
             ((2, 4), 2048, 14336, 12), ((2, 4), 1024, 8192, 5)]
    need = max(nm.spmm_workspace_bytes(R, C, T, N, M) for (N, M), R, C, T in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device=device())
    for k, ((N, M), R, C, T) in enumerate(cases):
        W = synth.weight(R, C, 3600 + k)
        v, m = nm.nm_pack(up_f16(W), N, M)
        X = up_f16(synth.activations(T, C, 3610 + k))
        got = down_bits16(nm.nm_spmm_ws(v, m, X, N, M, ws))
        want = down_bits16(nm.nm_spmm_ws(v, m, X, N, M, nm.spmm_workspace(R, C, T, N, M)))
        assert np.array_equal(got, want), ((N, M), R, C, T)


# boundaries of the skinny column split: 128 tiles (half the CUs of a 256-CU part: 2 splits)
# against 129 (none); batch 5 (first skinny size) and 16 (one full launch); a workspace of
# exactly nm_spmm_workspace_bytes
@pytest.mark.parametrize("R,C,T,N,M", [(2048, 8192, 5, 2, 4), (2064, 8192, 8, 2, 4), (2048, 8192, 16, 8, 16),
                                       (1040, 14336, 16, 2, 4)])
def test_skinny_column_split_boundaries(R, C, T, N, M):
    need = nm.spmm_workspace_bytes(R, C, T, N, M)
    cus = torch.cuda.get_device_properties(device()).multi_processor_count
    tiles = -(-R // 16)
    if 2 * tiles > cus:
        assert need == 0, (R, C, T, need)
    else:
        assert need > 0, (R, C, T)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=device())[:need] if need else None
    say(f"skinny split boundary {N}:{M} {R}x{C} vectors={T} workspace={need}")
    W = synth.weight(R, C, 3800 + R % 97 + T)
    X = synth.activations(T, C, 3801 + R % 97 + T)
    v, m = nm.nm_pack(up_f16(W), N, M)
    Xd = up_f16(X)
    got = down_f16(nm.nm_spmm_ws(v, m, Xd, N, M, ws))
    idx = sample_rows(R, k=24, rpb=16)
    rv, rm = oracle.pack_ref(W[idx], N, M)
    rep = oracle.y_tolerance_report(got[:, idx], oracle.spmm_ref(rv, rm, X, C, N, M))
    assert rep["ok"], rep
    if need == 0:   # no split: nm_spmm's kernels, bit for bit
        assert np.array_equal(down_bits16(nm.nm_spmm_ws(v, m, Xd, N, M, ws)), down_bits16(nm.nm_spmm(v, m, Xd, N, M)))
