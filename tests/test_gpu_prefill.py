"""GPU parity tests of the prefill products on the matrix cores (nm_spmm_prefill: 2:4 on the
sparse matrix instruction; nm_gemm_dense_prefill: dense) through the C ABI, against the CPU
oracle (spmm_ref, gemm_ref), and of the batch routing of nm_spmm / nm_gemm_dense.

Bars: Y within |y - ref| <= 2e-3 + 1e-2*|ref| per element and relative L2 <= 1e-3 (fp32
accumulation in the matrix instruction, fp16 output, fp64 oracle); exact special cases
(one-hot X) and structural properties (determinism, routing to the same kernel) bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import device, down_bits16, down_f16, down_u32, sample_rows, say, up_f16, up_u32

pytestmark = pytest.mark.gpu

# (rows, cols, tokens): ragged rows (tiles of 16, 64, 128 and 256 rows), ragged tokens
# (tiles of 16, 64, 128 and 256), a 32-column tail step, one step, many steps, a last block
# of mask steps cut short; every tile configuration the sparse kernel picks (64 x 64,
# 64 x 128, 128 x 64, 128 x 128, 256 x 128, 256 x 256: the larger ones where their grid
# still fills the CUs) and both of the dense kernel's
SMALL = [(1, 32, 1), (17, 64, 5), (16, 96, 16), (33, 128, 17), (64, 4064, 63), (65, 4096, 64),
         (127, 544, 65), (300, 1056, 255), (129, 2080, 257), (1000, 4064, 700), (4100, 1024, 2050),
         (4096, 160, 2048), (2600, 2208, 3000), (16400, 160, 1100), (16448, 160, 16), (16448, 1056, 80),
         (5440, 1056, 336)]


def check_prefill(W, X, tag, rows_idx=None, dense=True):
    """Pack on the GPU (checked bit-exact against the oracle on the compared rows), run the
    sparse and dense prefill products and compare the rows `rows_idx` (all if None) with
    the oracle over every token."""
    R, C = W.shape
    Wd = up_f16(W)
    values, masks = nm.nm_pack(Wd, 2, 4)
    Xd = up_f16(X)
    Y = down_f16(nm.nm_spmm_prefill(values, masks, Xd))
    Yd = down_f16(nm.nm_gemm_dense_prefill(Wd, Xd)) if dense else None
    idx = np.arange(R) if rows_idx is None else rows_idx
    it = torch.from_numpy(idx).to(device())
    rv, rm = oracle.pack_ref(W[idx], 2, 4)
    assert np.array_equal(down_u32(masks.index_select(0, it)), rm), tag
    assert np.array_equal(down_bits16(values.index_select(0, it)), rv), tag
    rep = oracle.y_tolerance_report(Y[:, idx], oracle.spmm_ref(rv, rm, X, C, 2, 4))
    assert rep["ok"], (tag, "sparse", rep)
    if dense:
        drep = oracle.y_tolerance_report(Yd[:, idx], oracle.gemm_ref(W[idx], X))
        assert drep["ok"], (tag, "dense", drep)
    return rep


def test_prefill_small_and_ragged():
    for i, (R, C, T) in enumerate(SMALL):
        say(f"prefill {R}x{C} tokens={T} {nm.prefill_variant(R, C, T, True)} / {nm.prefill_variant(R, C, T, False)}")
        W = synth.weight(R, C, seed=2100 + i)
        X = synth.activations(T, C, seed=2150 + i)
        rows_idx = None if R * T <= 300 * 300 else sample_rows(R, rpb=128)
        check_prefill(W, X, (R, C, T), rows_idx)


def test_prefill_both_tile_configurations_are_exercised():
    """The shapes above cover the small and the large tile configuration of both products."""
    if torch.cuda.get_device_properties(device()).multi_processor_count != 256:
        pytest.skip("the shapes are chosen for a 256-CU part")
    names = {nm.prefill_variant(R, C, T, s) for R, C, T in SMALL for s in (True, False)}
    assert names == {"prefill_spmm_kernel<1, 4, 64, 2>", "prefill_spmm_kernel<1, 8, 64, 2>",
                     "prefill_spmm_kernel<2, 4, 64, 2>",
                     "prefill_spmm_kernel<2, 8, 64, 2>", "prefill_spmm_kernel<4, 8, 64, 2>",
                     "prefill_spmm_kernel<4, 16, 64, 2>",
                     "prefill_gemm_kernel<1, 4, 64, 2>", "prefill_gemm_kernel<2, 16, 64, 2>"}, names


def test_prefill_one_hot_tokens_are_exact():
    """X = rows of the identity: token t gives column t of the pruned matrix, bit-exactly
    (one nonzero product, exact in fp32), for the sparse and the dense product."""
    R, C = 200, 256
    W = synth.weight(R, C, seed=2200)
    X = np.eye(C, dtype=np.float16)
    rv, rm = oracle.pack_ref(W, 2, 4)
    D = oracle.unpack_ref(rv, rm, C, 2, 4)            # pruned matrix, fp16 bits
    Y = down_bits16(nm.nm_spmm_prefill(up_f16(rv), up_u32(rm), up_f16(X)))
    want = D.T.copy()
    want[want == 0x8000] = 0                          # -0 weights give +0 in the fp32 sum
    assert np.array_equal(Y, want)
    Yd = down_bits16(nm.nm_gemm_dense_prefill(up_f16(W), up_f16(X)))
    wd = W.view(np.uint16).T.copy()
    wd[wd == 0x8000] = 0
    assert np.array_equal(Yd, wd)


def test_prefill_deterministic_and_unaligned_output():
    """Repeated calls give the same bits; an output not 8-byte aligned (scalar stores) gives
    the same bits as an aligned one."""
    R, C, T = 300, 1024, 300
    W = synth.weight(R, C, seed=2300)
    X = up_f16(synth.activations(T, C, seed=2301))
    rv, rm = oracle.pack_ref(W, 2, 4)
    v, m = up_f16(rv), up_u32(rm)
    Y0 = down_bits16(nm.nm_spmm_prefill(v, m, X))
    for _ in range(10):
        assert np.array_equal(down_bits16(nm.nm_spmm_prefill(v, m, X)), Y0)
    R4 = 256                                          # rows % 4 == 0: vector stores when aligned
    v4, m4 = up_f16(rv[:R4]), up_u32(rm[:R4])
    Ya = down_bits16(nm.nm_spmm_prefill(v4, m4, X))
    buf = torch.empty(T * R4 + 1, dtype=torch.float16, device=device())
    out = buf[1:].view(T, R4)
    nm.nm_spmm_prefill(v4, m4, X, out=out)
    assert np.array_equal(down_bits16(out), Ya)
    assert np.array_equal(Ya, Y0[:, :R4])


def test_batch_entry_points_route_to_prefill():
    """nm_spmm with 2:4 and nm_gemm_dense from 32 vectors on run the matrix-core kernels
    (same bits); below 32 vectors, and for the other 50% patterns at any size, the
    small-batch kernel runs 8 vectors at a time (within tolerance of the oracle;
    bit-identical per group)."""
    R, C = 200, 1024
    W = synth.weight(R, C, seed=2400)
    X40 = synth.activations(40, C, seed=2402)
    rv, rm = oracle.pack_ref(W, 2, 4)
    v, m = up_f16(rv), up_u32(rm)
    Xd = up_f16(X40)
    assert np.array_equal(down_bits16(nm.nm_spmm(v, m, Xd, 2, 4)), down_bits16(nm.nm_spmm_prefill(v, m, Xd)))
    assert np.array_equal(down_bits16(nm.nm_gemm_dense(up_f16(W), Xd)),
                          down_bits16(nm.nm_gemm_dense_prefill(up_f16(W), Xd)))
    T = 21
    X = synth.activations(T, C, seed=2401)
    Xd = up_f16(X)
    Yd = nm.nm_gemm_dense(up_f16(W), Xd)
    drep = oracle.y_tolerance_report(down_f16(Yd), oracle.gemm_ref(W, X))
    assert drep["ok"], drep
    assert np.array_equal(down_bits16(Yd)[8:16], down_bits16(nm.nm_gemm_dense(up_f16(W), up_f16(X[8:16]))))
    for N, M in ((2, 4), (4, 8), (8, 16), (16, 32)):
        rv, rm = oracle.pack_ref(W, N, M)
        v, m = up_f16(rv), up_u32(rm)
        Y = nm.nm_spmm(v, m, Xd, N, M)
        rep = oracle.y_tolerance_report(down_f16(Y), oracle.spmm_ref(rv, rm, X, C, N, M))
        assert rep["ok"], (N, M, rep)
        Y8 = nm.nm_spmm(v, m, up_f16(X[8:16]), N, M)
        assert np.array_equal(down_bits16(Y)[8:16], down_bits16(Y8))


def test_prefill_malformed_masks_stay_in_bounds():
    """Masks without two bits per 4-column group give an unspecified Y but the kernel runs
    to completion (every access is range-checked)."""
    R, C, T = 130, 1056, 70
    v = up_f16(synth.weight(R, C // 2, seed=2500))
    X = up_f16(synth.activations(T, C, seed=2501))
    for word in (0, 1, 0x80000000, 0xFFFFFFFF, 0x12345678):
        m = torch.full((R, C // 32), np.uint32(word).view(np.int32).item(), dtype=torch.int32, device=device())
        Y = nm.nm_spmm_prefill(v, m, X)
        torch.cuda.synchronize()
        assert Y.shape == (T, R)


def test_prefill_argument_errors():
    v = torch.zeros((4, 64), dtype=torch.float16, device=device())
    m = torch.zeros((4, 4), dtype=torch.int32, device=device())
    X = torch.zeros((3, 128), dtype=torch.float16, device=device())
    with pytest.raises(nm.NMArgumentError) as e:   # a 25% pattern: no matrix-core product
        nm.nm_spmm_prefill(torch.zeros((4, 32), dtype=torch.float16, device=device()), m, X, 1, 4)
    assert e.value.status == nm.NM_ERR_PATTERN
    with pytest.raises(ValueError):
        nm.nm_spmm_prefill(v, m, torch.zeros((3, 96), dtype=torch.float16, device=device()))


def _full_size_cases():
    return [pytest.param(name, R, C, id=f"{name}-{R}x{C}") for name, R, C in synth.LLAMA31_8B]


@pytest.mark.parametrize("name,R,C", _full_size_cases())
def test_prefill_full_size_llama8b(name, R, C):
    """The Llama-3.1-8B projection shapes with a 2048-token prompt, in the configuration
    the benchmark times: pack bit-exact and Y within tolerance on sampled rows (all tokens)."""
    T = 2048
    say(f"prefill full-size {name} {R}x{C} tokens={T} {nm.prefill_variant(R, C, T, True)}")
    W = synth.weight(R, C, synth.weight_seed(6, [l[0] for l in synth.LLAMA31_8B].index(name), (2, 4)))
    X = synth.activations(T, C, synth.x_seed(6, 0, (2, 4)))
    check_prefill(W, X, name, sample_rows(R, k=24, rpb=128))


# 4:8 and 8:16 (split into two 2:4 operands): ragged rows and tokens, a 32-column tail step,
# every tile configuration the split kernel picks (64 x 64, 64 x 128, 128 x 64, 128 x 128,
# 128 x 256, 256 x 128, 256 x 256)
SPLIT_SMALL = [(17, 64, 5), (33, 128, 17), (65, 4096, 64), (300, 1056, 255), (129, 2080, 257), (4100, 1024, 2050),
               (16400, 160, 1100), (2600, 2208, 3000), (16448, 1056, 16), (19648, 160, 272), (8256, 1056, 65)]
SPLIT_NAMES = {"prefill_split_kernel<1, 4, 64, 2>", "prefill_split_kernel<1, 8, 64, 2>",
               "prefill_split_kernel<2, 4, 64, 2>",
               "prefill_split_kernel<2, 8, 64, 2>", "prefill_split_kernel<2, 16, 64, 2>",
               "prefill_split_kernel<4, 8, 64, 2>", "prefill_split_kernel<4, 16, 64, 2>"}


def check_split(W, X, N, M, tag, rows_idx=None):
    R, C = W.shape
    values, masks = nm.nm_pack(up_f16(W), N, M)
    Y = down_f16(nm.nm_spmm_prefill(values, masks, up_f16(X), N, M))
    idx = np.arange(R) if rows_idx is None else rows_idx
    rv, rm = oracle.pack_ref(W[idx], N, M)
    rep = oracle.y_tolerance_report(Y[:, idx], oracle.spmm_ref(rv, rm, X, C, N, M))
    assert rep["ok"], (tag, N, M, rep)
    return rep


@pytest.mark.parametrize("N,M", [(4, 8), (8, 16)])
def test_prefill_split_small_and_ragged(N, M):
    names = set()
    for i, (R, C, T) in enumerate(SPLIT_SMALL):
        names.add(nm.prefill_variant(R, C, T, True, split=True))
        say(f"prefill split {N}:{M} {R}x{C} tokens={T} {nm.prefill_variant(R, C, T, True, split=True)}")
        W = synth.weight(R, C, seed=2600 + 10 * i + N)
        X = synth.activations(T, C, seed=2650 + i)
        check_split(W, X, N, M, (R, C, T), None if R * T <= 300 * 300 else sample_rows(R, rpb=128))
    if torch.cuda.get_device_properties(device()).multi_processor_count == 256:   # shapes chosen for 256 CUs
        assert names == SPLIT_NAMES, names


@pytest.mark.parametrize("N,M", [(4, 8), (8, 16)])
def test_prefill_split_one_hot_and_routing(N, M):
    """One-hot tokens give the pruned matrix's columns bit-exactly; nm_spmm from 32 vectors
    on runs the same kernel (same bits), and the result is deterministic."""
    R, C = 200, 256
    W = synth.weight(R, C, seed=2700 + N)
    rv, rm = oracle.pack_ref(W, N, M)
    D = oracle.unpack_ref(rv, rm, C, N, M)
    X = np.eye(C, dtype=np.float16)
    v, m = up_f16(rv), up_u32(rm)
    Y = down_bits16(nm.nm_spmm_prefill(v, m, up_f16(X), N, M))
    want = D.T.copy()
    want[want == 0x8000] = 0
    assert np.array_equal(Y, want)
    Xr = up_f16(synth.activations(40, C, seed=2701))
    assert nm.spmm_variant(R, C, 40, N, M).startswith("prefill_split_kernel")
    Y0 = down_bits16(nm.nm_spmm_prefill(v, m, Xr, N, M))
    assert np.array_equal(down_bits16(nm.nm_spmm(v, m, Xr, N, M)), Y0)
    for _ in range(5):
        assert np.array_equal(down_bits16(nm.nm_spmm_prefill(v, m, Xr, N, M)), Y0)


@pytest.mark.parametrize("N,M", [(4, 8), (8, 16)])
def test_prefill_split_malformed_masks_stay_in_bounds(N, M):
    R, C, T = 130, 1056, 70
    v = up_f16(synth.weight(R, C // 2, seed=2800))
    X = up_f16(synth.activations(T, C, seed=2801))
    for word in (0, 1, 0x80000000, 0xFFFFFFFF, 0x12345678):
        m = torch.full((R, C // 32), np.uint32(word).view(np.int32).item(), dtype=torch.int32, device=device())
        Y = nm.nm_spmm_prefill(v, m, X, N, M)
        torch.cuda.synchronize()
        assert Y.shape == (T, R)


@pytest.mark.parametrize("N,M", [(4, 8), (8, 16)])
def test_prefill_split_full_size_down_proj(N, M):
    """The Llama-3.1-8B down projection (4096 x 14336) with a 2048-token prompt, in the
    configuration nm_spmm_prefill picks: Y within tolerance on sampled rows (all tokens)."""
    R, C, T = 4096, 14336, 2048
    say(f"prefill split full-size {N}:{M} {R}x{C} tokens={T} {nm.prefill_variant(R, C, T, True, split=True)}")
    W = synth.weight(R, C, synth.weight_seed(6, 3, (N, M)))
    X = synth.activations(T, C, synth.x_seed(6, 0, (N, M)))
    check_split(W, X, N, M, "down", sample_rows(R, k=24, rpb=128))


# Column splits (nm_spmm_ws with a workspace of nm_spmm_workspace_bytes, batches of more than
# 16 vectors whose prefill grid leaves CUs idle): ragged rows (64-row tiles; rows % 8 != 0 on
# the direct stores), ragged tokens (32- and 64-token tiles), columns ending inside a
# 512-column block and a last split of one 32-column step (1056 columns over 2 splits),
# 2, 4, 7 (uneven: 28 blocks of 4) and 8 splits, one and two workgroups per CU
COLSPLIT = [(1000, 4064, 17), (130, 1056, 100), (1024, 4096, 32), (2048, 8192, 48), (4096, 4096, 64),
            (4096, 14336, 40), (1024, 8192, 256), (14336, 4096, 20), (4100, 1024, 150)]
COLSPLIT_NAMES = {(N, M): {f"prefill_colsplit_kernel<1, {tt}, 64, 2, {'false' if N == 2 else 'true'}>" for tt in (2, 4)}
                  for N, M in ((2, 4), (4, 8), (8, 16))}
COLSPLIT_NAMES[(16, 32)] = {f"prefill_colsplit_expand_kernel<1, {tt}, 64, 2>" for tt in (2, 4)}


def _counter_bytes():
    cus = torch.cuda.get_device_properties(device()).multi_processor_count
    return -(-(4 * cus) // 256) * 256


@pytest.mark.parametrize("N,M", [(2, 4), (4, 8), (8, 16), (16, 32)])
def test_colsplit_small_and_ragged(N, M):
    names = set()
    for i, (R, C, T) in enumerate(COLSPLIT):
        name = nm.spmm_ws_variant(R, C, T, N, M)
        names.add(name)
        need = nm.spmm_workspace_bytes(R, C, T, N, M)
        say(f"colsplit {N}:{M} {R}x{C} tokens={T} {name} workspace={need}")
        assert name in COLSPLIT_NAMES[(N, M)], (R, C, T, name)
        W = synth.weight(R, C, seed=4100 + 10 * i + N)
        X = synth.activations(T, C, seed=4150 + i)
        values, masks = nm.nm_pack(up_f16(W), N, M)
        ws = nm.spmm_workspace(R, C, T, N, M)
        assert ws.numel() == need
        Y = down_f16(nm.nm_spmm_ws(values, masks, up_f16(X), N, M, ws))
        assert int(ws[:_counter_bytes()].count_nonzero()) == 0   # every launch leaves them zero
        idx = np.arange(R) if R * T <= 300 * 300 else sample_rows(R, k=24, rpb=64)
        rv, rm = oracle.pack_ref(W[idx], N, M)
        rep = oracle.y_tolerance_report(Y[:, idx], oracle.spmm_ref(rv, rm, X, C, N, M))
        assert rep["ok"], ((R, C, T), N, M, rep)
    assert names == COLSPLIT_NAMES[(N, M)], names


def test_colsplit_one_hot_deterministic_and_shared_workspace():
    """One-hot tokens give the pruned matrix's columns bit-exactly (one nonzero product per
    output, the other splits add zeros); repeated calls give the same bits; one workspace
    sized for the largest shape serves a sequence of shapes and patterns, each bit-identical
    to its own fresh workspace's result."""
    R, C = 1000, 4096
    W = synth.weight(R, C, seed=4200)
    rv, rm = oracle.pack_ref(W, 2, 4)
    D = oracle.unpack_ref(rv, rm, C, 2, 4)
    X = np.eye(C, dtype=np.float16)[:40]
    v, m = up_f16(rv), up_u32(rm)
    assert nm.spmm_ws_variant(R, C, 40, 2, 4).startswith("prefill_colsplit_kernel")
    ws = nm.spmm_workspace(R, C, 40, 2, 4)
    Y = down_bits16(nm.nm_spmm_ws(v, m, up_f16(X), 2, 4, ws))
    want = D.T[:40].copy()
    want[want == 0x8000] = 0
    assert np.array_equal(Y, want)
    Xr = up_f16(synth.activations(40, C, seed=4201))
    Y0 = down_bits16(nm.nm_spmm_ws(v, m, Xr, 2, 4, ws))
    for _ in range(5):
        assert np.array_equal(down_bits16(nm.nm_spmm_ws(v, m, Xr, 2, 4, ws)), Y0)
    cases = [((2, 4), 1024, 4096, 32), ((8, 16), 4096, 14336, 40), ((2, 4), 130, 1056, 100), ((4, 8), 2048, 8192, 17),
             ((2, 4), 1024, 8192, 16)]
    big = torch.zeros(max(nm.spmm_workspace_bytes(R, C, T, N, M) for (N, M), R, C, T in cases), dtype=torch.uint8,
                      device=device())
    for k, ((N, M), R, C, T) in enumerate(cases):
        Wk = synth.weight(R, C, 4210 + k)
        vk, mk = nm.nm_pack(up_f16(Wk), N, M)
        Xk = up_f16(synth.activations(T, C, 4220 + k))
        got = down_bits16(nm.nm_spmm_ws(vk, mk, Xk, N, M, big))
        assert np.array_equal(got, down_bits16(nm.nm_spmm_ws(vk, mk, Xk, N, M, nm.spmm_workspace(R, C, T, N, M)))), k


def test_colsplit_small_workspace_takes_nm_spmm_route():
    """A workspace smaller than the column split needs (or none) runs nm_spmm's route, bit for
    bit: the prefill kernel at 64 vectors, skinny launches at 32 on a small layer."""
    for R, C, T in ((4096, 14336, 64), (1024, 4096, 32)):
        W = synth.weight(R, C, 4300 + T)
        v, m = nm.nm_pack(up_f16(W), 2, 4)
        X = up_f16(synth.activations(T, C, 4301 + T))
        need = nm.spmm_workspace_bytes(R, C, T, 2, 4)
        assert need > 0
        small = torch.zeros(need - 16, dtype=torch.uint8, device=device())
        want = down_bits16(nm.nm_spmm(v, m, X, 2, 4))
        assert np.array_equal(down_bits16(nm.nm_spmm_ws(v, m, X, 2, 4, None)), want)
        got = down_bits16(nm.nm_spmm_ws(v, m, X, 2, 4, small))
        if nm.spmm_variant(R, C, T, 2, 4).startswith("prefill"):
            assert np.array_equal(got, want)
        else:   # skinny launches may split their columns with the smaller workspace
            rv, rm = oracle.pack_ref(W[:64], 2, 4)
            rep = oracle.y_tolerance_report(down_f16(nm.nm_spmm_ws(v, m, X, 2, 4, small))[:, :64],
                                            oracle.spmm_ref(rv, rm, down_f16(X), C, 2, 4))
            assert rep["ok"], rep


# 16:32 (fragments expanded for the dense instruction): ragged rows and tokens, a 32-column
# tail step, a last block of mask steps cut short, every tile configuration it picks (64 x 64,
# 64 x 128, 64 x 256, 128 x 64, 128 x 128, 128 x 256)
EXPAND_SMALL = [(17, 64, 5), (33, 128, 17), (65, 4096, 64), (300, 1056, 255), (8256, 160, 65), (16448, 1056, 65),
                (2600, 2208, 3000), (10944, 160, 144), (16448, 160, 16)]
EXPAND_NAMES = {"prefill_expand_kernel<1, 4, 64, 2>", "prefill_expand_kernel<1, 8, 64, 2>",
                "prefill_expand_kernel<1, 16, 64, 2>", "prefill_expand_kernel<2, 4, 64, 2>",
                "prefill_expand_kernel<2, 8, 64, 2>", "prefill_expand_kernel<2, 16, 64, 2>"}


def test_prefill_expand_small_and_ragged():
    names = set()
    for i, (R, C, T) in enumerate(EXPAND_SMALL):
        names.add(nm.prefill_variant(R, C, T, True, expand=True))
        say(f"prefill 16:32 {R}x{C} tokens={T} {nm.prefill_variant(R, C, T, True, expand=True)}")
        W = synth.weight(R, C, seed=2900 + i)
        X = synth.activations(T, C, seed=2950 + i)
        check_split(W, X, 16, 32, (R, C, T), None if R * T <= 300 * 300 else sample_rows(R, rpb=128))
    if torch.cuda.get_device_properties(device()).multi_processor_count == 256:   # shapes chosen for 256 CUs
        assert names == EXPAND_NAMES, names


def test_prefill_expand_one_hot_routing_and_malformed_masks():
    """One-hot tokens give the pruned matrix's columns bit-exactly; nm_spmm from 64 vectors
    runs the same kernel (same bits) and below keeps its 16-vector launches; the result is
    deterministic; masks that are not 16:32 stay in bounds."""
    R, C = 200, 256
    W = synth.weight(R, C, seed=2990)
    rv, rm = oracle.pack_ref(W, 16, 32)
    D = oracle.unpack_ref(rv, rm, C, 16, 32)
    X = np.eye(C, dtype=np.float16)
    v, m = up_f16(rv), up_u32(rm)
    Y = down_bits16(nm.nm_spmm_prefill(v, m, up_f16(X), 16, 32))
    want = D.T.copy()
    want[want == 0x8000] = 0
    assert np.array_equal(Y, want)
    Xr = up_f16(synth.activations(70, C, seed=2991))
    assert nm.spmm_variant(R, C, 70, 16, 32).startswith("prefill_expand_kernel")
    assert not nm.spmm_variant(R, C, 63, 16, 32).startswith("prefill")
    Y0 = down_bits16(nm.nm_spmm_prefill(v, m, Xr, 16, 32))
    assert np.array_equal(down_bits16(nm.nm_spmm(v, m, Xr, 16, 32)), Y0)
    for _ in range(5):
        assert np.array_equal(down_bits16(nm.nm_spmm_prefill(v, m, Xr, 16, 32)), Y0)
    for word in (0, 1, 0xFFFFFFFF, 0x12345678):
        mm = torch.full((R, C // 32), np.uint32(word).view(np.int32).item(), dtype=torch.int32, device=device())
        Yb = nm.nm_spmm_prefill(v, mm, Xr, 16, 32)
        torch.cuda.synchronize()
        assert Yb.shape == (70, R)


@pytest.mark.parametrize("R,C,T", [(1000, 4064, 12), (2048, 4096, 16), (300, 1056, 13)])
def test_colsplit_expand_small_batches(R, C, T):
    """16:32 at 12..16 vectors on layers of at most 2048 rows takes the column-split
    expansion kernel with a workspace (Y within tolerance of the oracle on every row); on
    larger layers, or with fewer vectors, nm_spmm's route."""
    name = nm.spmm_ws_variant(R, C, T, 16, 32)
    say(f"colsplit 16:32 small batch {R}x{C} vectors={T} {name}")
    assert name in COLSPLIT_NAMES[(16, 32)], name
    W = synth.weight(R, C, seed=4400 + T)
    X = synth.activations(T, C, seed=4401 + T)
    v, m = nm.nm_pack(up_f16(W), 16, 32)
    ws = nm.spmm_workspace(R, C, T, 16, 32)
    Y = down_f16(nm.nm_spmm_ws(v, m, up_f16(X), 16, 32, ws))
    assert int(ws[:_counter_bytes()].count_nonzero()) == 0
    rv, rm = oracle.pack_ref(W, 16, 32)
    rep = oracle.y_tolerance_report(Y, oracle.spmm_ref(rv, rm, X, C, 16, 32))
    assert rep["ok"], rep
    assert nm.spmm_ws_variant(4096, 4096, 16, 16, 32) == nm.spmm_variant(4096, 4096, 16, 16, 32)
    assert nm.spmm_ws_variant(R, C, 11, 16, 32) == nm.spmm_variant(R, C, 11, 16, 32)


# Prompts of more than 128 tokens whose columns split better over taller tiles (nm_spmm_ws):
# 256 x 128 (2:4) and 128 x 128 tiles, 2, 4 and 8 splits, ragged rows (tiles of 128 and 256
# rows), ragged tokens (128-token tiles), columns ending inside a 512-column block, an uneven
# last split (28 blocks over 4), one and several hand-off rounds of partial loads
_CS = "prefill_colsplit_kernel"
TALL = {(2, 4): [(4000, 14304, 300, _CS + "<4, 8, 64, 2, false>"), (2050, 10240, 260, _CS + "<2, 8, 64, 2, false>"),
                 (1900, 8160, 1000, _CS + "<4, 8, 64, 2, false>"), (8100, 8160, 290, _CS + "<4, 8, 64, 2, false>")],
        (4, 8): [(4000, 14304, 300, _CS + "<2, 8, 64, 2, true>"), (1900, 8160, 1000, _CS + "<2, 8, 64, 2, true>")],
        (8, 16): [(2050, 10240, 260, _CS + "<2, 8, 64, 2, true>"), (3000, 6144, 600, _CS + "<2, 8, 64, 2, true>")],
        (16, 32): [(4000, 14304, 300, "prefill_colsplit_expand_kernel<2, 8, 64, 2>"),
                   (2050, 10240, 300, "prefill_colsplit_expand_kernel<2, 8, 64, 2>"),
                   (1900, 8160, 150, "prefill_colsplit_expand_kernel<2, 8, 64, 2>")]}


@pytest.mark.parametrize("N,M", [(2, 4), (4, 8), (8, 16), (16, 32)])
def test_tall_colsplit_ragged(N, M):
    """The taller column splits: Y within the oracle's tolerance on sampled rows (every token),
    the counters left at zero, the same bits on a second call; a workspace one block too small
    for them runs the route that ran before (within tolerance of the same rows)."""
    for i, (R, C, T, tmpl) in enumerate(TALL[(N, M)]):
        name = nm.spmm_ws_variant(R, C, T, N, M)
        need = nm.spmm_workspace_bytes(R, C, T, N, M)
        say(f"tall colsplit {N}:{M} {R}x{C} tokens={T} {name} workspace={need}")
        assert name == tmpl, (R, C, T, name)
        W = synth.weight(R, C, seed=4500 + 10 * i + N)
        X = synth.activations(T, C, seed=4550 + i)
        values, masks = nm.nm_pack(up_f16(W), N, M)
        Xd = up_f16(X)
        ws = nm.spmm_workspace(R, C, T, N, M)
        Yb = down_bits16(nm.nm_spmm_ws(values, masks, Xd, N, M, ws))
        assert int(ws[:_counter_bytes()].count_nonzero()) == 0
        assert np.array_equal(down_bits16(nm.nm_spmm_ws(values, masks, Xd, N, M, ws)), Yb)
        idx = sample_rows(R, k=24, rpb=128)
        rv, rm = oracle.pack_ref(W[idx], N, M)
        ref = oracle.spmm_ref(rv, rm, X, C, N, M)
        rep = oracle.y_tolerance_report(Yb.view(np.float16)[:, idx], ref)
        assert rep["ok"], ((R, C, T), N, M, rep)
        small = torch.zeros(need - 256, dtype=torch.uint8, device=device())
        rep = oracle.y_tolerance_report(down_f16(nm.nm_spmm_ws(values, masks, Xd, N, M, small))[:, idx], ref)
        assert rep["ok"], ((R, C, T), N, M, "smaller workspace", rep)


@pytest.mark.parametrize("N,M,R,C,T", [(2, 4, 4000, 14304, 300), (4, 8, 1900, 8160, 1000)])
def test_tall_colsplit_one_hot_columns_are_exact(N, M, R, C, T):
    """Token t one-hot at column (37 t) mod C, so the nonzero products fall in every split:
    each output is one kept weight (the other splits add zeros), bit-exact."""
    W = synth.weight(R, C, seed=4600 + N)
    rv, rm = oracle.pack_ref(W, N, M)
    D = oracle.unpack_ref(rv, rm, C, N, M)
    cols = (37 * np.arange(T)) % C
    X = np.zeros((T, C), dtype=np.float16)
    X[np.arange(T), cols] = 1.0
    assert nm.spmm_ws_variant(R, C, T, N, M).startswith("prefill_colsplit_kernel<" + ("4" if N == 2 else "2") + ", 8")
    ws = nm.spmm_workspace(R, C, T, N, M)
    Y = down_bits16(nm.nm_spmm_ws(up_f16(rv), up_u32(rm), up_f16(X), N, M, ws))
    want = D[:, cols].T.copy()
    want[want == 0x8000] = 0
    assert np.array_equal(Y, want)
