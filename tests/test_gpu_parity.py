"""GPU parity tests: the HIP path (through the C ABI) against the CPU oracle.

Bars: nm_pack bit-exact; y within |y - ref| <= 2e-3 + 1e-2*|ref| per element and
relative L2 <= 1e-3 (fp32 accumulation, fp16 output, fp64 oracle); exact special
cases bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import (check_full_layer, device, down_bits16, down_f16, down_u32, sample_rows,
                               say, up_f16, up_u32)

pytestmark = pytest.mark.gpu
PATTERNS = synth.PATTERNS

# small shapes the oracle finishes fast: 1, 2 and 3 mask words (a ragged last step of
# 128 columns), word counts of 4k+1, 4k+2 and 4k+3 after full steps, row counts that are
# not multiples of the workgroup's rows, several workgroups, and layers with fewer and
# more than 8 rows per CU
SMALL = [(1, 32), (3, 64), (17, 96), (5, 160), (9, 192), (7, 224), (37, 544), (16, 4096),
         (100, 2080), (256, 512), (33, 1056), (2100, 96), (2064, 160)]


def test_native_library_is_the_in_tree_build():
    lib = nm.lib()
    assert lib._name == nm.LIB_PATH
    assert nm.max_cols() >= 28672, "x of the widest layer (28672 columns) must fit in LDS"


@pytest.mark.parametrize("N,M", PATTERNS)
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_pack_bit_exact_small(N, M, kind):
    for i, (R, C) in enumerate(SMALL):
        W = synth.weight(R, C, seed=100 + i) if kind == "normal" else synth.tie_heavy_weight(R, C, seed=200 + i)
        values, masks = nm.nm_pack(up_f16(W), N, M)
        rv, rm = oracle.pack_ref(W, N, M)
        assert np.array_equal(down_u32(masks), rm), (R, C)
        assert np.array_equal(down_bits16(values), rv), (R, C)


@pytest.mark.parametrize("N,M", PATTERNS)
def test_spmv_small(N, M):
    for i, (R, C) in enumerate(SMALL):
        W = synth.weight(R, C, seed=300 + i)
        x = synth.activation(C, seed=400 + i)
        rv, rm = oracle.pack_ref(W, N, M)            # oracle-packed input: no GPU pack involved
        y = nm.nm_spmv(up_f16(rv), up_u32(rm), up_f16(x), N, M)
        rep = oracle.y_tolerance_report(down_f16(y), oracle.spmv_ref(rv, rm, x, C, N, M))
        assert rep["ok"], ((R, C), rep)
        # the GPU-packed input gives the very same bits
        gv, gm = nm.nm_pack(up_f16(W), N, M)
        y2 = nm.nm_spmv(gv, gm, up_f16(x), N, M)
        assert np.array_equal(down_bits16(y2), down_bits16(y)), (R, C)


def test_gemv_small():
    for i, (R, C) in enumerate(SMALL):
        W = synth.weight(R, C, seed=500 + i)
        x = synth.activation(C, seed=600 + i)
        y = nm.nm_gemv_dense(up_f16(W), up_f16(x))
        rep = oracle.y_tolerance_report(down_f16(y), oracle.gemv_ref(W, x))
        assert rep["ok"], ((R, C), rep)


# one or more shapes in each regime of the workgroup-shape rule: narrow layers (at most
# 8 rows per CU), regular rows, long rows (more than 64 steps of 128 columns) in one and
# in two rounds; ragged row counts (the last workgroup holds fewer rows than its row
# groups cover) and ragged column counts (a last step of 1..3 mask words). The long-row
# kernel keeps two batches of 4 steps in flight; its waves see 1, 2, 3 and 4+ full batches
# and 0..3 remaining steps across these shapes (199 x 20000: 12 waves of 13 steps).
REGIMES = [(255, 4096), (2048, 1024), (1500, 2080), (2049, 512), (5121, 4096), (300, 8320),
           (777, 16416), (10241, 8320), (199, 20000), (1023, 4096), (510, 2048), (1024, 2080),
           (1024, 4608)]


@pytest.mark.parametrize("N,M", PATTERNS)
def test_workgroup_regimes(N, M):
    for i, (R, C) in enumerate(REGIMES):
        say(f"regime {R}x{C} {N}:{M} {nm.spmv_launch_shape(R, C, N, M)}")
        W = synth.weight(R, C, seed=800 + i)
        x = synth.activation(C, seed=850 + i)
        check_full_layer(W, x, N, M, f"regime-{R}x{C}", check_dense=(N == 2))


def test_narrow_kernel_routing():
    """16:32 layers of at most 8 rows per CU whose workgroups hold 1, 2 or 4 rows take the
    narrow kernel when the row's steps of 128 columns split into 8 / rows column ranges of
    exactly 4 steps per wave (steps / (4 * 8 / rows) waves); other shapes and patterns keep
    spmv_kernel. The shapes of test_workgroup_regimes and the closed-form tests cover both."""
    assert nm.spmv_variant(1024, 4096, 16, 32) == "spmv_narrow_kernel<16, 4, true, 3, 2>"
    assert nm.spmv_launch_shape(1024, 4096, 16, 32)["waves_per_row_group"] == 4
    assert nm.spmv_variant(1023, 4096, 16, 32) == "spmv_narrow_kernel<16, 4, true, 3, 2>"
    assert nm.spmv_variant(510, 2048, 16, 32) == "spmv_narrow_kernel<16, 4, true, 3, 4>"
    assert nm.spmv_variant(255, 4096, 16, 32) == "spmv_narrow_kernel<16, 4, true, 3, 8>"
    assert nm.spmv_launch_shape(255, 4096, 16, 32)["waves_per_row_group"] == 1
    assert nm.spmv_variant(1024, 4096, 2, 4) == "spmv_kernel<2, 4, true, 1>"   # table decoders
    assert nm.spmv_variant(1024, 4096, 8, 16) == "spmv_kernel<8, 4, true, 2>"
    assert nm.spmv_launch_shape(1024, 4096, 8, 16)["waves_per_row_group"] == 8
    assert nm.spmv_variant(1024, 2080, 16, 32) == "spmv_kernel<16, 4, true, 3>"   # a partial last step
    assert nm.spmv_variant(1024, 4608, 16, 32) == "spmv_kernel<16, 4, true, 3>"   # 36 steps: no 4-step split
    assert nm.spmv_variant(1500, 4096, 16, 32) == "spmv_kernel<16, 4, true, 3>"   # 6 rows per workgroup
    assert nm.spmv_variant(4096, 4096, 16, 32) == "spmv_kernel<16, 4, true, 3>"


def test_config1_single_24():
    """256 x 512, 2:4, the seeded single-layer case."""
    W = synth.weight(256, 512, synth.weight_seed(1, 0, (2, 4)))
    x = synth.activation(512, synth.x_seed(1, 0, (2, 4)))
    rep = check_full_layer(W, x, 2, 4, "cfg1")
    say(f"cfg1 {rep}")


@pytest.mark.parametrize("N,M", PATTERNS)
def test_one_hot_x_is_exact(N, M):
    """x = e_c gives column c of the pruned matrix bit-exactly (one exact product), including
    fp16 subnormal weights, which must not be flushed."""
    R, C = 40, 256
    W = synth.weight(R, C, seed=700)
    # first 32 columns: zeros except a subnormal column 5 and a normal column 1, so both
    # survive the selection under every pattern
    W[:, :32] = 0
    W[:, 5] = (np.float16(2.0 ** -24) * np.arange(1, R + 1)).astype(np.float16)
    W[:, 1] = np.float16(0.75)
    pruned = oracle.prune_ref(W, N, M).view(np.float16)
    values, masks = nm.nm_pack(up_f16(W), N, M)
    for c in (0, 1, 5, 31, 32, 200, 255):
        x = np.zeros(C, np.float16)
        x[c] = 1
        y = down_f16(nm.nm_spmv(values, masks, up_f16(x), N, M))
        assert np.array_equal(y.astype(np.float64), pruned[:, c].astype(np.float64)), c
    yd = down_f16(nm.nm_gemv_dense(up_f16(W), up_f16(np.eye(1, C, 5, dtype=np.float16)[0])))
    assert np.array_equal(yd.astype(np.float64), W[:, 5].astype(np.float64))


@pytest.mark.parametrize("N,M", PATTERNS)
def test_sign_and_power_of_two_symmetry(N, M):
    R, C = 64, 2048
    W = synth.weight(R, C, seed=710)
    x = synth.activation(C, seed=711)
    x[np.abs(x.astype(np.float32)) < 2.0 ** -12] = 0  # so that x * 2^k stays exact in fp16
    values, masks = nm.nm_pack(up_f16(W), N, M)
    y = down_f16(nm.nm_spmv(values, masks, up_f16(x), N, M)).astype(np.float64)
    yn = down_f16(nm.nm_spmv(values, masks, up_f16(-x), N, M)).astype(np.float64)
    assert np.array_equal(yn, -y)
    for k in (1, -1, 3):
        ys = down_f16(nm.nm_spmv(values, masks, up_f16((x.astype(np.float32) * 2.0 ** k).astype(np.float16)),
                                 N, M)).astype(np.float64)
        ok = np.abs(y) > 2.0 ** -10  # away from fp16 subnormals after scaling
        assert np.array_equal(ys[ok], y[ok] * 2.0 ** k), k


@pytest.mark.parametrize("N,M", PATTERNS)
def test_deterministic(N, M):
    W = synth.weight(1000, 4096, seed=720)
    x = up_f16(synth.activation(4096, seed=721))
    values, masks = nm.nm_pack(up_f16(W), N, M)
    first = nm.nm_spmv(values, masks, x, N, M).clone()
    out = torch.empty_like(first)
    for _ in range(100):
        nm.nm_spmv(values, masks, x, N, M, out=out)
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    W_d = up_f16(W)
    d0 = nm.nm_gemv_dense(W_d, x).clone()
    for _ in range(20):
        assert torch.equal(nm.nm_gemv_dense(W_d, x).view(torch.int16), d0.view(torch.int16))


@pytest.mark.parametrize("N,M", PATTERNS)
def test_unit_sum_closed_form(N, M):
    C = 4096
    W = np.full((50, C), 2.0 ** -6, np.float16)
    values, masks = nm.nm_pack(up_f16(W), N, M)
    y = down_f16(nm.nm_spmv(values, masks, up_f16(np.ones(C, np.float16)), N, M))
    assert np.all(y == 32.0)
    assert np.all(down_u32(masks) == {2: 0x33333333, 4: 0x0F0F0F0F, 8: 0x00FF00FF, 16: 0x0000FFFF}[N])


@pytest.mark.parametrize("N,M", PATTERNS)
def test_whole_byte_halves(N, M):
    """Groups whose kept values all sit in one byte of a mask half-word: magnitudes rising or
    falling across each group of M, chosen at random per group, so that 8:16 half-words read
    0xFF/0x00 and 0x00/0xFF (the byte-table decoder's shift of 64 and of 0) in every mix."""
    R, C = 64, 4096
    rng = np.random.default_rng(4242)
    ramp = (np.arange(1, M + 1, dtype=np.float32) / M) * 0.05
    W = np.empty((R, C), np.float32)
    for g in range(C // M):
        rise = rng.integers(0, 2, size=R).astype(bool)
        mags = np.where(rise[:, None], ramp[None, :], ramp[None, ::-1])
        W[:, g * M:(g + 1) * M] = mags * rng.choice([-1.0, 1.0], size=(R, M))
    W = W.astype(np.float16)
    x = synth.activation(C, seed=4243)
    values, masks = nm.nm_pack(up_f16(W), N, M)
    rv, rm = oracle.pack_ref(W, N, M)
    assert np.array_equal(down_bits16(values), rv) and np.array_equal(down_u32(masks), rm)
    if N == 8:
        halves = np.concatenate([rm & 0xFFFF, rm >> 16]).ravel()
        assert {0x00FF, 0xFF00} <= set(halves.tolist())
    y = down_f16(nm.nm_spmv(values, masks, up_f16(x), N, M))
    rep = oracle.y_tolerance_report(y, oracle.spmv_ref(rv, rm, x, C, N, M))
    assert rep["ok"], rep


def test_cross_path_sparse_vs_dense_of_pruned():
    R, C = 300, 4096
    W = synth.weight(R, C, seed=730)
    x = synth.activation(C, seed=731)
    for N, M in PATTERNS:
        values, masks = nm.nm_pack(up_f16(W), N, M)
        ys = down_f16(nm.nm_spmv(values, masks, up_f16(x), N, M))
        pruned = oracle.prune_ref(W, N, M).view(np.float16)
        yd = down_f16(nm.nm_gemv_dense(up_f16(pruned), up_f16(x)))
        ref = oracle.gemv_ref(pruned, x)
        assert oracle.y_tolerance_report(ys, ref)["ok"]
        assert oracle.y_tolerance_report(yd, ref)["ok"]


def test_edge_shapes_and_errors():
    mc = nm.max_cols()
    # widest x the kernel stages (every pattern falls back to the plain bit walk there),
    # a single row and a ragged row count
    for R, C in ((1, 32), (3, mc), (17, 32)):
        W = synth.weight(R, C, seed=740)
        x = synth.activation(C, seed=741)
        for N, M in PATTERNS:
            rv, rm = oracle.pack_ref(W, N, M)
            y = nm.nm_spmv(up_f16(rv), up_u32(rm), up_f16(x), N, M)
            assert oracle.y_tolerance_report(down_f16(y), oracle.spmv_ref(rv, rm, x, C, N, M))["ok"], (R, C)
        yd = nm.nm_gemv_dense(up_f16(W), up_f16(x))
        assert oracle.y_tolerance_report(down_f16(yd), oracle.gemv_ref(W, x))["ok"], (R, C)
    # too wide: rejected on the host before any launch
    wide = mc + 32
    v = torch.zeros((1, wide // 2), dtype=torch.float16, device=device())
    m = torch.zeros((1, wide // 32), dtype=torch.int32, device=device())
    xw = torch.zeros(wide, dtype=torch.float16, device=device())
    with pytest.raises(nm.NMArgumentError) as e:
        nm.nm_spmv(v, m, xw, 2, 4)
    assert e.value.status == nm.NM_ERR_TOO_WIDE
    with pytest.raises(nm.NMArgumentError):
        nm.nm_gemv_dense(torch.zeros((1, wide), dtype=torch.float16, device=device()), xw)
    # empty input: no rows is an invalid shape
    with pytest.raises(nm.NMArgumentError) as e:
        nm.nm_pack(torch.zeros((0, 64), dtype=torch.float16, device=device()), 2, 4)
    assert e.value.status == nm.NM_ERR_SHAPE
    with pytest.raises(nm.NMArgumentError):
        nm.nm_spmv(torch.zeros((0, 32), dtype=torch.float16, device=device()),
                   torch.zeros((0, 2), dtype=torch.int32, device=device()),
                   torch.zeros(64, dtype=torch.float16, device=device()), 2, 4)


def test_malformed_masks_stay_in_bounds():
    """Masks with too few set bits give an unspecified y but run to completion: every LDS
    read stays inside the word's x window by construction (bit 31 sentinel)."""
    for R, C in ((64, 1024), (64, 4096)):   # 64 x 4096: the narrow kernel for 16:32
        v = up_f16(synth.weight(R, C // 2, seed=750))
        x = up_f16(synth.activation(C, seed=751))
        for N, M in PATTERNS:
            for word in (0, 1, 0x80000000, 0xFFFFFFFF):
                m = torch.full((R, C // 32), np.uint32(word).view(np.int32).item(), dtype=torch.int32,
                               device=device())
                y = nm.nm_spmv(v, m, x, N, M)
                torch.cuda.synchronize()
                assert y.shape == (R,)


def test_non_default_stream():
    W = synth.weight(512, 4096, seed=760)
    x = synth.activation(4096, seed=761)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        values, masks = nm.nm_pack(up_f16(W), 2, 4)
        y = nm.nm_spmv(values, masks, up_f16(x), 2, 4)
    s.synchronize()
    rv, rm = oracle.pack_ref(W, 2, 4)
    assert oracle.y_tolerance_report(down_f16(y), oracle.spmv_ref(rv, rm, x, 4096, 2, 4))["ok"]


def _full_size_cases():
    cases = []
    for cfg in (2, 3, 4):
        wl = synth.WORKLOADS[cfg]
        for li, (name, R, C) in enumerate(wl["layers"]):
            for pat in wl["patterns"]:
                cases.append(pytest.param(cfg, li, name, R, C, pat, id=f"cfg{cfg}-{name}-{R}x{C}-{pat[0]}:{pat[1]}"))
    return cases


@pytest.mark.slow
@pytest.mark.parametrize("cfg,li,name,R,C,pat", _full_size_cases())
def test_full_size_layer(cfg, li, name, R, C, pat):
    """Every layer shape and pattern of the Llama-3.1-8B, Qwen3-14B/32B and Llama-3.3-70B
    projection workloads at full size, in the launch configuration the bench times:
    pack bit-exact and y within tolerance on sampled rows (the oracle computes them one
    by one)."""
    N, M = pat
    say(f"full-size cfg{cfg} {name} {R}x{C} {N}:{M}")
    W = synth.weight(R, C, synth.weight_seed(cfg, li, pat))
    x = synth.activation(C, synth.x_seed(cfg, li, pat))
    rep = check_full_layer(W, x, N, M, f"cfg{cfg}-{name}", check_dense=(pat == wl_first_pattern(cfg)))
    say(f"  {rep}")


def wl_first_pattern(cfg):
    return tuple(synth.WORKLOADS[cfg]["patterns"][0])


@pytest.mark.slow
@pytest.mark.parametrize("block", [0, 31])
def test_decode_sweep_blocks(block):
    """Two of the 32 transformer blocks of the Llama-3.1-8B decode sweep, every projection at
    full size with its own seeds (the other 30 blocks repeat these shapes)."""
    for p, (name, R, C) in enumerate(synth.LLAMA31_8B_DECODE_LAYER):
        say(f"decode block {block} {name} {R}x{C}")
        W = synth.weight(R, C, synth.decode_seed(block, p))
        x = synth.activation(C, synth.decode_x_seed(block, p))
        check_full_layer(W, x, 2, 4, f"decode-{block}-{name}", check_dense=(p in (0, 4)))


@pytest.mark.slow
@pytest.mark.parametrize("parts,name", [((0, 1, 2), "qkv"), ((4, 5), "gate_up")])
def test_decode_fused_products(parts, name):
    """The fused products the decode benchmark times: q/k/v (6144 x 4096) and gate/up
    (28672 x 4096) of block 0, each part packed alone and the packed rows concatenated, all
    parts applied to the x of the first: pack bit-exact per part and y within tolerance on
    sampled rows of the fused product, in its own launch configuration."""
    shapes = [synth.LLAMA31_8B_DECODE_LAYER[p] for p in parts]
    C = shapes[0][2]
    Ws = [synth.weight(R, C, synth.decode_seed(0, p)) for p, (_, R, _) in zip(parts, shapes)]
    x = synth.activation(C, synth.decode_x_seed(0, parts[0]))
    packed = [nm.nm_pack(up_f16(W), 2, 4) for W in Ws]
    values = torch.cat([v for v, _ in packed])
    masks = torch.cat([m for _, m in packed])
    R = values.shape[0]
    say(f"decode fused {name} {R}x{C} rpb={nm.spmv_launch_shape(R, C, 2, 4)['rows_per_workgroup']}")
    y = down_f16(nm.nm_spmv(values, masks, up_f16(x), 2, 4))
    Wcat = np.concatenate(Ws)
    idx = sample_rows(R, k=64, rpb=nm.spmv_launch_shape(R, C, 2, 4)["rows_per_workgroup"])
    # the part boundaries and their neighbours too
    edges = np.cumsum([W.shape[0] for W in Ws])[:-1]
    idx = np.unique(np.concatenate([idx, edges - 1, edges]))
    it = torch.from_numpy(idx).to(device())
    rv, rm = oracle.pack_ref(Wcat[idx], 2, 4)
    assert np.array_equal(down_u32(masks.index_select(0, it)), rm)
    assert np.array_equal(down_bits16(values.index_select(0, it)), rv)
    rep = oracle.y_tolerance_report(y[idx], oracle.spmv_ref(rv, rm, x, C, 2, 4))
    assert rep["ok"], (name, rep)
