"""CPU tests: the oracle against facts other than itself (no GPU needed)."""
import numpy as np
import pytest

import oracle
import synth
from tests import oracle_pins as pins


def test_worked_example_golden():
    pins.check_worked_example(oracle.pack_ref, oracle.spmv_ref)


def test_selection_matches_textbook_sort():
    pins.check_selection_textbook(oracle.keep_ref)


def test_canonical_masks_closed_form():
    pins.check_canonical_masks(oracle.pack_ref)


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_invariants(kind):
    if kind == "normal":
        W = synth.weight(9, 160, seed=77)
    else:
        W = synth.tie_heavy_weight(9, 160, seed=78)
    pins.check_invariants(oracle.pack_ref, oracle.unpack_ref, oracle.prune_ref, W)


def test_cross_pattern_identity():
    pins.check_cross_pattern(oracle.pack_ref)


def test_spmv_brute_force():
    pins.check_spmv_bruteforce(oracle.pack_ref, oracle.spmv_ref)


def test_gemv_brute_force():
    pins.check_gemv_bruteforce(oracle.gemv_ref)


def test_exact_ref_closed_forms():
    pins.check_exact_ref(oracle.exact_ref)


def test_exact_ref_matches_brute_force():
    rng = np.random.default_rng(4)
    W = rng.standard_normal((4, 64)).astype(np.float16)
    x = rng.standard_normal(64).astype(np.float16)
    assert oracle.exact_ref(W, x) == pins.brute_force_y(W, x)


def test_unit_sum_closed_form():
    pins.check_unit_sum(oracle.pack_ref, oracle.spmv_ref)


def test_one_hot_x_selects_column():
    """x = e_c gives column c of the pruned matrix exactly."""
    W = synth.weight(6, 64, seed=12)
    for n, m in pins.PATTERNS:
        v, mk = oracle.pack_ref(W, n, m)
        pruned = oracle.prune_ref(W, n, m).view(np.float16)
        for c in (0, 17, 63):
            x = np.zeros(64, np.float16)
            x[c] = 1
            y = oracle.spmv_ref(v, mk, x, 64, n, m)
            assert np.array_equal(y, pruned[:, c].astype(np.float64))


def test_unpack_rejects_malformed_masks():
    v = np.zeros((1, 16), np.uint16)
    with pytest.raises(ValueError):
        oracle.unpack_ref(v, np.array([[0x7]], np.uint32), 32, 2, 4)


def test_dropped_entries_unpack_to_plus_zero():
    W = np.full((1, 32), -1.0, np.float16)
    v, mk = oracle.pack_ref(W, 2, 4)
    d = oracle.unpack_ref(v, mk, 32, 2, 4)
    assert np.all((d == 0) | (d == np.float16(-1.0).view(np.uint16)))
    assert np.count_nonzero(d == 0) == 16


def test_tolerance_discriminates_fp16_accumulation():
    """The y tolerance rejects fp16 accumulation and accepts fp32 accumulation at a
    realistic size (4096 columns, N(0, 0.02) weights, N(0, 1) x)."""
    W = synth.weight(64, 4096, seed=21)
    x = synth.activation(4096, seed=22)
    v, mk = oracle.pack_ref(W, 2, 4)
    ref = oracle.spmv_ref(v, mk, x, 4096, 2, 4)
    Wp = oracle.prune_ref(W, 2, 4).view(np.float16)
    acc32 = np.zeros(64, np.float32)
    acc16 = np.zeros(64, np.float16)
    for c in range(4096):
        prod = Wp[:, c].astype(np.float32) * np.float32(x[c])
        acc32 += prod
        acc16 = (acc16.astype(np.float32) + prod).astype(np.float16)
    assert oracle.y_within_tolerance(acc32.astype(np.float16), ref)
    assert not oracle.y_within_tolerance(acc16, ref)


def test_tolerance_flags_nonfinite_and_shape():
    ref = np.ones(4)
    assert not oracle.y_within_tolerance(np.array([1, 1, np.nan, 1]), ref)
    with pytest.raises(ValueError):
        oracle.y_tolerance_report(np.ones(3), ref)


def test_spmm_worked_example_golden():
    pins.check_spmm_worked_example(oracle.pack_ref, oracle.spmm_ref)


def test_spmm_brute_force():
    pins.check_spmm_bruteforce(oracle.pack_ref, oracle.spmm_ref)


def test_spmm_exact_linearity_and_permutation():
    pins.check_spmm_exact_linearity(oracle.pack_ref, oracle.spmm_ref)


def test_gemm_brute_force():
    pins.check_gemm_bruteforce(oracle.gemm_ref)


# ---------------------------------------------------------------- 25% density (8 values per word)
def test_quarter_worked_example_golden():
    pins.check_worked_example(oracle.pack_ref, oracle.spmv_ref, name="worked_row32_quarter.txt")


def test_quarter_selection_matches_textbook_sort():
    pins.check_selection_textbook(oracle.keep_ref, patterns=pins.PATTERNS_QUARTER)


def test_quarter_canonical_masks_closed_form():
    pins.check_canonical_masks(oracle.pack_ref, patterns=pins.PATTERNS_QUARTER)


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_quarter_invariants(kind):
    W = synth.weight(6, 128, seed=31) if kind == "normal" else synth.tie_heavy_weight(6, 128, seed=32)
    pins.check_invariants(oracle.pack_ref, oracle.unpack_ref, oracle.prune_ref, W, patterns=pins.PATTERNS_QUARTER)


def test_quarter_spmv_brute_force():
    pins.check_spmv_bruteforce(oracle.pack_ref, oracle.spmv_ref, patterns=pins.PATTERNS_QUARTER)
