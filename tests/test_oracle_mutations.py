"""CPU tests: plausible mistakes planted in copies of the oracle are caught by the pins.

Every mutant below is a small, realistic slip (a flipped tie rule, a reversed bit
order, a transposed operand, a dropped term, an off-by-one offset). Each must make at
least one pin of tests/oracle_pins.py fail; the real oracle passes all of them.
"""
import numpy as np
import pytest

import oracle
from oracle import nm_oracle as O
from tests import oracle_pins as pins


# ---------------------------------------------------------------- mutants
def keep_ties_high(W, N, M):
    bits = O._as_bits(W)
    R, C = bits.shape
    key = O.magnitude_key(bits).reshape(R, C // M, M)
    ki, kk = key[..., :, None], key[..., None, :]
    col = np.arange(M)
    higher = col[None, :] > col[:, None]
    rank = (kk > ki).sum(-1) + ((kk == ki) & higher).sum(-1)
    return (rank < N).reshape(R, C)


def keep_smallest(W, N, M):
    bits = O._as_bits(W)
    R, C = bits.shape
    key = O.magnitude_key(bits).reshape(R, C // M, M)
    ki, kk = key[..., :, None], key[..., None, :]
    col = np.arange(M)
    lower = col[None, :] < col[:, None]
    rank = (kk < ki).sum(-1) + ((kk == ki) & lower).sum(-1)
    return (rank < N).reshape(R, C)


def keep_signed(W, N, M):
    """Compares signed values instead of magnitudes."""
    f = O._as_bits(W).view(np.float16).astype(np.float64)
    R, C = f.shape
    key = f.reshape(R, C // M, M)
    ki, kk = key[..., :, None], key[..., None, :]
    col = np.arange(M)
    lower = col[None, :] < col[:, None]
    rank = (kk > ki).sum(-1) + ((kk == ki) & lower).sum(-1)
    return (rank < N).reshape(R, C)


def make_pack(keep_fn=O.keep_ref, reverse_bits=False, reverse_values=False):
    def pack(W, N, M):
        bits = O._as_bits(W)
        R, C = bits.shape
        kept = keep_fn(bits, N, M)
        pos = np.arange(32, dtype=np.uint64)
        if reverse_bits:
            pos = 31 - pos
        masks = (kept.reshape(R, C // 32, 32).astype(np.uint64) << pos).sum(-1).astype(np.uint32)
        vals = bits[kept].reshape(R, C // 32, 32 * N // M)
        if reverse_values:
            vals = vals[..., ::-1]
        return vals.reshape(R, C * N // M).astype(np.uint16), masks
    return pack


def make_prune(keep_fn):
    def prune(W, N, M):
        bits = O._as_bits(W)
        return np.where(keep_fn(bits, N, M), bits, np.uint16(0)).astype(np.uint16)
    return prune


def unpack_off_by_one(values, masks, cols, N, M):
    """Uses an inclusive prefix count for the value index (skips each word's first value)."""
    masks = np.asarray(masks, np.uint32)
    values = np.asarray(values).view(np.uint16)
    R, nw = masks.shape
    pw = 32 * N // M
    bit = ((masks[..., None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.int64)
    idx = np.minimum(np.cumsum(bit, -1), pw - 1)
    g = np.take_along_axis(values.reshape(R, nw, pw), idx, -1)
    return np.where(bit.astype(bool), g, 0).reshape(R, cols).astype(np.uint16)


def spmv_x_reversed(values, masks, x, cols, N, M):
    D = O.unpack_ref(values, masks, cols, N, M).view(np.float16).astype(np.float64)
    return D @ np.asarray(x, np.float16)[::-1].astype(np.float64)


def spmv_drop_last_word(values, masks, x, cols, N, M):
    D = O.unpack_ref(values, masks, cols, N, M).view(np.float16).astype(np.float64)
    D[:, -32:] = 0
    return D @ np.asarray(x, np.float16).astype(np.float64)


def spmv_fp32_sum(values, masks, x, cols, N, M):
    """Accumulates in fp32 instead of fp64 (precision slip)."""
    D = O.unpack_ref(values, masks, cols, N, M).view(np.float16).astype(np.float32)
    return (D @ np.asarray(x, np.float16).astype(np.float32)).astype(np.float64)


def gemv_transposed(W, x):
    Wd = O._as_bits(W).view(np.float16).astype(np.float64)
    C = Wd.shape[1]
    xd = np.asarray(x, np.float16).astype(np.float64)
    # uses the transpose of the leading square block: a classic operand slip
    out = np.zeros(Wd.shape[0])
    for r in range(Wd.shape[0]):
        for c in range(C):
            out[r] += Wd[c % Wd.shape[0], r % C] * xd[c]
    return out


def exact_drop_scale(W, x):
    res = O.exact_ref(W, x)
    return [v * 2 ** 24 for v in res]


def spmm_transposed(values, masks, X, cols, N, M):
    """Returns [rows, B] instead of [B, rows]."""
    return O.spmm_ref(values, masks, X, cols, N, M).T


def spmm_batch_reversed(values, masks, X, cols, N, M):
    return O.spmm_ref(values, masks, np.asarray(X)[::-1], cols, N, M)


def spmm_first_row_only(values, masks, X, cols, N, M):
    """Applies the first activation vector to every batch row."""
    X = np.asarray(X)
    return O.spmm_ref(values, masks, np.repeat(X[:1], X.shape[0], axis=0), cols, N, M)


def spmm_fp32_sum(values, masks, X, cols, N, M):
    D = O.unpack_ref(values, masks, cols, N, M).view(np.float16).astype(np.float32)
    return (np.asarray(X, np.float16).astype(np.float32) @ D.T).astype(np.float64)


def spmm_unpruned_order(values, masks, X, cols, N, M):
    """Multiplies the packed values by the first cols/2 entries of x (ignores the masks)."""
    V = np.asarray(values).view(np.float16).astype(np.float64)
    Xf = np.asarray(X, np.float16).astype(np.float64)
    return Xf[:, :V.shape[1]] @ V.T


def gemm_transposed_operand(W, X):
    Wd = O._as_bits(W).view(np.float16).astype(np.float64)
    Xf = np.asarray(X, np.float16).astype(np.float64)
    return (Wd @ Xf.T).T[:, ::-1]


def _spmm_pin_fails(spmm):
    checks = [lambda: pins.check_spmm_worked_example(O.pack_ref, spmm),
              lambda: pins.check_spmm_bruteforce(O.pack_ref, spmm),
              lambda: pins.check_spmm_exact_linearity(O.pack_ref, spmm)]
    return any(_fails(c) for c in checks)


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError):
        return True
    return False


def _any_pin_fails(keep=O.keep_ref, pack=O.pack_ref, unpack=O.unpack_ref, prune=O.prune_ref,
                   spmv=O.spmv_ref):
    W = __import__("synth").weight(5, 96, seed=90)
    checks = [
        lambda: pins.check_worked_example(pack, spmv),
        lambda: pins.check_selection_textbook(keep),
        lambda: pins.check_canonical_masks(pack),
        lambda: pins.check_invariants(pack, unpack, prune, W),
        lambda: pins.check_cross_pattern(pack),
        lambda: pins.check_spmv_bruteforce(pack, spmv),
        lambda: pins.check_unit_sum(pack, spmv),
    ]
    return any(_fails(c) for c in checks)


def test_real_oracle_passes_every_pin():
    assert not _any_pin_fails()


@pytest.mark.parametrize("name,kw", [
    ("ties_to_higher_column", dict(keep=keep_ties_high, pack=make_pack(keep_ties_high),
                                   prune=make_prune(keep_ties_high))),
    ("keeps_smallest", dict(keep=keep_smallest, pack=make_pack(keep_smallest),
                            prune=make_prune(keep_smallest))),
    ("signed_not_magnitude", dict(keep=keep_signed, pack=make_pack(keep_signed),
                                  prune=make_prune(keep_signed))),
    ("mask_bits_reversed", dict(pack=make_pack(reverse_bits=True))),
    ("values_descending_in_word", dict(pack=make_pack(reverse_values=True))),
    ("unpack_off_by_one", dict(unpack=unpack_off_by_one)),
    ("x_reversed", dict(spmv=spmv_x_reversed)),
    ("last_word_dropped", dict(spmv=spmv_drop_last_word)),
    ("fp32_accumulation", dict(spmv=spmv_fp32_sum)),
])
def test_mutant_is_caught(name, kw):
    assert _any_pin_fails(**kw), name


def test_gemv_mutant_is_caught():
    assert _fails(pins.check_gemv_bruteforce, gemv_transposed)
    assert not _fails(pins.check_gemv_bruteforce, oracle.gemv_ref)


def test_exact_mutant_is_caught():
    assert _fails(pins.check_exact_ref, exact_drop_scale)


@pytest.mark.parametrize("mutant", [spmm_transposed, spmm_batch_reversed, spmm_first_row_only,
                                    spmm_fp32_sum, spmm_unpruned_order])
def test_spmm_mutant_is_caught(mutant):
    assert _spmm_pin_fails(mutant), mutant.__name__
    assert not _spmm_pin_fails(O.spmm_ref)


def test_gemm_mutant_is_caught():
    assert _fails(pins.check_gemm_bruteforce, gemm_transposed_operand)
    assert not _fails(pins.check_gemm_bruteforce, oracle.gemm_ref)


@pytest.mark.parametrize("name,kw", [
    ("ties_to_higher_column", dict(keep=keep_ties_high, pack=make_pack(keep_ties_high))),
    ("keeps_smallest", dict(keep=keep_smallest, pack=make_pack(keep_smallest))),
    ("mask_bits_reversed", dict(pack=make_pack(reverse_bits=True))),
    ("values_descending_in_word", dict(pack=make_pack(reverse_values=True))),
    ("x_reversed", dict(spmv=spmv_x_reversed)),
])
def test_quarter_mutant_is_caught(name, kw):
    """The same slips are caught by the pins of the 25% patterns (8 values per word)."""
    keep, pack, spmv = kw.get("keep", O.keep_ref), kw.get("pack", O.pack_ref), kw.get("spmv", O.spmv_ref)
    Q = pins.PATTERNS_QUARTER
    checks = [lambda: pins.check_worked_example(pack, spmv, name="worked_row32_quarter.txt"),
              lambda: pins.check_selection_textbook(keep, patterns=Q),
              lambda: pins.check_canonical_masks(pack, patterns=Q),
              lambda: pins.check_spmv_bruteforce(pack, spmv, patterns=Q)]
    assert any(_fails(c) for c in checks), name
    real = [lambda: pins.check_worked_example(O.pack_ref, O.spmv_ref, name="worked_row32_quarter.txt"),
            lambda: pins.check_selection_textbook(O.keep_ref, patterns=Q),
            lambda: pins.check_canonical_masks(O.pack_ref, patterns=Q),
            lambda: pins.check_spmv_bruteforce(O.pack_ref, O.spmv_ref, patterns=Q)]
    assert not any(_fails(c) for c in real)
