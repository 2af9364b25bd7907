"""Checks that pin the CPU oracle to facts other than itself.

Each check takes the oracle functions it exercises as arguments, so the same
check can be run against the real oracle (tests/test_oracle_pins.py) and
against deliberately broken copies of it (tests/test_oracle_mutations.py),
which shows that a plausible mistake in the oracle does not go unnoticed.

Sources of the facts (pages cited by title and section):
  news.bitwarelabs.com "SparseDecoding: decoding-aware pruning for accurate and
  fast LLM generation", "What's new": N of every M consecutive weights kept.
  aimodeling.com SparseDecoding article, "The Kernel Is the Other Half of the
  Answer": a 32-bit mask word per 32 columns, exactly 16 set bits at 50%.
  The small-batch product (B activation vectors against one packed matrix) is the
  matrix-matrix side of the SpMV / SpMM split the first page draws ("What's new").
"""
from __future__ import annotations

import itertools
import os
from fractions import Fraction

import numpy as np

PATTERNS = ((2, 4), (4, 8), (8, 16), (16, 32))
PATTERNS_QUARTER = ((1, 4), (2, 8), (4, 16), (8, 32))   # 8 kept values per mask word
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# independent restatements used only as pins
# ----------------------------------------------------------------------------
def textbook_keep_group(keys, N):
    """Kept positions of one group: sort by (magnitude desc, column asc), take N."""
    order = sorted(range(len(keys)), key=lambda c: (-int(keys[c]), c))
    return set(order[:N])


def textbook_prune_dense(W16, N, M):
    """Pruned dense fp16 matrix built with the sort-based textbook rule."""
    bits = W16.view(np.uint16)
    out = bits.copy()
    R, C = bits.shape
    for r in range(R):
        for g in range(C // M):
            keys = [int(b) & 0x7FFF for b in bits[r, g * M:(g + 1) * M]]
            keep = textbook_keep_group(keys, N)
            for c in range(M):
                if c not in keep:
                    out[r, g * M + c] = 0
    return out.view(np.float16)


def brute_force_y(Wd16, x16):
    """Exact y of a dense fp16 matrix, written independently of the oracle (nested loops
    over Fractions built from float64, which holds every fp16 exactly)."""
    Wf = Wd16.astype(np.float64)
    xf = x16.astype(np.float64)
    out = []
    for r in range(Wf.shape[0]):
        acc = Fraction(0)
        for c in range(Wf.shape[1]):
            acc += Fraction(float(Wf[r, c])) * Fraction(float(xf[c]))
        out.append(acc)
    return out


def parse_token(tok):
    if tok == "-0":
        return np.float16(-0.0)
    if tok.startswith("2^"):
        return np.float16(2.0 ** int(tok[2:]))
    return np.float16(float(tok))


def load_worked_row(name="worked_row32.txt", ncases=4):
    """Parse a golden worked-row file under tests/golden/."""
    row = x = None
    cases = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            t = line.split()
            if t[0] == "row":
                row = np.array([parse_token(v) for v in t[1:]], dtype=np.float16)
            elif t[0] == "x":
                assert t[1] == "c/8"
                x = (np.arange(32) / 8.0).astype(np.float16)
            elif t[0] == "case":
                n, m = (int(v) for v in t[1].split(":"))
                assert t[2] == "mask"
                mask = int(t[3], 16)
                vi = t.index("values")
                yi = t.index("y")
                vals = np.array([parse_token(v) for v in t[vi + 1:yi]], dtype=np.float16)
                y = Fraction(t[yi + 1]) + int(t[yi + 2]) * Fraction(2) ** int(t[yi + 3])
                cases.append((n, m, mask, vals, y))
    assert row is not None and x is not None and len(row) == 32 and len(cases) == ncases
    return row, x, cases


# ----------------------------------------------------------------------------
# checks
# ----------------------------------------------------------------------------
def check_worked_example(pack_fn, spmv_fn, name="worked_row32.txt"):
    """Hand-worked golden row: masks, value bits and exact y (rounded to fp64)."""
    row, x, cases = load_worked_row(name)
    W = row.reshape(1, 32)
    for n, m, mask, vals, y in cases:
        values, masks = pack_fn(W, n, m)
        assert int(masks[0, 0]) == mask, f"{n}:{m} mask {int(masks[0, 0]):#010x} != {mask:#010x}"
        assert np.array_equal(np.asarray(values).view(np.uint16)[0], vals.view(np.uint16)), \
            f"{n}:{m} values differ"
        got = spmv_fn(values, masks, x, 32, n, m)
        assert float(got[0]) == float(y), f"{n}:{m} y {got[0]!r} != {float(y)!r}"


def check_selection_textbook(keep_fn, seed=1, patterns=PATTERNS):
    """keep_fn agrees with the sort-based rule on random groups and on every tie pattern
    of M=4 over a 3-value alphabet (with random signs, including -0)."""
    rng = np.random.default_rng(seed)
    # exhaustive M=4 tie patterns: all 4-tuples over magnitudes {0, 1.0, 2.0}, signs random
    mags = np.array([0.0, 1.0, 2.0], dtype=np.float16)
    tuples = np.array(list(itertools.product(range(3), repeat=4)))
    groups = mags[tuples]  # 81 groups of 4
    signs = rng.integers(0, 2, size=groups.shape).astype(bool)
    groups = np.where(signs, -groups, groups).astype(np.float16)
    flat = groups.reshape(-1)
    pad = (-len(flat)) % 32
    flat = np.concatenate([flat, np.zeros(pad, np.float16)])
    W = flat.reshape(-1, 32)
    for n, m in patterns:
        kept = keep_fn(W, n, m)
        bits = W.view(np.uint16)
        for r in range(W.shape[0]):
            for g in range(32 // m):
                keys = [int(b) & 0x7FFF for b in bits[r, g * m:(g + 1) * m]]
                want = textbook_keep_group(keys, n)
                got = {c for c in range(m) if kept[r, g * m + c]}
                assert got == want, (n, m, keys, got, want)
    # random groups with a small alphabet (many ties) and with continuous values
    for trial in range(2):
        if trial == 0:
            W = rng.choice(np.array([0, 0.5, -0.5, 1, -1, 2, 2 ** -24], np.float16), size=(6, 64))
        else:
            W = (rng.standard_normal((6, 64)) * 0.02).astype(np.float16)
        W = W.astype(np.float16)
        for n, m in patterns:
            kept = keep_fn(W, n, m)
            bits = W.view(np.uint16)
            for r in range(W.shape[0]):
                for g in range(64 // m):
                    keys = [int(b) & 0x7FFF for b in bits[r, g * m:(g + 1) * m]]
                    want = textbook_keep_group(keys, n)
                    got = {c for c in range(m) if kept[r, g * m + c]}
                    assert got == want, (n, m, keys, got, want)


CANON_LOW = {(2, 4): 0x33333333, (4, 8): 0x0F0F0F0F, (8, 16): 0x00FF00FF, (16, 32): 0x0000FFFF,
             (1, 4): 0x11111111, (2, 8): 0x03030303, (4, 16): 0x000F000F, (8, 32): 0x000000FF}
CANON_HIGH = {(2, 4): 0xCCCCCCCC, (4, 8): 0xF0F0F0F0, (8, 16): 0xFF00FF00, (16, 32): 0xFFFF0000,
              (1, 4): 0x88888888, (2, 8): 0xC0C0C0C0, (4, 16): 0xF000F000, (8, 32): 0xFF000000}


def check_canonical_masks(pack_fn, patterns=PATTERNS):
    """Closed forms: equal magnitudes (any signs) or strictly decreasing magnitudes keep
    the N lowest columns of each group; strictly increasing ones keep the N highest."""
    rng = np.random.default_rng(3)
    for (n, m) in patterns:
        eq = np.full((3, 64), 0.75, np.float16)
        eq = np.where(rng.integers(0, 2, eq.shape).astype(bool), -eq, eq).astype(np.float16)
        _, masks = pack_fn(eq, n, m)
        assert np.all(masks == CANON_LOW[(n, m)]), (n, m, hex(int(masks[0, 0])))
        ramp_in_group = np.arange(64) % m
        dec = (1.0 + (m - ramp_in_group)).astype(np.float16)[None, :].repeat(2, 0)
        dec[1] = -dec[1]
        _, masks = pack_fn(dec, n, m)
        assert np.all(masks == CANON_LOW[(n, m)]), (n, m, "decreasing")
        inc = (1.0 + ramp_in_group).astype(np.float16)[None, :].repeat(2, 0)
        _, masks = pack_fn(inc, n, m)
        assert np.all(masks == CANON_HIGH[(n, m)]), (n, m, "increasing")


def check_invariants(pack_fn, unpack_fn, prune_fn, W, patterns=PATTERNS):
    """Structural invariants of one packed matrix, for every pattern."""
    bits = W.view(np.uint16)
    R, C = W.shape
    for n, m in patterns:
        values, masks = pack_fn(W, n, m)
        values = np.asarray(values).view(np.uint16)
        assert values.shape == (R, C * n // m) and masks.shape == (R, C // 32)
        # 32*N/M set bits per word, N per M-bit field
        pc = np.array([[bin(int(w)).count("1") for w in row] for row in masks])
        assert np.all(pc == 32 * n // m)
        for f in range(32 // m):
            field = (masks.astype(np.uint64) >> np.uint64(f * m)) & np.uint64((1 << m) - 1)
            assert np.all(np.vectorize(lambda v: bin(int(v)).count("1"))(field) == n)
        # kept magnitudes dominate dropped ones in every group
        kept = ((masks[..., None] >> np.arange(32, dtype=np.uint32)) & 1).astype(bool).reshape(R, C)
        key = (bits & 0x7FFF).astype(np.int64).reshape(R, C // m, m)
        kk = kept.reshape(R, C // m, m)
        min_kept = np.where(kk, key, 1 << 20).min(-1)
        max_drop = np.where(~kk, key, -1).max(-1)
        assert np.all(min_kept >= max_drop)
        # round trip and idempotence
        dense = unpack_fn(values, masks, C, n, m)
        assert np.array_equal(dense, prune_fn(W, n, m))
        v2, m2 = pack_fn(np.asarray(dense).view(np.float16), n, m)
        assert np.array_equal(np.asarray(v2).view(np.uint16), values) and np.array_equal(m2, masks)


def check_cross_pattern(pack_fn):
    """A matrix that is already 2:4 with nonzero kept values encodes identically under every
    pattern (each group of M holds exactly M/2 nonzeros, and they win the selection)."""
    rng = np.random.default_rng(11)
    R, C = 5, 96
    W = (rng.standard_normal((R, C)) * 0.02).astype(np.float16)
    W[W == 0] = np.float16(0.001)
    for r in range(R):
        for g in range(C // 4):
            drop = rng.choice(4, size=2, replace=False)
            W[r, g * 4 + drop] = 0
    ref_v, ref_m = pack_fn(W, 2, 4)
    for n, m in PATTERNS[1:]:
        v, mk = pack_fn(W, n, m)
        assert np.array_equal(np.asarray(v).view(np.uint16), np.asarray(ref_v).view(np.uint16))
        assert np.array_equal(mk, ref_m)


def check_spmv_bruteforce(pack_fn, spmv_fn, seed=5, patterns=PATTERNS):
    """spmv of the packed matrix equals the exact product of the textbook-pruned dense matrix
    (within fp64 summation error) on tiny shapes, for every pattern."""
    rng = np.random.default_rng(seed)
    for R, C in ((1, 32), (2, 64), (3, 96), (7, 64)):
        for n, m in patterns:
            W = (rng.standard_normal((R, C)) * 0.5).astype(np.float16)
            # adversarial magnitudes: large values, subnormals and cancellation
            W[0, :4] = np.array([1000.0, -1000.0, 2 ** -24, 3.0], np.float16)
            x = rng.standard_normal(C).astype(np.float16)
            x[:3] = np.array([1.0, 1.0, 2 ** -14], np.float16)
            values, masks = pack_fn(W, n, m)
            got = spmv_fn(values, masks, x, C, n, m)
            Wp = textbook_prune_dense(W, n, m)
            exact = brute_force_y(Wp, x)
            scale = np.abs(Wp.astype(np.float64)) @ np.abs(x.astype(np.float64))
            for r in range(R):
                assert abs(Fraction(float(got[r])) - exact[r]) <= Fraction(1e-12) * Fraction(float(scale[r]) + 1e-300), \
                    (R, C, n, m, r, float(got[r]), float(exact[r]))


def check_gemv_bruteforce(gemv_fn, seed=6):
    """Dense product on non-square shapes against nested-loop exact sums."""
    rng = np.random.default_rng(seed)
    for R, C in ((3, 32), (5, 64), (2, 96)):
        W = rng.standard_normal((R, C)).astype(np.float16)
        x = rng.standard_normal(C).astype(np.float16)
        got = gemv_fn(W, x)
        exact = brute_force_y(W, x)
        scale = np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64))
        for r in range(R):
            assert abs(Fraction(float(got[r])) - exact[r]) <= Fraction(1e-12) * Fraction(float(scale[r])), (R, C, r)


def check_exact_ref(exact_fn):
    """exact_ref on closed forms: subnormal products, sums of ones, and cancellation."""
    tiny = np.float16(2.0 ** -24)
    W = np.array([[tiny, 0, 0, 0], [1, 1, 1, 1], [65504, -65504, 1, 0]], np.float16)
    x = np.array([tiny, 1, 1, 1], np.float16)
    y = exact_fn(W, x)
    assert y[0] == Fraction(1, 2 ** 48)
    assert y[1] == Fraction(3) + Fraction(1, 2 ** 24)
    assert y[2] == Fraction(65504, 2 ** 24) - 65504 + 1


def check_unit_sum(pack_fn, spmv_fn):
    """All weights equal c = 2^-6 and x = ones: y_r = (C/2)*c exactly, for every pattern."""
    C = 4096
    W = np.full((3, C), 2.0 ** -6, np.float16)
    x = np.ones(C, np.float16)
    for n, m in PATTERNS:
        v, mk = pack_fn(W, n, m)
        y = spmv_fn(v, mk, x, C, n, m)
        assert np.all(y == 32.0), (n, m, y)


# ----------------------------------------------------------------------------
# small-batch product (B activation vectors, one per row of X)
# ----------------------------------------------------------------------------
def check_spmm_worked_example(pack_fn, spmm_fn):
    """The golden row against a batch of hand-checkable vectors: x = c/8 gives the golden
    exact y; x = ones gives the exact sum of the kept values; a one-hot x = e_c gives
    w_c if column c is kept and 0 otherwise (all exact in fp64)."""
    row, x, cases = load_worked_row()
    W = row.reshape(1, 32)
    onehots = (0, 9, 22, 31)
    X = np.zeros((2 + len(onehots), 32), np.float16)
    X[0] = x
    X[1] = 1.0
    for i, c in enumerate(onehots):
        X[2 + i, c] = 1.0
    for n, m, mask, vals, y in cases:
        values, masks = pack_fn(W, n, m)
        got = np.asarray(spmm_fn(values, masks, X, 32, n, m))
        assert got.shape == (X.shape[0], 1), got.shape
        assert float(got[0, 0]) == float(y), (n, m, "x = c/8")
        total = sum(Fraction(float(v)) for v in vals.astype(np.float64))
        assert float(got[1, 0]) == float(total), (n, m, "x = ones")
        for i, c in enumerate(onehots):
            want = float(row[c]) if (mask >> c) & 1 else 0.0
            assert float(got[2 + i, 0]) == want, (n, m, "one-hot", c)


def check_spmm_bruteforce(pack_fn, spmm_fn, seed=7):
    """Every row of the batch against nested-loop exact sums over the textbook-pruned
    matrix, on tiny non-square shapes (B differs from rows, so a transposed result or
    operand fails)."""
    rng = np.random.default_rng(seed)
    for R, C, B in ((1, 32, 2), (3, 64, 3), (7, 96, 5), (2, 64, 8)):
        for n, m in PATTERNS:
            W = (rng.standard_normal((R, C)) * 0.5).astype(np.float16)
            W[0, :4] = np.array([1000.0, -1000.0, 2 ** -24, 3.0], np.float16)
            X = rng.standard_normal((B, C)).astype(np.float16)
            X[:, 0] = np.arange(B, dtype=np.float16)          # distinct rows
            values, masks = pack_fn(W, n, m)
            got = np.asarray(spmm_fn(values, masks, X, C, n, m))
            assert got.shape == (B, R), (got.shape, B, R)
            Wp = textbook_prune_dense(W, n, m)
            for b in range(B):
                exact = brute_force_y(Wp, X[b])
                scale = np.abs(Wp.astype(np.float64)) @ np.abs(X[b].astype(np.float64))
                for r in range(R):
                    assert abs(Fraction(float(got[b, r])) - exact[r]) <= \
                        Fraction(1e-12) * Fraction(float(scale[r]) + 1e-300), (R, C, B, n, m, b, r)


def check_spmm_exact_linearity(pack_fn, spmm_fn, seed=8):
    """With small-integer weights and activations every product and sum is exact in fp64,
    so the batch product must be exactly linear in X and must permute with the rows of X."""
    rng = np.random.default_rng(seed)
    R, C, B = 5, 64, 4
    W = rng.integers(-8, 9, (R, C)).astype(np.float16)
    X1 = rng.integers(-4, 5, (B, C)).astype(np.float16)
    X2 = rng.integers(-4, 5, (B, C)).astype(np.float16)
    perm = np.array([2, 0, 3, 1])
    for n, m in PATTERNS:
        v, mk = pack_fn(W, n, m)
        y1 = np.asarray(spmm_fn(v, mk, X1, C, n, m))
        y2 = np.asarray(spmm_fn(v, mk, X2, C, n, m))
        y12 = np.asarray(spmm_fn(v, mk, (X1 + X2).astype(np.float16), C, n, m))
        assert np.array_equal(y12, y1 + y2), (n, m)
        assert np.array_equal(np.asarray(spmm_fn(v, mk, X1[perm], C, n, m)), y1[perm]), (n, m)


def check_gemm_bruteforce(gemm_fn, seed=9):
    """Dense batch product on non-square shapes against nested-loop exact sums."""
    rng = np.random.default_rng(seed)
    for R, C, B in ((3, 32, 2), (5, 64, 7), (2, 96, 3)):
        W = rng.standard_normal((R, C)).astype(np.float16)
        X = rng.standard_normal((B, C)).astype(np.float16)
        got = np.asarray(gemm_fn(W, X))
        assert got.shape == (B, R), got.shape
        for b in range(B):
            exact = brute_force_y(W, X[b])
            scale = np.abs(W.astype(np.float64)) @ np.abs(X[b].astype(np.float64))
            for r in range(R):
                assert abs(Fraction(float(got[b, r])) - exact[r]) <= Fraction(1e-12) * Fraction(float(scale[r])), (R, C, B, b, r)
