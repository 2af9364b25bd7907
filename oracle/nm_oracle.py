"""Plain, slow, obviously-correct CPU oracle (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module. It shares no code with the HIP
path and the HIP path never routes through it.

Sources (the pages, cited by title and section):

[NEWS-NEW]  news.bitwarelabs.com, "SparseDecoding: decoding-aware pruning for
            accurate and fast LLM generation", section "What's new": batch-one
            decoding is memory-bandwidth bound and dominated by sparse
            matrix-vector products; the system pairs N:M semi-structured
            sparsity (N kept of every M consecutive weights) with a custom
            SpMV kernel using bitmask indexing and fixed-step traversal.
[KERNEL]    aimodeling.com article on SparseDecoding, section "The Kernel Is
            the Other Half of the Answer": one 32-bit mask word indexes 32
            consecutive input columns; at 50% sparsity every word has exactly
            16 set bits; the bitmask stands in for per-nonzero 32-bit column
            indices; the patterns 2:4, 4:8, 8:16 and 16:32 all keep half the
            weights with the same metadata traffic.

Readings where the pages are silent (each is also listed with its reason in
the design notes of the repository):

* Precision: W, x and y are fp16 (IEEE binary16); the oracle computes in fp64
  and returns y unrounded.
* Selection: the magnitude of an fp16 weight is its bit pattern with the sign
  bit cleared, compared as an unsigned integer (this orders |w| for every
  non-NaN value and makes -0 equal +0). In each aligned group of M columns the
  N largest magnitudes are kept; equal magnitudes go to the lower column.
* Groups are aligned at multiples of M; M divides 32, so no group straddles a
  mask word.
* Bit j (least significant = 0) of mask word w of a row covers column 32*w + j.
* Values are stored row by row; within a row mask word by mask word; within a
  word in ascending column order. A row of C columns therefore owns C*N/M
  values and C/32 mask words, and word w's values start at (32*N/M)*w.
* Dropped positions unpack to +0 (bits 0x0000).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

PATTERNS = ((2, 4), (4, 8), (8, 16), (16, 32))
# 25% density with the same bitmask: 32*N/M = 8 kept values per mask word. [NEWS-NEW]
# states the method for N:M in general; the pages measure only the 50% patterns.
PATTERNS_QUARTER = ((1, 4), (2, 8), (4, 16), (8, 32))
SUPPORTED_PATTERNS = PATTERNS + PATTERNS_QUARTER
WORD_BITS = 32  # columns covered by one mask word [KERNEL]

# Tolerance for fp16 y computed with fp32 accumulation against the fp64 oracle:
# per element |y - ref| <= ATOL + RTOL*|ref|, and relative L2 error <= REL_L2.
ATOL = 2e-3
RTOL = 1e-2
REL_L2 = 1e-3


def _check_pattern(N: int, M: int) -> None:
    if (N, M) not in SUPPORTED_PATTERNS:
        raise ValueError(f"unsupported N:M pattern {N}:{M}")


def _as_bits(W) -> np.ndarray:
    W = np.asarray(W)
    if W.dtype == np.float16:
        return W.view(np.uint16)
    if W.dtype == np.uint16:
        return W
    raise TypeError("expected fp16 values or their uint16 bit patterns")


def fp16_rne(y) -> np.ndarray:
    """Round float64 values to fp16 with round-to-nearest-even (numpy's cast)."""
    return np.asarray(y, dtype=np.float64).astype(np.float16)


def magnitude_key(W) -> np.ndarray:
    """Integer magnitude of fp16 weights: the bit pattern with the sign bit cleared."""
    return (_as_bits(W) & np.uint16(0x7FFF)).astype(np.int32)


def keep_ref(W, N: int, M: int, row_chunk: int = 256) -> np.ndarray:
    """Boolean [R, C]: which weights an N:M magnitude selection keeps.

    [NEWS-NEW]: N of every M consecutive weights survive. For element i of an
    aligned group of M columns its rank is the number of group members with a
    strictly larger magnitude plus the number of members at a lower column
    with an equal magnitude; it is kept iff rank < N. This rank is a
    permutation of 0..M-1 within every group, so exactly N are kept.
    """
    _check_pattern(N, M)
    bits = _as_bits(W)
    R, C = bits.shape
    if C % WORD_BITS:
        raise ValueError("cols must be a multiple of 32")
    out = np.empty((R, C), dtype=bool)
    col = np.arange(M)
    lower_col = col[None, :] < col[:, None]          # [i, k]: k is left of i
    for r0 in range(0, R, row_chunk):
        key = magnitude_key(bits[r0:r0 + row_chunk]).reshape(-1, C // M, M)
        ki = key[..., :, None]                        # element i
        kk = key[..., None, :]                        # other member k
        rank = (kk > ki).sum(-1) + ((kk == ki) & lower_col).sum(-1)
        out[r0:r0 + row_chunk] = (rank < N).reshape(-1, C)
    return out


def prune_ref(W, N: int, M: int) -> np.ndarray:
    """fp16 bits [R, C]: W with every non-kept weight replaced by +0."""
    bits = _as_bits(W)
    return np.where(keep_ref(bits, N, M), bits, np.uint16(0)).astype(np.uint16)


def pack_ref(W, N: int, M: int):
    """Encode W as (values uint16 [R, C*N/M], masks uint32 [R, C/32]).

    [KERNEL]: mask word w of a row has bit j set iff column 32*w + j is kept;
    the kept fp16 values are laid out in row order (row-major gather of the
    kept entries, which visits each row's columns in ascending order).
    """
    bits = _as_bits(W)
    R, C = bits.shape
    kept = keep_ref(bits, N, M)
    weights = np.uint64(1) << np.arange(WORD_BITS, dtype=np.uint64)
    masks = (kept.reshape(R, C // WORD_BITS, WORD_BITS).astype(np.uint64) * weights).sum(-1)
    values = bits[kept].reshape(R, C * N // M)
    return values.astype(np.uint16), masks.astype(np.uint32)


def unpack_ref(values, masks, cols: int, N: int, M: int) -> np.ndarray:
    """Dense fp16 bits [R, cols] from (values, masks); dropped entries are +0.

    [KERNEL]: every word holds exactly 32*N/M kept values, so word w's values
    start at a fixed offset (32*N/M)*w; the value for set bit j is the one at
    that offset plus the number of set bits below j.
    """
    _check_pattern(N, M)
    masks = np.asarray(masks, dtype=np.uint32)
    values = np.asarray(values).view(np.uint16) if np.asarray(values).dtype == np.float16 \
        else np.asarray(values, dtype=np.uint16)
    R, nw = masks.shape
    if nw * WORD_BITS != cols:
        raise ValueError("masks shape does not match cols")
    per_word = WORD_BITS * N // M
    if values.shape != (R, nw * per_word):
        raise ValueError("values shape does not match masks")
    bit = ((masks[..., None] >> np.arange(WORD_BITS, dtype=np.uint32)) & np.uint32(1)).astype(np.int64)
    if not np.all(bit.sum(-1) == per_word):
        raise ValueError(f"a mask word does not have exactly {per_word} set bits")
    below = np.cumsum(bit, axis=-1) - bit                       # set bits strictly below j
    vals = values.reshape(R, nw, per_word)
    gathered = np.take_along_axis(vals, np.minimum(below, per_word - 1), axis=-1)
    dense = np.where(bit.astype(bool), gathered, np.uint16(0))
    return dense.reshape(R, cols).astype(np.uint16)


def spmv_ref(values, masks, x, cols: int, N: int, M: int) -> np.ndarray:
    """y (float64, unrounded) = unpack(values, masks) @ x, densified and accumulated in fp64.

    Every fp16 x fp16 product is exact in fp64, so the only error is the fp64
    summation.
    """
    D = unpack_ref(values, masks, cols, N, M).view(np.float16).astype(np.float64)
    return D @ np.asarray(x, dtype=np.float16).astype(np.float64)


def gemv_ref(W, x) -> np.ndarray:
    """Dense y (float64, unrounded) = W @ x for the dense baseline."""
    Wd = _as_bits(W).view(np.float16).astype(np.float64)
    return Wd @ np.asarray(x, dtype=np.float16).astype(np.float64)


def spmm_ref(values, masks, X, cols: int, N: int, M: int) -> np.ndarray:
    """Y (float64, unrounded) [B, rows]: row b is the pruned matrix times row b of X.

    X is fp16 [B, cols], one activation vector per row (the layout of a batch of B
    tokens). [NEWS-NEW] splits inference into batch-one decoding, dominated by
    sparse matrix-vector products, and prefill / larger batches, which run sparse
    matrix-matrix products; for a small batch the same packed matrix is applied to
    each of the B vectors. Densified and accumulated in fp64, like spmv_ref.
    """
    D = unpack_ref(values, masks, cols, N, M).view(np.float16).astype(np.float64)
    Xf = np.asarray(X, dtype=np.float16).astype(np.float64)
    if Xf.ndim != 2 or Xf.shape[1] != cols:
        raise ValueError(f"X must be [B, {cols}], got {Xf.shape}")
    return Xf @ D.T


def gemm_ref(W, X) -> np.ndarray:
    """Dense Y (float64, unrounded) [B, rows] = X @ W.T: the dense baseline of spmm_ref."""
    Wd = _as_bits(W).view(np.float16).astype(np.float64)
    Xf = np.asarray(X, dtype=np.float16).astype(np.float64)
    if Xf.ndim != 2 or Xf.shape[1] != Wd.shape[1]:
        raise ValueError(f"X must be [B, {Wd.shape[1]}], got {Xf.shape}")
    return Xf @ Wd.T


def exact_ref(W, x) -> list:
    """Exact y = W @ x as Fractions, for tiny inputs (Python-int brute force).

    Every finite fp16 is an integer multiple of 2**-24 (the smallest
    subnormal), so each product is an integer times 2**-48 and the sum is an
    exact integer in Python.
    """
    Wf = _as_bits(W).view(np.float16).astype(np.float64)
    xf = np.asarray(x, dtype=np.float16).astype(np.float64)
    scale = 2 ** 24
    xi = [int(v * scale) for v in xf]
    for v, i in zip(xf, xi):
        assert i == v * scale, "non-finite or non-fp16 input"
    out = []
    for row in Wf:
        acc = 0
        for w, xv in zip(row, xi):
            wi = int(w * scale)
            assert wi == w * scale, "non-finite or non-fp16 input"
            acc += wi * xv
        out.append(Fraction(acc, scale * scale))
    return out


def y_tolerance_report(y, y_ref) -> dict:
    """Compare a computed fp16 y with the fp64 reference.

    Returns the worst |y - ref| / (ATOL + RTOL*|ref|) ratio, the relative L2
    error and whether every element is finite.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {y_ref.shape}")
    finite = bool(np.all(np.isfinite(y)))
    err = np.abs(y - y_ref)
    bound = ATOL + RTOL * np.abs(y_ref)
    worst = float(np.max(err / bound)) if y.size else 0.0
    den = float(np.linalg.norm(y_ref))
    rel = float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y - y_ref))
    return {"max_err_over_bound": worst, "rel_l2": rel, "finite": finite,
            "ok": finite and worst <= 1.0 and rel <= REL_L2}


def y_within_tolerance(y, y_ref) -> bool:
    return y_tolerance_report(y, y_ref)["ok"]
