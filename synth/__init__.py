"""Seeded synthetic inputs for the batch-one N:M sparse matrix-vector product.

This module only draws random numbers and describes workload shapes. It holds
none of the method's arithmetic (no magnitude selection, no packing, no
products), so both the HIP path and the CPU oracle can be fed from it without
sharing any of their computation.

Distributions (the pages measure pruned Llama-3.1-8B / Llama-3.3-70B /
Qwen3-14B/32B layers, whose trained weights are not available, so these seeded
layers of the same shapes stand in for them):

* W: fp32 standard normal scaled by 0.02 (standard deviation 0.02), rounded to
  fp16 with round-to-nearest-even.
* x: fp32 standard normal rounded to fp16 (RNE).

Every array is a pure function of (shape, seed): the flat index space is cut
into fixed blocks of ``BLOCK`` elements and block ``b`` draws from
``PCG64(SeedSequence([seed, b]))``, so the result does not depend on how many
threads fill it.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 1 << 22
BASE_SEED = 20261008
WEIGHT_STD = 0.02

PATTERNS = ((2, 4), (4, 8), (8, 16), (16, 32))
PATTERNS_QUARTER = ((1, 4), (2, 8), (4, 16), (8, 32))   # 25% density, 8 values per mask word
PATTERN_ID = {p: i for i, p in enumerate(PATTERNS + PATTERNS_QUARTER)}

# Workloads: name -> list of (layer name, rows, cols); rows = output features,
# cols = input features (W is [out, in] row-major, y = W @ x).
LLAMA31_8B = [("q_proj", 4096, 4096), ("kv_proj", 1024, 4096),
              ("gate_up_proj", 14336, 4096), ("down_proj", 4096, 14336)]
QWEN3 = [("q14b_proj", 5120, 5120), ("kv_proj", 1024, 5120),
         ("up_gate14b_proj", 17408, 5120), ("down14b_proj", 5120, 17408),
         ("q32b_proj", 8192, 5120), ("up_gate32b_proj", 25600, 5120),
         ("down32b_proj", 5120, 25600)]
LLAMA33_70B = [("qo_proj", 8192, 8192), ("kv_proj", 1024, 8192),
               ("gate_up_proj", 28672, 8192), ("down_proj", 8192, 28672)]
# One GPU's share of the Llama-3.3-70B MLP split 8 ways: the gate/up rows (28672 / 8) and
# the down projection's columns (28672 / 8, whole 32-column mask words).
LLAMA33_70B_TP8_SHARDS = [("gate_up_rows_1of8", 3584, 8192), ("down_cols_1of8", 8192, 3584)]
LLAMA31_8B_DECODE_LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096),
                           ("o", 4096, 4096), ("gate", 14336, 4096), ("up", 14336, 4096),
                           ("down", 4096, 14336)]

WORKLOADS = {
    1: {"name": "single-2:4-256x512", "layers": [("single", 256, 512)], "patterns": [(2, 4)]},
    2: {"name": "llama3.1-8b-projections", "layers": LLAMA31_8B, "patterns": list(PATTERNS)},
    3: {"name": "qwen3-14b-32b-projections", "layers": QWEN3, "patterns": [(2, 4), (16, 32)]},
    4: {"name": "llama3.3-70b-projections", "layers": LLAMA33_70B, "patterns": [(2, 4)]},
    5: {"name": "llama3.1-8b-decode-step-32-layers", "layers": LLAMA31_8B_DECODE_LAYER,
        "n_layers": 32, "patterns": [(2, 4)]},
}


def weight_seed(cfg: int, layer_idx: int, pattern) -> int:
    """Seed of W for workload ``cfg``, layer ``layer_idx`` and N:M ``pattern``."""
    return BASE_SEED + 1000 * cfg + 10 * layer_idx + PATTERN_ID[tuple(pattern)]


def x_seed(cfg: int, layer_idx: int, pattern) -> int:
    return weight_seed(cfg, layer_idx, pattern) + 500


def decode_seed(block: int, proj: int) -> int:
    """Seed of W for the 32-layer decode sweep, transformer block ``block``, projection ``proj``."""
    return BASE_SEED + 100000 + 100 * block + proj


def decode_x_seed(block: int, proj: int) -> int:
    return decode_seed(block, proj) + 50


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def standard_normal_f32(n: int, seed: int, threads: int | None = None) -> np.ndarray:
    """n fp32 standard normals, block-seeded (see module docstring)."""
    out = np.empty(n, np.float32)
    nblocks = (n + BLOCK - 1) // BLOCK

    def fill(b):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b])))
        lo = b * BLOCK
        hi = min(n, lo + BLOCK)
        g.standard_normal(out=out[lo:hi], dtype=np.float32)

    threads = threads or _threads()
    if nblocks <= 1 or threads == 1:
        for b in range(nblocks):
            fill(b)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblocks)))
    return out


def weight(rows: int, cols: int, seed: int, std: float = WEIGHT_STD) -> np.ndarray:
    """fp16 [rows, cols]: N(0, std^2) drawn in fp32, rounded to fp16 (RNE)."""
    z = standard_normal_f32(rows * cols, seed)
    z *= np.float32(std)
    return z.astype(np.float16).reshape(rows, cols)


def activation(cols: int, seed: int) -> np.ndarray:
    """fp16 [cols]: N(0, 1) drawn in fp32, rounded to fp16 (RNE)."""
    return standard_normal_f32(cols, seed).astype(np.float16)


def activations(tokens: int, cols: int, seed: int) -> np.ndarray:
    """fp16 [tokens, cols]: a batch of activation rows (prompt tokens), N(0, 1) drawn in
    fp32 as one stream, rounded to fp16 (RNE)."""
    return standard_normal_f32(tokens * cols, seed).reshape(tokens, cols).astype(np.float16)


def weight_rows(rows_idx, rows: int, cols: int, seed: int, std: float = WEIGHT_STD) -> np.ndarray:
    """The listed rows of ``weight(rows, cols, seed)`` without drawing the whole matrix.

    Rows are regenerated block by block, so the result is bit-identical to
    slicing the full matrix.
    """
    rows_idx = np.asarray(rows_idx, dtype=np.int64)
    out = np.empty((len(rows_idx), cols), np.float16)
    cache = {}
    for i, r in enumerate(rows_idx):
        lo = int(r) * cols
        hi = lo + cols
        parts = []
        for b in range(lo // BLOCK, (hi - 1) // BLOCK + 1):
            if b not in cache:
                g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b])))
                blen = min(BLOCK, rows * cols - b * BLOCK)
                blk = np.empty(blen, np.float32)
                g.standard_normal(out=blk, dtype=np.float32)
                cache[b] = blk
            blk = cache[b]
            s = max(lo, b * BLOCK) - b * BLOCK
            e = min(hi, (b + 1) * BLOCK) - b * BLOCK
            parts.append(blk[s:e])
        z = np.concatenate(parts)
        out[i] = (z * np.float32(std)).astype(np.float16)
    return out


def tie_heavy_weight(rows: int, cols: int, seed: int) -> np.ndarray:
    """fp16 [rows, cols] drawn from a small alphabet so magnitude ties are common.

    The alphabet mixes signs, both zeros, subnormals, normal values, the largest
    finite value and infinities, so every ordering corner of a magnitude key is
    exercised.  No NaN (its result under the product is unspecified).
    """
    alphabet = np.array([0.0, -0.0, 2.0 ** -24, -(2.0 ** -24), 2.0 ** -20, 0.5, -0.5,
                         1.0, -1.0, 0.0625, -0.0625, 65504.0, -65504.0, np.inf, -np.inf],
                        dtype=np.float16)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xA1])))
    # weight the alphabet towards a few values so equal keys are frequent
    p = np.array([4, 2, 2, 2, 2, 6, 6, 4, 4, 3, 3, 1, 1, 1, 1], dtype=np.float64)
    idx = g.choice(len(alphabet), size=rows * cols, p=p / p.sum())
    return alphabet[idx].reshape(rows, cols)
