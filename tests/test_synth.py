"""CPU tests of the seeded input generators."""
import numpy as np

import synth


def test_weight_is_deterministic_and_thread_independent():
    n = synth.BLOCK + 1000  # spans two blocks
    a = synth.standard_normal_f32(n, seed=5, threads=1)
    b = synth.standard_normal_f32(n, seed=5, threads=4)
    assert np.array_equal(a, b)
    assert not np.array_equal(a[:100], synth.standard_normal_f32(100, seed=6))


def test_weight_rows_match_full_matrix():
    rows, cols = 3000, 1536  # 4.6M elements: crosses a block boundary mid-row
    W = synth.weight(rows, cols, seed=9)
    idx = [0, 1, 2730, 2731, 2999]
    assert np.array_equal(synth.weight_rows(idx, rows, cols, seed=9).view(np.uint16),
                          W[idx].view(np.uint16))


def test_distributions():
    W = synth.weight(512, 1024, seed=1)
    x = synth.activation(8192, seed=2)
    assert W.dtype == np.float16 and x.dtype == np.float16
    assert abs(float(W.astype(np.float64).std()) - 0.02) < 1e-3
    assert abs(float(x.astype(np.float64).std()) - 1.0) < 0.05
    t = synth.tie_heavy_weight(4, 64, seed=3)
    assert t.dtype == np.float16 and not np.isnan(t.astype(np.float32)).any()


def test_seed_scheme_distinct():
    seeds = {synth.weight_seed(c, l, p) for c in (1, 2, 3, 4) for l in range(7) for p in synth.PATTERNS}
    seeds |= {synth.decode_seed(b, p) for b in range(32) for p in range(7)}
    assert len(seeds) == 4 * 7 * 4 + 32 * 7
