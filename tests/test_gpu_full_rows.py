"""All-row parity at full size: every row of every Qwen3-14B/32B and Llama-3.3-70B projection
layer (and their patterns), in the launch configuration the bench times. The packed values
and masks are compared bit for bit with the oracle's encoding on every row, which covers every
grid-stride pass of the encoder, and y is within the tolerance on every row."""
import pytest

import synth
from tests.gpu_helpers import check_all_rows, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _cases():
    out = []
    for cfg in (3, 4):
        wl = synth.WORKLOADS[cfg]
        for li, (name, R, C) in enumerate(wl["layers"]):
            for pat in wl["patterns"]:
                out.append(pytest.param(cfg, li, name, R, C, pat, id=f"cfg{cfg}-{name}-{R}x{C}-{pat[0]}:{pat[1]}"))
    return out


@pytest.mark.parametrize("cfg,li,name,R,C,pat", _cases())
def test_every_row(cfg, li, name, R, C, pat):
    N, M = pat
    say(f"all rows cfg{cfg} {name} {R}x{C} {N}:{M}")
    W = synth.weight(R, C, synth.weight_seed(cfg, li, pat))
    x = synth.activation(C, synth.x_seed(cfg, li, pat))
    rep = check_all_rows(W, x, N, M, f"cfg{cfg}-{name}")
    say(f"  {R} rows: {rep}")
