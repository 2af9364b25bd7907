"""GPU tests of the entry points under HIP graph capture: every product is captured once
into a torch.cuda.CUDAGraph and replayed several times, with the program's own eager work
(other products, torch ops, a new input written in place) between the replays. Each replay
must give the bits an eager call gives on the same inputs (the kernels are deterministic),
and the first eager result is checked against the CPU oracle, so the captured path is tied
to the oracle too. The library allocates nothing and records no memset (the column split
resets its counters in its kernels), so nothing it captures depends on the capture-time
state of its buffers."""
import numpy as np
import pytest
import torch

import oracle
import semi_structured_sparse_amd as nm
import synth
from tests.gpu_helpers import device, down_bits16, down_f16, say, up_f16

pytestmark = pytest.mark.gpu
REPLAYS = 4


def _replay_and_check(run, inputs, out, reseed):
    """run(): the product writing into `out`; inputs: tensors it reads; reseed(i): new
    contents for the inputs (written in place) before replay i. Captures run(), then for
    each replay: refresh the inputs, do unrelated eager work, replay, and compare with an
    eager call on the same inputs."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, dtype=torch.float16, device=device())
    for i in range(REPLAYS):
        reseed(i)
        scratch.normal_()                         # eager work between the replays
        _ = (scratch * 2).sum()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = down_bits16(out).copy()
        out.fill_(float("nan"))
        run()                                     # eager on the same inputs
        torch.cuda.synchronize()
        want = down_bits16(out)
        assert np.array_equal(got, want), f"replay {i} differs from the eager call"
    del g


# 2100 x 4096: spmv_kernel; 1024 x 4096: at 16:32 the narrow kernel
@pytest.mark.parametrize("R,C", [(2100, 4096), (1024, 4096)])
@pytest.mark.parametrize("N,M", synth.PATTERNS)
def test_spmv_graph_replays(N, M, R, C):
    say(f"graph spmv {N}:{M} {R}x{C} {nm.spmv_variant(R, C, N, M)}")
    W = synth.weight(R, C, 5000 + N)
    x = synth.activation(C, 5001 + N)
    values, masks = nm.nm_pack(up_f16(W), N, M)
    xd = up_f16(x)
    y = torch.empty(R, dtype=torch.float16, device=device())
    nm.nm_spmv(values, masks, xd, N, M, out=y)
    torch.cuda.synchronize()
    rv, rm = oracle.pack_ref(W[:64], N, M)
    assert oracle.y_tolerance_report(down_f16(y)[:64], oracle.spmv_ref(rv, rm, x, C, N, M))["ok"]

    def reseed(i):
        xd.copy_(up_f16(synth.activation(C, 5100 + 10 * N + i)))

    _replay_and_check(lambda: nm.nm_spmv(values, masks, xd, N, M, out=y), [values, masks, xd], y, reseed)


def test_gemv_dense_graph_replays():
    R, C = 1500, 4096
    W = up_f16(synth.weight(R, C, 5200))
    x = synth.activation(C, 5201)
    xd = up_f16(x)
    y = torch.empty(R, dtype=torch.float16, device=device())
    _replay_and_check(lambda: nm.nm_gemv_dense(W, xd, out=y), [W, xd], y,
                      lambda i: xd.copy_(up_f16(synth.activation(C, 5210 + i))))


# batch products: the small-batch kernel (B = 4), the skinny kernel (2:4 at B = 8) and its
# split variant (4:8 at B = 8; 8:16 at B = 20: 16 on it, the last 4 on the small-batch kernel),
# three skinny launches (2:4 at B = 40) and the prefill kernel (B = 64)
BATCH_CASES = [(2, 4, 4), (2, 4, 8), (4, 8, 8), (8, 16, 20), (16, 32, 6), (2, 4, 40), (2, 4, 64)]


@pytest.mark.parametrize("N,M,B", BATCH_CASES)
def test_spmm_graph_replays(N, M, B):
    R, C = 2064, 1024
    say(f"graph spmm {N}:{M} {R}x{C} B={B} {nm.spmm_variant(R, C, B, N, M)}")
    W = synth.weight(R, C, 5300 + N + B)
    X = synth.activations(B, C, 5301 + N + B)
    values, masks = nm.nm_pack(up_f16(W), N, M)
    Xd = up_f16(X)
    Y = torch.empty((B, R), dtype=torch.float16, device=device())
    nm.nm_spmm(values, masks, Xd, N, M, out=Y)
    torch.cuda.synchronize()
    rv, rm = oracle.pack_ref(W[:48], N, M)
    rep = oracle.y_tolerance_report(down_f16(Y)[:, :48], oracle.spmm_ref(rv, rm, X, C, N, M))
    assert rep["ok"], rep

    def reseed(i):
        Xd.copy_(up_f16(synth.activations(B, C, 5400 + 10 * B + i)))

    _replay_and_check(lambda: nm.nm_spmm(values, masks, Xd, N, M, out=Y), [values, masks, Xd], Y, reseed)


def test_prefill_graph_replays():
    R, C, T = 1000, 2048, 300
    W = synth.weight(R, C, 5500)
    values, masks = nm.nm_pack(up_f16(W), 2, 4)
    Wd = up_f16(W)
    Xd = up_f16(synth.activations(T, C, 5501))
    Y = torch.empty((T, R), dtype=torch.float16, device=device())
    Yd = torch.empty((T, R), dtype=torch.float16, device=device())

    def reseed(i):
        Xd.copy_(up_f16(synth.activations(T, C, 5510 + i)))

    _replay_and_check(lambda: nm.nm_spmm_prefill(values, masks, Xd, out=Y), [values, masks, Xd], Y, reseed)
    _replay_and_check(lambda: nm.nm_gemm_dense_prefill(Wd, Xd, out=Yd), [Wd, Xd], Yd, reseed)


# column splits (nm_spmm_ws, and nm_spmm_noalloc on the library's static scratch): the
# counters are reset by the kernels themselves, so replays find them at zero
SPLIT_GRAPH_CASES = [(2, 4, 1024, 8192, 8), (4, 8, 1024, 4096, 12), (2, 4, 1000, 8192, 17), (8, 16, 4096, 4096, 64),
                     (2, 4, 1024, 4096, 256), (16, 32, 1024, 4096, 16), (16, 32, 4096, 14336, 40),
                     (2, 4, 4000, 14304, 300), (8, 16, 2050, 10240, 260)]


@pytest.mark.parametrize("N,M,R,C,B", SPLIT_GRAPH_CASES)
def test_spmm_column_split_graph_replays(N, M, R, C, B):
    need = nm.spmm_workspace_bytes(R, C, B, N, M)
    assert need > 0
    say(f"graph spmm column split {N}:{M} {R}x{C} B={B} workspace={need}")
    W = synth.weight(R, C, 5600 + N + B)
    X = synth.activations(B, C, 5601 + N + B)
    values, masks = nm.nm_pack(up_f16(W), N, M)
    Xd = up_f16(X)
    ws = nm.spmm_workspace(R, C, B, N, M)
    Y = torch.empty((B, R), dtype=torch.float16, device=device())
    nm.nm_spmm_ws(values, masks, Xd, N, M, ws, out=Y)
    torch.cuda.synchronize()
    rv, rm = oracle.pack_ref(W[:48], N, M)
    rep = oracle.y_tolerance_report(down_f16(Y)[:, :48], oracle.spmm_ref(rv, rm, X, C, N, M))
    assert rep["ok"], rep

    def reseed(i):
        Xd.copy_(up_f16(synth.activations(B, C, 5700 + 10 * B + i)))

    _replay_and_check(lambda: nm.nm_spmm_ws(values, masks, Xd, N, M, ws, out=Y), [values, masks, Xd], Y, reseed)
    cus = torch.cuda.get_device_properties(device()).multi_processor_count
    assert int(ws[:-(-(4 * cus) // 256) * 256].count_nonzero()) == 0
    Yn = torch.empty((B, R), dtype=torch.float16, device=device())
    _replay_and_check(lambda: nm.nm_spmm_noalloc(values, masks, Xd, N, M, out=Yn), [values, masks, Xd], Yn, reseed)
    assert np.array_equal(down_bits16(Yn), down_bits16(nm.nm_spmm_ws(values, masks, Xd, N, M, ws)))
