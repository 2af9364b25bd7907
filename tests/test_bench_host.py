"""Host logic of bench.py, on the CPU: the one-GPU guard, the algorithmic byte counts the
roofline divides by, the source hash that voids committed counter figures once a kernel
changes, and the roofline object of the decode sweep."""
import os
import subprocess
import sys

import bench


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_algorithmic_bytes_closed_forms():
    """values + masks + x + y: 1.125 R C + 2 (R + C) bytes at 50% (R C / 2 fp16 values and
    one 4-byte word per 32 columns), 0.625 R C + 2 (R + C) at 25%, 2 R C + 2 (R + C) dense;
    a batch of B vectors moves B copies of x and y."""
    for R, C in ((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (256, 512), (28672, 8192)):
        for N, M in ((2, 4), (4, 8), (8, 16), (16, 32)):
            assert bench.alg_bytes_sparse(R, C, N, M) == 9 * R * C // 8 + 2 * (R + C)
        for N, M in ((1, 4), (2, 8), (4, 16), (8, 32)):
            assert bench.alg_bytes_sparse(R, C, N, M) == 5 * R * C // 8 + 2 * (R + C)
        assert bench.alg_bytes_dense(R, C) == 2 * R * C + 2 * (R + C)
        assert bench.alg_bytes_sparse(R, C, 2, 4, B=8) == 9 * R * C // 8 + 8 * 2 * (R + C)
        assert bench.alg_bytes_dense(R, C, B=4) == 2 * R * C + 4 * 2 * (R + C)
    # the per-launch figure of the 4096 x 4096 layers in the committed counter summaries
    assert bench.alg_bytes_sparse(4096, 4096, 2, 4) == 18_890_752


def test_traffic_figures_are_void_once_the_kernel_code_changes(tmp_path):
    src = tmp_path / "kernel.h"
    src.write_text("int a = 1;  // a comment\n/* block */\n")
    counters = tmp_path / "counters.txt"
    counters.write_text(f"# header\nkernel_source_sha256: {bench.kernel_source_sha([str(src)])}\n"
                        "fetch_factor: 2.0\ntraffic k<1, 2>: 123456\n")
    assert bench.read_traffic("k<1, 2>", str(counters), [str(src)]) == 123456.0
    assert bench.read_traffic("k<3, 4>", str(counters), [str(src)]) is None
    src.write_text("int a = 1;   // another comment\n\n")   # comments and spacing only: still valid
    assert bench.read_traffic("k<1, 2>", str(counters), [str(src)]) == 123456.0
    src.write_text("int a = 2;\n")                            # a change of code voids them
    assert bench.read_traffic("k<1, 2>", str(counters), [str(src)]) is None
    assert bench.read_traffic("k<1, 2>", str(tmp_path / "missing.txt"), [str(src)]) is None


class _Variants:
    """Stands in for the binding's kernel-name query."""

    def __init__(self, names):
        self.names = names

    def spmv_variant(self, R, C, N, M):
        return self.names[(R, C)]


def test_decode_roofline():
    items = [dict(R=4096, C=4096, bytes=30_000_000), dict(R=1024, C=4096, bytes=40_000_000)]
    one = _Variants({(4096, 4096): "k", (1024, 4096): "k"})
    r = bench.decode_roofline(one, items, ms_token=0.01, N=2, M=4)   # 10 us per token, 2 launches
    assert r["kernel"] == "k" and r["launches_per_step"] == 2
    assert r["bytes_per_launch"] == 35_000_000 and abs(r["avg_launch_us"] - 5.0) < 1e-9
    assert abs(r["achieved"] - 7000.0) < 0.05 and abs(r["frac"] - 0.875) < 1e-4
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["traffic"] is None
    two = _Variants({(4096, 4096): "k", (1024, 4096): "other"})
    assert bench.decode_roofline(two, items, ms_token=0.01, N=2, M=4) is None


def test_parity_gate_finds_every_failed_record(capsys):
    """Any parity record (a dict under a key starting with "parity") whose ok is false, at any
    depth, fails the run: the JSON line is still printed, and the exit status is 3."""
    good = {"max_err_over_bound": 0.05, "rel_l2": 2e-4, "ok": True}
    bad = {"max_err_over_bound": 1703.5, "rel_l2": 1.45, "ok": False}
    out = {"value": 1.0, "cpu_baseline": {"parity_vs_gpu": dict(good)},
           "decode": {"parity": {"plain": dict(good), "grouped": dict(bad), "fused": dict(good)},
                      "cpu_baseline": {"parity_vs_gpu": dict(good)}},
           "per_layer": [{"parity_rows": dict(bad)}]}
    assert bench.parity_failures(out) == ["decode.parity.grouped", "per_layer[0].parity_rows"]
    assert bench.emit(out) == 3
    line = capsys.readouterr().out.strip()
    assert '"parity_ok": false' in line and line.startswith("{")
    out["decode"]["parity"]["grouped"] = dict(good)
    out["per_layer"] = []
    assert bench.parity_failures(out) == []
    assert bench.emit(out) == 0
    assert '"parity_ok": true' in capsys.readouterr().out
    # a record with no verdict, or a non-parity "ok", is not a failure
    assert bench.parity_failures({"parity": {"rows": 3}, "status": {"ok": False}}) == []


def test_pattern_spread():
    per_layer = [
        {"shape": "4096x4096", "pattern": "2:4", "us": 5.0},
        {"shape": "4096x4096", "pattern": "16:32", "us": 5.5},
        {"shape": "4096x4096", "pattern": "4:8", "us": 5.2},
        {"shape": "1024x4096", "pattern": "2:4", "us": 3.0},
        {"shape": "28672x8192", "pattern": "2:4", "us": 39.0, "in_step": False},
        {"shape": "28672x8192", "pattern": "16:32", "us": 45.0, "in_step": False},
    ]
    s = bench.pattern_spread(per_layer)
    assert set(s) == {"4096x4096"}   # one pattern only, or outside the step: no spread
    assert abs(s["4096x4096"]["spread"] - 0.1) < 1e-9
    assert s["4096x4096"]["fastest"] == "2:4" and s["4096x4096"]["slowest"] == "16:32"


def test_pool_copies():
    assert bench.pool_copies(600e6, 1 << 30) == 2
    assert bench.pool_copies(4.7e6, 1 << 30) == 229
    assert bench.pool_copies(3e9, 1 << 30) == 2


def test_best_dense_is_the_faster_of_ours_and_the_vendor_blas():
    assert bench.best_dense_us(299.5, 206.3) == 206.3
    assert bench.best_dense_us(80.2, 84.1) == 80.2
    assert bench.best_dense_us(80.2, float("nan")) == 80.2


def test_batch_workspace_arguments_and_kernel_names():
    """--batch B > 1 runs nm_spmm_ws: a layer with a workspace passes its pointer and size and
    is named as nm_spmm_ws's routing names it; one without passes NULL and is named as
    nm_spmm's routing names it; batch one passes nothing."""
    import bench

    class FakeWs:
        def data_ptr(self):
            return 0x1000

        def numel(self):
            return 263168

    class FakeNm:
        @staticmethod
        def spmm_variant(R, C, B, N, M):
            return f"routed<{R},{C},{B},{N},{M}>"

        @staticmethod
        def spmm_ws_variant(R, C, B, N, M):
            return f"ws<{R},{C},{B},{N},{M}>"

    L2 = dict(R=1024, C=8192, N=2, M=4, ws=FakeWs())
    L8 = dict(R=1024, C=4096, N=8, M=16, ws=FakeWs())
    Ln = dict(R=4096, C=4096, N=2, M=4, ws=None)
    assert bench.ws_args(L2, 1) == ()
    assert bench.ws_args(L2, 8) == (0x1000, 263168)
    assert bench.ws_args(Ln, 8) == (None, 0)
    assert bench.batch_kernel_name(FakeNm, L2, 8) == "ws<1024,8192,8,2,4>"
    assert bench.batch_kernel_name(FakeNm, L8, 12) == "ws<1024,4096,12,8,16>"
    assert bench.batch_kernel_name(FakeNm, Ln, 8) == "routed<4096,4096,8,2,4>"


def test_prefill_summary_and_parity_gate():
    """The default line's prefill object keeps the prefill line's headline fields, roofline
    and per-layer figures; a failed parity record inside it (or inside a batch summary)
    fails the whole line."""
    import bench
    full = {"value": 600.0, "unit": "TFLOP/s", "ms_per_step": 0.47, "speedup_vs_dense": 1.5,
            "speedup_vs_best_dense_per_layer_sum": 1.2, "dense_equiv_TFLOPs": 1200.0,
            "config": {"workload": "w", "tokens": 2048},
            "roofline": {"kernel": "k", "achieved": 700.0, "peak": 2500.0, "frac": 0.28, "traffic": None,
                         "bound": "mfma"},
            "per_layer": [{"layer": "q", "kernel": "k", "us": 50.0, "useful_TFLOPs": 600.0, "dense_us": 70.0,
                           "torch_mm_us": 80.0, "speedup_vs_best_dense": 1.4, "extra": 1}],
            "cpu_baseline": {"sample": "s", "parity_vs_gpu": {"max_err_over_bound": 0.05, "rel_l2": 2e-4,
                                                              "ok": True}}}
    out = bench.prefill_summary(full)
    assert out["value"] == 600.0 and out["roofline"]["frac"] == 0.28 and out["config"] == "w"
    assert out["per_layer"] == [{"layer": "q", "kernel": "k", "us": 50.0, "useful_TFLOPs": 600.0, "dense_us": 70.0,
                                 "torch_mm_us": 80.0, "speedup_vs_best_dense": 1.4}]
    assert out["parity_vs_gpu"]["ok"] is True and out["parity_vs_gpu"]["rows"] == "s"
    line = {"value": 1.0, "prefill": out, "batch_products": [{"batch": 8, "parity_vs_gpu": {"ok": True}}]}
    assert bench.parity_failures(line) == []
    line["batch_products"][0]["parity_vs_gpu"]["ok"] = False
    assert bench.parity_failures(line) == ["batch_products[0].parity_vs_gpu"]
