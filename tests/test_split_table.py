"""Host checks of the lane-shuffle tables of the batch products: the split tables that let
4:8 and 8:16 run on the 2:4 sparse matrix instruction (tests/split_table_check.cpp: every
16-bit mask chunk a 4:8 or 8:16 row can hold) and the expansion table that lets 16:32 run on
the dense matrix instruction (tests/expand_table_check.cpp: every mask byte and window
start). Each check is host code built with hipcc and run here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "semi_structured_sparse_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_split_tables_rebuild_every_mask_chunk(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "split_table_check")
    src = os.path.join(ROOT, "tests", "split_table_check.cpp")
    build = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{CSRC}",
                            src, "-o", exe], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:]
    assert "4:8 chunks 4900, 8:16 chunks 12870, failures 0" in run.stdout


def test_expand_table_places_every_byte_pattern(tmp_path):
    """The 16:32 expansion table: every mask byte, every start of the lane's 8-half window."""
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "expand_table_check")
    src = os.path.join(ROOT, "tests", "expand_table_check.cpp")
    build = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{CSRC}",
                            src, "-o", exe], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:]
    assert "expand bytes 256, cases 3328, failures 0" in run.stdout
