"""CPU oracle for the batch-one N:M semi-structured sparse matrix-vector product
(and its small-batch counterpart, the product with B activation vectors).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package. It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing) and it
never imports it; the only code both sides use is the seeded input generator
in ``synth``.

See ``oracle/nm_oracle.py`` for the functions and the passages of the pages
each one follows.
"""
from .nm_oracle import (  # noqa: F401
    PATTERNS,
    PATTERNS_QUARTER,
    SUPPORTED_PATTERNS,
    magnitude_key,
    keep_ref,
    prune_ref,
    pack_ref,
    unpack_ref,
    spmv_ref,
    gemv_ref,
    spmm_ref,
    gemm_ref,
    exact_ref,
    fp16_rne,
    y_tolerance_report,
    y_within_tolerance,
)
