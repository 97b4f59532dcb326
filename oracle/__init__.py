"""fp64 CPU oracle for shifted-chunk attention and the shifted all-gather
GEMM (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library.
"""

from .attention_fp64 import (  # noqa: F401
    attend_rows,
    attention,
    attention_rows,
    chunk_attention,
    lse_merge,
    shifted_attention,
    softmax_weights,
)
from .gemm_fp64 import gemm, gemm_rows, shifted_allgather_gemm  # noqa: F401
