"""Plain fp64 CPU oracle for one rank's share of a shifted all-gather GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; it takes numpy-convertible arrays and returns numpy fp64 arrays.

What it computes (sources, cited by page and section):

* The operator is a tensor-parallel matrix product in which every rank owns
  a slice of one operand and all ranks need the whole of it: a conventional
  schedule replicates the shared operand (all-gather) and runs identical loop
  nests, Mercury keeps it sharded and shifts the order in which each rank
  consumes its pieces (Silicon & Systems digest of Mercury, section "The
  hidden cost of synchronized operators"); the pages measure it as the
  all-gather GEMM (digest, section "What Mercury finds that templates
  miss").  The shift primitive visits pieces in the order ``(j + i) % J``
  (papers.lqhl.me summary "Mercury (SOSP 2025)", section 核心方法), and the
  local product is a known-good GEMM kept as a "patch" (digest, section
  "CommIR makes communication transformable").
* Reading taken (the pages give no layout): the gathered operand is the
  activation ``A`` [M, K], sharded by rows over ``J`` ranks (chunk ``c`` is
  rows ``[c*M/J, (c+1)*M/J)``); the rank's local weight shard is ``W``
  [N, K] (a column-parallel linear layer, stored out_features x
  in_features); the product is ``C = A W^T`` [M, N].  Rank ``i`` visits
  chunk ``c_j = (j + i) % J`` for ``j = 0..J-1`` and writes C's row block
  of that chunk.  The row blocks are disjoint, so the visit order decides
  when each block is produced, never its value.

Pinned by ``tests/test_oracle_gemm.py`` against torch's float64 matmul (a
library routine), a scalar triple loop, hand-derived values in
``tests/golden/gemm_closed_forms.json`` and closed-form cases.
"""

from __future__ import annotations

import numpy as np

__all__ = ["gemm", "gemm_rows", "shifted_allgather_gemm"]


def _f64(x) -> np.ndarray:
    """Upcast any array-like (numpy, or a CPU torch tensor) to fp64 exactly."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def gemm(a, w):
    """``C = A W^T`` in fp64: ``C[m, n] = sum_k A[m, k] W[n, k]``.

    Args:
      a: [M, K]; w: [N, K] (any float dtype; bf16 and fp32 upcast exactly).
    Returns:
      C [M, N], fp64.
    """
    a64 = _f64(a)
    w64 = _f64(w)
    if a64.shape[1] != w64.shape[1]:
        raise ValueError("A and W must share the contraction length K")
    return a64 @ w64.T


def gemm_rows(a, w, rows):
    """:func:`gemm` for selected rows of A only (for sampled checks)."""
    rows = np.asarray(rows, dtype=np.int64)
    return _f64(a)[rows] @ _f64(w).T


def shifted_allgather_gemm(a, w, *, num_chunks: int, rank: int, order=None, visit=None):
    """One rank's share of the shifted all-gather GEMM.

    The gathered A (all ``J = num_chunks`` row chunks, ``M`` a multiple of
    ``J``) is consumed chunk by chunk in the order ``c_j = (j + rank) % J``;
    chunk ``c``'s product with ``W^T`` fills C's rows ``[c*M/J, (c+1)*M/J)``.
    ``order`` overrides the visit order (for the order-invariance property);
    ``visit``, if given, is a list the visited chunk indices are appended to.
    """
    a64 = _f64(a)
    w64 = _f64(w)
    m = a64.shape[0]
    if m % num_chunks:
        raise ValueError("M must be a multiple of the chunk count")
    clen = m // num_chunks
    seq = [(j + rank) % num_chunks for j in range(num_chunks)] if order is None else list(order)
    c = np.zeros((m, w64.shape[0]), dtype=np.float64)
    for ch in seq:
        if visit is not None:
            visit.append(ch)
        rows = slice(ch * clen, (ch + 1) * clen)
        c[rows] = a64[rows] @ w64.T
    return c
