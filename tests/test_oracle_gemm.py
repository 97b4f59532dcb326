"""Pins of the fp64 shifted all-gather GEMM oracle against things other than
itself.

Each pin is chosen so that a plausible slip (a missing transpose of W, a
swapped operand, a wrong chunk size or row offset, a visit order that is not
(j + i) % J, a chunk written to the wrong rows) fails at least one of them:

* torch's float64 ``matmul`` of A with W transposed (a library routine);
* a scalar triple loop on tiny shapes;
* hand-derived products in ``tests/golden/gemm_closed_forms.json``;
* closed forms: one-hot rows of A select columns of W^T, W of ones gives
  row sums of A, the identity W returns A;
* the shift: the visit order is (j + i) % J, every chunk order gives the
  same C, and each row block depends on its own chunk of A only.
"""

import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gemm_closed_forms.json")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (7, 5, 3), (64, 33, 128), (130, 70, 96)])
def test_matches_torch_matmul_float64(m, n, k):
    a, w = _rand((m, k), 1), _rand((n, k), 2)
    ref = torch.matmul(torch.from_numpy(a), torch.from_numpy(w).T).numpy()
    np.testing.assert_allclose(oracle.gemm(a, w), ref, atol=1e-12, rtol=0)


def test_scalar_triple_loop():
    m, n, k = 4, 3, 5
    a, w = _rand((m, k), 3), _rand((n, k), 4)
    ref = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            s = 0.0
            for p in range(k):
                s += a[i, p] * w[j, p]
            ref[i, j] = s
    np.testing.assert_allclose(oracle.gemm(a, w), ref, atol=1e-13, rtol=0)


def test_golden_closed_forms():
    cases = json.load(open(GOLDEN))["cases"]
    assert cases
    for c in cases:
        got = oracle.gemm(np.array(c["a"], float), np.array(c["w"], float))
        np.testing.assert_array_equal(got, np.array(c["c"], float), err_msg=c["name"])


def test_closed_forms():
    k, n = 16, 6
    w = _rand((n, k), 5)
    # One-hot rows: row i of A selects column k_i of W^T, i.e. W[:, k_i].
    picks = [0, 3, 15, 7]
    a = np.zeros((len(picks), k))
    a[np.arange(len(picks)), picks] = 1.0
    np.testing.assert_array_equal(oracle.gemm(a, w), w[:, picks].T)
    # W of ones: every column of C is the row sum of A.
    a2 = _rand((5, k), 6)
    np.testing.assert_allclose(oracle.gemm(a2, np.ones((3, k))),
                               np.repeat(a2.sum(axis=1, keepdims=True), 3, axis=1),
                               atol=1e-13, rtol=0)
    # The identity W (N = K) returns A.
    np.testing.assert_array_equal(oracle.gemm(a2, np.eye(k)), a2)


@pytest.mark.parametrize("j_total", [1, 2, 4, 8])
def test_shift_visit_order_and_order_invariance(j_total):
    m, n, k = 8 * j_total, 5, 12
    a, w = _rand((m, k), 7), _rand((n, k), 8)
    full = oracle.gemm(a, w)
    for rank in range(j_total):
        visit = []
        c = oracle.shifted_allgather_gemm(a, w, num_chunks=j_total, rank=rank, visit=visit)
        assert visit == [(j + rank) % j_total for j in range(j_total)]
        np.testing.assert_array_equal(c, full)
    perms = itertools.permutations(range(j_total)) if j_total <= 4 else \
        [np.random.default_rng(9).permutation(j_total) for _ in range(6)]
    for order in perms:
        np.testing.assert_array_equal(
            oracle.shifted_allgather_gemm(a, w, num_chunks=j_total, rank=0, order=order), full)


def test_row_block_depends_on_its_chunk_only():
    j_total, clen, n, k = 4, 6, 5, 9
    a, w = _rand((j_total * clen, k), 10), _rand((n, k), 11)
    c0 = oracle.shifted_allgather_gemm(a, w, num_chunks=j_total, rank=2)
    a2 = a.copy()
    a2[clen:2 * clen] += 100.0  # perturb chunk 1 only
    c1 = oracle.shifted_allgather_gemm(a2, w, num_chunks=j_total, rank=2)
    rows = np.arange(j_total * clen)
    same = (rows < clen) | (rows >= 2 * clen)
    np.testing.assert_array_equal(c0[same], c1[same])
    assert not np.allclose(c0[~same], c1[~same])


def test_rows_helper_matches_full():
    a, w = _rand((40, 24), 12), _rand((9, 24), 13)
    rows = np.array([0, 5, 39, 17])
    np.testing.assert_array_equal(oracle.gemm_rows(a, w, rows), oracle.gemm(a, w)[rows])


def test_bf16_inputs_upcast_exactly():
    a = torch.randn(6, 10, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    w = torch.randn(4, 10, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    ref = torch.matmul(a.double(), w.double().T).numpy()
    np.testing.assert_allclose(oracle.gemm(a, w), ref, atol=1e-12, rtol=0)
