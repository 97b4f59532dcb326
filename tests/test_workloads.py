"""The workload table and the seeded input generator (CPU only)."""

import numpy as np
import pytest
import torch

from long_context_attention_attn_amd.workloads import BY_NAME, WORKLOADS, gen_qkv, slice_seed


def _pairs_brute(w):
    t = np.arange(w.seq_q, dtype=np.int64)
    if not w.causal:
        return w.seq_q * w.seq_kv
    return int(np.minimum(w.q_pos0 + t + 1, w.seq_kv).clip(min=0).sum())


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_visible_pairs_closed_form_matches_count(w):
    assert w.visible_pairs_per_head() == _pairs_brute(w)
    assert w.seq_kv % w.num_chunks == 0
    assert w.heads_q % w.heads_kv == 0
    assert 0 <= w.rank < w.num_chunks
    assert sorted(w.visit_order()) == list(range(w.num_chunks))
    assert w.visit_order()[0] == w.rank


def test_table_shapes():
    shapes = [(w.dtype, w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seq_q, w.seq_kv,
               w.num_chunks, w.rank, w.causal) for w in WORKLOADS]
    assert shapes == [
        ("f32", 1, 8, 2, 128, 1024, 1024, 4, 1, False),
        ("bf16", 1, 32, 8, 128, 4096, 32768, 8, 3, True),
        ("bf16", 16, 32, 32, 128, 4096, 16384, 4, 2, False),
        ("bf16", 1, 64, 8, 128, 2048, 524288, 64, 32, True),
        ("bf16", 16, 32, 8, 128, 1024, 131072, 16, 15, True),
        ("bf16", 1, 4, 1, 128, 32768, 32768, 1, 0, True),
        ("bf16", 1, 32, 8, 128, 262144, 2097152, 8, 3, True),
    ]
    # Q shards sit at rank * Sq on the global axis for the causal workloads.
    assert BY_NAME["llama3_8b_gqa_32k"].q_pos0 == 3 * 4096
    assert BY_NAME["llama3_70b_gqa_512k"].q_pos0 == 262144
    assert BY_NAME["gqa_b16_128k_heavy"].q_pos0 == 131072 - 1024
    assert BY_NAME["llama3_8b_ulysses_32k"].q_pos0 == 0
    assert BY_NAME["llama3_8b_gqa_2m"].q_pos0 == 3 * 262144
    # Head-sharded 8 ways, the 32K model does 1/8 of the full causal attention
    # of its 32 query heads per GPU.
    w = BY_NAME["llama3_8b_ulysses_32k"]
    assert w.flops() * 8 == 4 * 128 * 32 * (32768 * 32769 // 2)
    # Algorithmic flops of the headline workload (4 * D * B * Hq * pairs).
    assert BY_NAME["llama3_8b_gqa_32k"].flops() == 4 * 128 * 32 * 58_722_304


def test_generator_is_deterministic_and_slice_seeded():
    kw = dict(batch=2, heads_q=4, heads_kv=2, seq_q=8, seq_kv=16, head_dim=8,
              dtype=torch.bfloat16, seed=7)
    a = gen_qkv(**kw)
    b = gen_qkv(**kw)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # One slice can be regenerated alone from its seed.
    g = torch.Generator().manual_seed(slice_seed(7, 1, 1, 0))
    k10 = torch.randn((16, 8), generator=g).to(torch.bfloat16)
    assert torch.equal(a[1][1, 0], k10)
    assert a[0].dtype == torch.bfloat16 and a[0].shape == (2, 4, 8, 8)


def test_heavy_rows():
    q, k, v = gen_qkv(batch=1, heads_q=2, heads_kv=1, seq_q=4, seq_kv=1000, head_dim=16,
                      dtype=torch.float32, seed=4, heavy_frac=0.01, heavy_mult=8.0)
    g = torch.Generator().manual_seed(slice_seed(4, 1, 0, 0))
    base = torch.randn((1000, 16), generator=g)
    ratio = (k[0, 0] / base)
    heavy = (ratio - 8.0).abs().amax(dim=1) < 1e-6
    plain = (ratio - 1.0).abs().amax(dim=1) < 1e-6
    assert int(heavy.sum()) == 10 and bool((heavy | plain).all())


def test_gemm_table_and_generator():
    from long_context_attention_attn_amd.workloads import GEMM_BY_NAME, GEMM_WORKLOADS, gen_gemm

    for w in GEMM_WORKLOADS:
        assert w.m % w.num_chunks == 0 and 0 <= w.rank < w.num_chunks
        assert w.k % 64 == 0 and w.n % 8 == 0  # what the kernel supports
        assert sorted(w.visit_order()) == list(range(w.num_chunks))
        assert w.visit_order()[0] == w.rank
        assert w.flops() == 2 * w.m * w.n * w.k
    big = GEMM_BY_NAME["llama3_8b_tp8_mlp_b16"]
    assert (big.m, big.n, big.k, big.num_chunks) == (16 * 2048, 2 * 14336 // 8, 4096, 8)
    qkv = GEMM_BY_NAME["llama3_8b_tp8_qkv_b16"]
    assert qkv.n == (4096 + 2 * 1024) // 8
    # Deterministic; each row chunk of A comes from its own generator, so one
    # chunk can be regenerated alone; W is scaled by 1/sqrt(K).
    a1, w1 = gen_gemm(m=12, n=8, k=64, num_chunks=3, seed=5)
    a2, w2 = gen_gemm(m=12, n=8, k=64, num_chunks=3, seed=5)
    assert torch.equal(a1, a2) and torch.equal(w1, w2)
    g = torch.Generator().manual_seed(slice_seed(5, 0, 0, 1))
    assert torch.equal(a1[4:8], torch.randn((4, 64), generator=g).to(torch.bfloat16))
    g = torch.Generator().manual_seed(slice_seed(5, 1, 0, 0))
    assert torch.equal(w1, (torch.randn((8, 64), generator=g) / 8.0).to(torch.bfloat16))
    assert a1.dtype == torch.bfloat16 and w1.shape == (8, 64)
