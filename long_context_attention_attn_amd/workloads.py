"""Workload table and seeded synthetic input generators.

This module holds shapes and random numbers only: none of the attention
arithmetic.  Both the HIP path (tests, bench) and the fp64 oracle are fed from
it, so it is the only code the two sides share.

The five workloads are Llama-3-like multi-head / grouped-query attention
shapes at batch 1 and 16 with long contexts, the kind of workload the
Silicon & Systems digest of Mercury describes in "What Mercury finds that
templates miss"; each is one rank's share of a shifted schedule (Q shard of
rank ``i``, KV buffer in ``J`` chunks visited in order ``(j + i) % J``).

Input recipe (a reading; the pages fix no distribution): every (tensor, batch,
head) slice is drawn from its own seeded generator, seed
``(workload << 40) + (tensor << 32) + (batch << 16) + head`` with tensor
Q=0, K=1, V=2; values are N(0, 1) float32 times ``std``; in the heavy-row
workload a seeded choice of ``round(heavy_frac * Skv)`` K rows per (batch, KV
head) (seed tensor id 3) is multiplied by ``heavy_mult`` in float32; finally
the tensor is rounded to the workload dtype (round-to-nearest-even for bf16).
The per-slice seeds let a sampled check regenerate one slice on its own.  The
random stream depends on the device the generator runs on; a parity check
always feeds the oracle the very tensors the GPU saw.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "BY_NAME", "slice_seed", "gen_qkv", "make_inputs",
           "GemmWorkload", "GEMM_WORKLOADS", "GEMM_BY_NAME", "gen_gemm", "make_gemm_inputs"]


@dataclass(frozen=True)
class Workload:
    """One attention call: shapes, chunking, rank, masking and input recipe."""

    index: int
    name: str
    dtype: str  # "f32" or "bf16": Q/K/V element type
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_q: int
    q_pos0: int
    seq_kv: int
    num_chunks: int
    rank: int
    causal: bool
    std: float = 1.0
    heavy_frac: float = 0.0
    heavy_mult: float = 1.0
    summary: str = field(default="", compare=False)

    @property
    def chunk_len(self) -> int:
        return self.seq_kv // self.num_chunks

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def visit_order(self):
        return [(j + self.rank) % self.num_chunks for j in range(self.num_chunks)]

    def visible_pairs_per_head(self) -> int:
        """Unmasked (query, key) pairs of one (batch, query head)."""
        if not self.causal:
            return self.seq_q * self.seq_kv
        total = 0
        # Row t sees keys 0 .. q_pos0 + t, capped at the KV length.
        first = self.q_pos0 + 1
        last = self.q_pos0 + self.seq_q
        full_from = max(first, self.seq_kv)  # rows at or past the KV end
        lo, hi = first, min(last, self.seq_kv - 1)
        if hi >= lo:
            total += (lo + hi) * (hi - lo + 1) // 2
        if last >= full_from:
            total += (last - full_from + 1) * self.seq_kv
        return total

    def flops(self) -> int:
        """Algorithmic flops: 4 * D per unmasked pair (QK^T and PV)."""
        return 4 * self.head_dim * self.batch * self.heads_q * self.visible_pairs_per_head()

    def visible_kv_rows(self) -> int:
        """KV rows that at least one query of the shard can see."""
        if not self.causal:
            return self.seq_kv
        return min(self.seq_kv, self.q_pos0 + self.seq_q)

    def min_bytes(self) -> int:
        """Q + visible K/V + O + LSE, in bytes (O in the input dtype)."""
        el = 4 if self.dtype == "f32" else 2
        q = self.batch * self.heads_q * self.seq_q * self.head_dim * el
        kv = 2 * self.batch * self.heads_kv * self.visible_kv_rows() * self.head_dim * el
        lse = self.batch * self.heads_q * self.seq_q * 4
        return q + kv + q + lse


WORKLOADS = (
    Workload(0, "tiny_gqa_f32", "f32", 1, 8, 2, 128, 1024, 1024, 1024, 4, 1, False,
             summary="Tiny GQA chunked attention, fp32, rank 1 of 4, 4 chunks of 256"),
    Workload(1, "llama3_8b_gqa_32k", "bf16", 1, 32, 8, 128, 4096, 3 * 4096, 32768, 8, 3,
             True, std=0.5,
             summary="Llama-3-8B-like GQA, 32K context on 8 ranks, rank 3, causal"),
    Workload(2, "mha_b16_16k", "bf16", 16, 32, 32, 128, 4096, 2 * 4096, 16384, 4, 2, False,
             summary="MHA batch 16, 16K KV in 4 chunks, rank 2, non-causal"),
    Workload(3, "llama3_70b_gqa_512k", "bf16", 1, 64, 8, 128, 2048, 262144, 524288, 64, 32,
             True, std=0.5,
             summary="Llama-3-70B-like GQA, 512K KV in 64 chunks, rank 32, causal"),
    Workload(4, "gqa_b16_128k_heavy", "bf16", 16, 32, 8, 128, 1024, 130048, 131072, 16, 15,
             True, heavy_frac=0.01, heavy_mult=8.0,
             summary="Batch-16 GQA, 128K KV in 16 chunks, rank 15, causal, 1% of K rows x8"),
    # One GPU's share under two other schedules of the same attention.
    # Head-sharded (Ulysses / USP): after the all-to-all each of 8 GPUs holds
    # Hq/8 query heads and Hkv/8 KV heads over the whole sequence (GQA caps
    # the split at Hkv ways), i.e. one chunk, rank 0, positions from 0.
    Workload(5, "llama3_8b_ulysses_32k", "bf16", 1, 4, 1, 128, 32768, 0, 32768, 1, 0, True,
             std=0.5,
             summary="Llama-3-8B-like GQA, 32K context head-sharded over 8 GPUs: "
                     "4 query heads, 1 KV head, whole sequence, causal"),
    # The 2M-token end of the context sweep on 8 GPUs: rank 3's 256K-row Q
    # shard against the 2M-row KV buffer in 8 chunks.
    Workload(6, "llama3_8b_gqa_2m", "bf16", 1, 32, 8, 128, 262144, 3 * 262144, 2097152, 8, 3,
             True, std=0.5,
             summary="Llama-3-8B-like GQA, 2M-token context on 8 ranks, rank 3, causal"),
)

BY_NAME = {w.name: w for w in WORKLOADS}


def slice_seed(workload: int, tensor: int, b: int, h: int) -> int:
    """Seed of one (tensor, batch, head) slice: Q=0, K=1, V=2, heavy rows=3."""
    return (workload << 40) + (tensor << 32) + (b << 16) + h


def _randn(shape, seed: int, device) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def gen_qkv(*, batch: int, heads_q: int, heads_kv: int, seq_q: int, seq_kv: int,
            head_dim: int, dtype: torch.dtype, device="cpu", seed: int = 0,
            std: float = 1.0, heavy_frac: float = 0.0, heavy_mult: float = 1.0):
    """Seeded Q [B,Hq,Sq,D], K and V [B,Hkv,Skv,D] in ``dtype`` on ``device``.

    ``seed`` plays the role of the workload index in :func:`slice_seed`.
    """
    dev = torch.device(device)
    q = torch.empty((batch, heads_q, seq_q, head_dim), dtype=dtype, device=dev)
    k = torch.empty((batch, heads_kv, seq_kv, head_dim), dtype=dtype, device=dev)
    v = torch.empty_like(k)
    n_heavy = int(round(heavy_frac * seq_kv))
    for b in range(batch):
        for h in range(heads_q):
            x = _randn((seq_q, head_dim), slice_seed(seed, 0, b, h), dev)
            q[b, h] = (x * std if std != 1.0 else x).to(dtype)
        for h in range(heads_kv):
            x = _randn((seq_kv, head_dim), slice_seed(seed, 1, b, h), dev)
            if std != 1.0:
                x = x * std
            if n_heavy:
                gen = torch.Generator(device="cpu")
                gen.manual_seed(slice_seed(seed, 3, b, h))
                rows = torch.randperm(seq_kv, generator=gen)[:n_heavy].to(dev)
                x[rows] *= heavy_mult
            k[b, h] = x.to(dtype)
            x = _randn((seq_kv, head_dim), slice_seed(seed, 2, b, h), dev)
            v[b, h] = (x * std if std != 1.0 else x).to(dtype)
    return q, k, v


def make_inputs(w: Workload, device="cpu"):
    """Q, K, V of workload ``w`` following the recipe in the module docstring."""
    return gen_qkv(batch=w.batch, heads_q=w.heads_q, heads_kv=w.heads_kv, seq_q=w.seq_q,
                   seq_kv=w.seq_kv, head_dim=w.head_dim, dtype=w.torch_dtype,
                   device=device, seed=w.index, std=w.std, heavy_frac=w.heavy_frac,
                   heavy_mult=w.heavy_mult)


# ---------------------------------------------------------------------------
# Shifted all-gather GEMM: one rank's share of a tensor-parallel projection.
# The activation A [M, K] is sharded by rows over J ranks and gathered; the
# rank's weight shard W [N, K] (column-parallel, out x in) is local; the rank
# consumes A's row chunks in the order (j + rank) % J and computes
# C = A W^T [M, N].  The pages measure this pattern as the all-gather GEMM at
# batch 16 (Silicon & Systems digest of Mercury, "What Mercury finds that
# templates miss").
#
# Input recipe (a reading; the pages give none): A ~ N(0, 1) (activations),
# W ~ N(0, 1) / sqrt(K) (so C ~ N(0, 1)), each drawn in float32 from its own
# seeded generator, seed (workload << 40) + (tensor << 32) + chunk with
# tensor A = 0 (one generator per row chunk), W = 1, then rounded to bf16.
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class GemmWorkload:
    """One shifted all-gather GEMM call: C [M, N] = A [M, K] W [N, K]^T."""

    index: int
    name: str
    m: int
    n: int
    k: int
    num_chunks: int
    rank: int
    summary: str = field(default="", compare=False)

    @property
    def chunk_rows(self) -> int:
        return self.m // self.num_chunks

    def visit_order(self):
        return [(j + self.rank) % self.num_chunks for j in range(self.num_chunks)]

    def flops(self) -> int:
        return 2 * self.m * self.n * self.k

    def min_bytes(self) -> int:
        """A + W read once, C written once (bf16 everywhere)."""
        return 2 * (self.m * self.k + self.n * self.k + self.m * self.n)


GEMM_WORKLOADS = (
    GemmWorkload(100, "gemm_tiny_ragged", 1000, 200, 256, 4, 1,
                 summary="1000 x 256 activation in 4 chunks of 250 rows, 200 outputs: "
                         "ragged against every tile size"),
    GemmWorkload(101, "llama3_8b_tp8_mlp_b16", 32768, 3584, 4096, 8, 3,
                 summary="Llama-3-8B-like MLP gate+up projection, tensor parallel over 8 "
                         "GPUs: batch 16 x 2048 tokens gathered from 8 row chunks, the "
                         "rank's 3584-column weight shard (2 x 14336 / 8), rank 3"),
    GemmWorkload(102, "llama3_8b_tp8_qkv_b16", 32768, 768, 4096, 8, 5,
                 summary="Llama-3-8B-like attention QKV projection, tensor parallel over "
                         "8 GPUs: the same gathered activation, the rank's 768-column "
                         "weight shard ((4096 + 2 x 1024) / 8), rank 5"),
)

GEMM_BY_NAME = {w.name: w for w in GEMM_WORKLOADS}


def gen_gemm(*, m: int, n: int, k: int, num_chunks: int, device="cpu", seed: int = 0):
    """Seeded A [M, K] (one generator per row chunk) and W [N, K], bf16."""
    dev = torch.device(device)
    a = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    clen = -(-m // num_chunks)
    for c in range(num_chunks):
        r0, r1 = c * clen, min(m, (c + 1) * clen)
        if r1 > r0:
            a[r0:r1] = _randn((r1 - r0, k), slice_seed(seed, 0, 0, c), dev).to(torch.bfloat16)
    w = (_randn((n, k), slice_seed(seed, 1, 0, 0), dev) / math.sqrt(k)).to(torch.bfloat16)
    return a, w


def make_gemm_inputs(w: GemmWorkload, device="cpu"):
    return gen_gemm(m=w.m, n=w.n, k=w.k, num_chunks=w.num_chunks, device=device, seed=w.index)
