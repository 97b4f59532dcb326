"""GPU parity of every bf16 workload at its full size, in the launch
configuration the benchmark times (one fused ``attn_shifted_fwd`` launch),
against the fp64 oracle.

Coverage per workload:

* ``llama3_8b_gqa_32k`` and ``llama3_8b_ulysses_32k``: every element of the
  output and every LSE (the oracle finishes them in seconds);
* ``mha_b16_16k``, ``llama3_70b_gqa_512k``, ``gqa_b16_128k_heavy``: every
  (batch, query head), one row from every 32-row query block at an offset
  that varies with the block and the head (so every work item, wave and
  query block is checked, and across heads every position inside a block),
  on every fourth head the rows at work-item (256) and wave (64) edges, and
  every row of two heads;
* ``llama3_8b_gqa_2m`` (10 GiB of inputs, millions of keys per row): rows at
  the item and wave edges plus random rows of 4 heads.

Each launch runs twice, with bf16 and with fp32 output; the bf16 output must
equal the fp32 output rounded to bf16 bit for bit, and both are compared
with the oracle (bf16 O within 2e-2, LSE within 1e-3).  The largest errors
are printed and, when ``SHATTN_PARITY_LOG`` names a file, appended to it as
one JSON line per workload.
"""

import json
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from long_context_attention_attn_amd import binding
from long_context_attention_attn_amd.workloads import BY_NAME

pytestmark = pytest.mark.gpu

TOL_O = 2e-2
TOL_LSE = 1e-3
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _record(rec):
    _say("parity " + json.dumps(rec))
    path = os.environ.get("SHATTN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def edge_rows(sq):
    """Rows at work-item (256-row) and wave (64-row) edges, the shard's ends."""
    cand = {0, 1, sq // 2, sq - 1}
    for base in (64, 256):
        for e in range(base, sq, base):
            if e % 1024 == 0 or e < 1024 or e >= sq - 1024:
                cand.update((e - 1, e))
    return sorted(r for r in cand if 0 <= r < sq)


def block_rows(sq, salt):
    """One row from every 32-row query block, at offset (5 i + salt) mod 32."""
    i = np.arange((sq + 31) // 32)
    return np.minimum(32 * i + (5 * i + salt) % 32, sq - 1)


def _launch(w, q, k, v, out_dtype):
    o, lse = binding.attn_shifted_fwd(q, k, v, num_chunks=w.num_chunks, rank=w.rank,
                                      causal=w.causal, q_pos0=w.q_pos0, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse


def _errors(o_rows, lse_rows, o_ref, lse_ref):
    """Max |dO| and |dLSE| of one slice's rows; the empty-row pattern must match."""
    g = o_rows.astype(np.float64)
    eo = float(np.max(np.abs(g - o_ref))) if g.size else 0.0
    gl = lse_rows.astype(np.float64)
    assert np.array_equal(np.isneginf(gl), np.isneginf(lse_ref)), "empty-row pattern differs"
    fin = np.isfinite(lse_ref)
    el = float(np.max(np.abs(gl[fin] - lse_ref[fin]))) if fin.any() else 0.0
    return eo, el


def check_rows(w, q, k, v, o16, o32, lse, rows_for, deadline_s=None):
    """Compares selected rows of every (batch, query head) with the oracle.

    ``rows_for(b, h)`` gives the rows of slice (b, h) (None: skip it).  K/V of
    each (batch, KV head) are upcast once for the heads of its group; only
    keys some query of the shard can see are taken.  Returns
    (max |dO| bf16 out, max |dO| fp32 out, max |dLSE|, rows checked)."""
    group = w.heads_q // w.heads_kv
    nk = w.visible_kv_rows()
    k_pos = np.arange(nk, dtype=np.int64)
    e16 = e32 = el = 0.0
    n_rows = 0
    t0 = time.perf_counter()
    for b in range(w.batch):
        for hk in range(w.heads_kv):
            heads = [(h, rows_for(b, h)) for h in range(hk * group, (hk + 1) * group)]
            heads = [(h, r) for h, r in heads if r is not None and len(r)]
            if not heads:
                continue
            k64 = k[b, hk, :nk].cpu().double().numpy()
            v64 = v[b, hk, :nk].cpu().double().numpy()
            for h, rows in heads:
                rows = np.asarray(rows, dtype=np.int64)
                rows_t = torch.from_numpy(rows).to(o16.device)
                q64 = q[b, h].index_select(0, rows_t).cpu().double().numpy()
                o_ref, lse_ref = oracle.attend_rows(q64, k64, v64, w.q_pos0 + rows, k_pos,
                                                    causal=w.causal, scale=w.scale)
                a16 = o16[b, h].index_select(0, rows_t).float().cpu().numpy()
                a32 = o32[b, h].index_select(0, rows_t).cpu().numpy()
                al = lse[b, h].index_select(0, rows_t).cpu().numpy()
                x16, xl = _errors(a16, al, o_ref, lse_ref)
                x32, _ = _errors(a32, al, o_ref, lse_ref)
                e16, e32, el = max(e16, x16), max(e32, x32), max(el, xl)
                n_rows += len(rows)
            if deadline_s is not None and time.perf_counter() - t0 > deadline_s:
                raise AssertionError("oracle comparison ran past its time budget")
    return e16, e32, el, n_rows


def _run_workload(w, rows_for, coverage):
    _say(f"workload {w.name}: generating inputs")
    from long_context_attention_attn_amd.workloads import make_inputs

    q, k, v = make_inputs(w, DEV)
    torch.cuda.synchronize()
    _say(f"workload {w.name}: launching (bf16 and fp32 output)")
    o16, lse = _launch(w, q, k, v, torch.bfloat16)
    o32, lse32 = _launch(w, q, k, v, torch.float32)
    assert torch.isfinite(o32).all() and torch.isfinite(lse).all()
    assert torch.equal(lse32, lse)
    assert torch.equal(o32.to(torch.bfloat16), o16)
    _say(f"workload {w.name}: oracle ({coverage})")
    t0 = time.perf_counter()
    e16, e32, el, n_rows = check_rows(w, q, k, v, o16, o32, lse, rows_for)
    rec = {"workload": w.name, "coverage": coverage, "rows_checked": n_rows,
           "rows_total": w.batch * w.heads_q * w.seq_q,
           "max_abs_dO_bf16_out": e16, "max_abs_dO_f32_out": e32, "max_abs_dLSE": el,
           "tol_O": TOL_O, "tol_LSE": TOL_LSE, "oracle_s": round(time.perf_counter() - t0, 1)}
    _record(rec)
    assert e16 <= TOL_O and e32 <= TOL_O and el <= TOL_LSE, rec
    del q, k, v, o16, o32, lse, lse32
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["llama3_8b_gqa_32k", "llama3_8b_ulysses_32k"])
def test_workload_every_element(name):
    w = BY_NAME[name]
    all_rows = np.arange(w.seq_q)
    _run_workload(w, lambda b, h: all_rows, "every element")


@pytest.mark.parametrize("name", ["mha_b16_16k", "llama3_70b_gqa_512k", "gqa_b16_128k_heavy"])
def test_workload_every_head_every_block(name):
    w = BY_NAME[name]
    full = {(0, 0), (w.batch - 1, w.heads_q - 1)}
    edges = edge_rows(w.seq_q)
    all_rows = np.arange(w.seq_q)

    def rows_for(b, h):
        if (b, h) in full:
            return all_rows
        rows = block_rows(w.seq_q, 7 * b + 3 * h)
        # Item and wave edges on every fourth head (the block rows already
        # reach every block of every head).
        return np.union1d(rows, edges) if (b * w.heads_q + h) % 4 == 0 else rows

    _run_workload(w, rows_for, "every (batch, head): one row per 32-row block; item and "
                  "wave edges on every 4th head; every row of 2 heads")


def test_workload_2m_sampled():
    w = BY_NAME["llama3_8b_gqa_2m"]
    rng = np.random.default_rng(3)
    heads = {(0, 0): None, (0, 11): None, (0, 22): None, (0, w.heads_q - 1): None}
    edges = edge_rows(w.seq_q)
    for key in heads:
        heads[key] = np.union1d(edges, rng.integers(0, w.seq_q, size=24))

    _run_workload(w, lambda b, h: heads.get((b, h)),
                  "4 heads: item and wave edges at the ends, every 1024th row, 24 random rows")
