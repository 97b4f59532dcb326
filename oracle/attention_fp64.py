"""Plain fp64 CPU oracle for one rank's share of shifted-chunk attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants); it takes numpy-convertible
arrays and returns numpy fp64 arrays.

What it computes (sources, cited by page and section):

* The local operator is single-device softmax attention: Mercury keeps a
  known-good local attention kernel as a "patch" and schedules around it
  (Silicon & Systems digest of Mercury, section "CommIR makes communication
  transformable"; papers.lqhl.me summary "Mercury (SOSP 2025)", section
  核心方法 / core method), and distributed results are checked numerically
  against single-device attention (digest, section "The tuning bill").  The
  pages never write the formula out, so :func:`attention` is the textbook
  definition: for each query row, ``s_k = scale * q . k_k`` over its visible
  keys, ``O = sum_k softmax(s)_k v_k`` and ``LSE = log sum_k exp(s_k)``.
* Grouped-query attention maps query head ``h`` to KV head ``h // (Hq/Hkv)``
  (GQA is named in the digest, section "The hidden cost of synchronized
  operators"; the contiguous-group reading is ours).
* Causal visibility is inclusive on global positions: key position ``p_k`` is
  visible to query position ``p_q`` iff ``p_k <= p_q``.
* The shift primitive visits KV chunks in the order ``c_j = (j + i) % J``
  (summary, section 核心方法; digest, section "The hidden cost of synchronized
  operators", temporal decoupling).  :func:`shifted_attention` follows that
  order literally: attention of the Q shard against chunk ``c_j`` alone, then
  a log-sum-exp merge of the partial (O, LSE) pair into the running pair.

Conventions where the pages are silent (each is listed with its reasoning in
the design notes): natural-log LSE of the scaled scores; partial outputs are
normalised by their own softmax denominator; a row with no visible key has
``O = 0`` and ``LSE = -inf``, which is the identity of the merge.

Pinned by ``tests/test_oracle.py`` against torch's float64 SDPA (a library
special case), closed forms, invariants and the three required properties.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "attend_rows",
    "attention",
    "attention_rows",
    "lse_merge",
    "chunk_attention",
    "shifted_attention",
    "softmax_weights",
]

# Score-block height: keeps the fp64 score block at <= 256 rows x keys.
_ROW_BLOCK = 256


def _f64(x) -> np.ndarray:
    """Upcast any array-like (numpy, or a CPU torch tensor) to fp64 exactly."""
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _default_scale(head_dim: int, scale) -> float:
    return 1.0 / math.sqrt(head_dim) if scale is None else float(scale)


def attend_rows(q_rows, k_rows, v_rows, q_pos, k_pos, *, causal: bool, scale: float):
    """Softmax attention of ``n`` query rows against ``m`` key/value rows.

    Monolithic (one softmax over every visible key), no chunking, no online
    rescaling.

    Args:
      q_rows: [n, D]; k_rows, v_rows: [m, D].
      q_pos: [n] integer global positions of the query rows.
      k_pos: [m] integer global positions of the key rows.
      causal: if true, key k is visible to query t iff k_pos[k] <= q_pos[t].
      scale: multiplier applied to q . k.

    Returns:
      (O [n, D] fp64, LSE [n] fp64).  Rows with no visible key: O = 0,
      LSE = -inf.
    """
    q = _f64(q_rows)
    k = _f64(k_rows)
    v = _f64(v_rows)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    n, m = q.shape[0], k.shape[0]
    d_v = v.shape[1]
    out = np.zeros((n, d_v), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if n == 0 or m == 0:
        return out, lse
    for r0 in range(0, n, _ROW_BLOCK):
        r1 = min(n, r0 + _ROW_BLOCK)
        qp = q_pos[r0:r1]
        if causal:
            # Only keys visible to at least one row of the block take part.
            keep = k_pos <= qp.max()
            kb, vb, kp = k[keep], v[keep], k_pos[keep]
        else:
            kb, vb, kp = k, v, k_pos
        if kb.shape[0] == 0:
            continue
        s = scale * (q[r0:r1] @ kb.T)  # [rows, keys]
        if causal:
            s = np.where(kp[None, :] <= qp[:, None], s, -np.inf)
        m_row = s.max(axis=1)
        empty = m_row == -np.inf
        m_safe = np.where(empty, 0.0, m_row)
        p = np.exp(s - m_safe[:, None])  # masked entries give exp(-inf) = 0
        l_row = p.sum(axis=1)
        if np.isfinite(vb).all():
            o_blk = p @ vb
        else:
            # Sum over each row's visible keys only, so that a non-finite
            # value row reaches exactly the queries that see it (a masked
            # weight of 0 times NaN would otherwise leak it).
            o_blk = np.stack([p[i, p_vis] @ vb[p_vis] for i, p_vis in
                              enumerate(np.isfinite(s))]) if len(s) else p @ vb
        with np.errstate(invalid="ignore", divide="ignore"):
            o_blk = np.where(empty[:, None], 0.0, o_blk / l_row[:, None])
            lse_blk = np.where(empty, -np.inf, m_safe + np.log(l_row))
        out[r0:r1] = o_blk
        lse[r0:r1] = lse_blk
    return out, lse


def softmax_weights(q_rows, k_rows, q_pos, k_pos, *, causal: bool, scale: float):
    """The normalised attention weights [n, m] of :func:`attend_rows` (for the
    rows-sum-to-one property); masked entries are 0, empty rows all 0."""
    q = _f64(q_rows)
    k = _f64(k_rows)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    s = scale * (q @ k.T)
    if causal:
        s = np.where(k_pos[None, :] <= q_pos[:, None], s, -np.inf)
    m_row = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    m_safe = np.where(m_row == -np.inf, 0.0, m_row)
    p = np.exp(s - m_safe[:, None])
    l_row = p.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(l_row[:, None] > 0, p / l_row[:, None], 0.0)


def attention(q, k, v, *, causal: bool = False, q_pos0: int = 0, kv_pos0: int = 0,
              scale=None):
    """Monolithic attention of a Q shard against a KV buffer.

    Args:
      q: [B, Hq, Sq, D]; k, v: [B, Hkv, Skv, D] (any float dtype; upcast to
        fp64, which is exact for bf16 and fp32).
      causal: inclusive causal mask on global positions.
      q_pos0: global position of Q row 0; kv_pos0: global position of K/V
        row 0.
      scale: score multiplier, default 1/sqrt(D).

    Returns:
      (O [B, Hq, Sq, D], LSE [B, Hq, Sq]) in fp64.
    """
    q64 = _f64(q)
    bsz, hq, sq, dim = q64.shape
    hkv, skv = k.shape[1], k.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    sc = _default_scale(dim, scale)
    q_pos = q_pos0 + np.arange(sq, dtype=np.int64)
    k_pos = kv_pos0 + np.arange(skv, dtype=np.int64)
    out = np.zeros((bsz, hq, sq, v.shape[3]), dtype=np.float64)
    lse = np.full((bsz, hq, sq), -np.inf, dtype=np.float64)
    for b in range(bsz):
        for hk in range(hkv):
            k64 = _f64(k[b, hk])
            v64 = _f64(v[b, hk])
            for h in range(hk * group, (hk + 1) * group):
                out[b, h], lse[b, h] = attend_rows(q64[b, h], k64, v64, q_pos, k_pos,
                                                   causal=causal, scale=sc)
    return out, lse


def attention_rows(q, k, v, b: int, h: int, rows, *, causal: bool = False,
                   q_pos0: int = 0, kv_pos0: int = 0, scale=None):
    """:func:`attention` for selected Q rows of one (batch, query head) only.

    Used for sampled parity at sizes where the full oracle would take too long.
    Returns (O [len(rows), D], LSE [len(rows)]).
    """
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    rows = np.asarray(rows, dtype=np.int64)
    dim = q.shape[3]
    q_rows = _f64(q[b, h])[rows]
    n_keys = k.shape[2]
    if causal and len(rows):
        # Keys after the last sampled query are invisible to every sampled row;
        # leaving them out changes nothing and saves the fp64 upcast.
        n_keys = int(min(n_keys, max(0, q_pos0 + rows.max() - kv_pos0 + 1)))
    k64 = _f64(k[b, h // group][:n_keys])
    v64 = _f64(v[b, h // group][:n_keys])
    k_pos = kv_pos0 + np.arange(n_keys, dtype=np.int64)
    return attend_rows(q_rows, k64, v64, q_pos0 + rows, k_pos, causal=causal,
                       scale=_default_scale(dim, scale))


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two partial results over disjoint key sets.

    ``L = M + log(exp(L_a - M) + exp(L_b - M))`` with ``M = max(L_a, L_b)``,
    ``O = exp(L_a - L) O_a + exp(L_b - L) O_b``; two empty rows (both LSE
    -inf) stay empty (O = 0, LSE = -inf).  Softmax over a disjoint union of
    key sets decomposes exactly this way; the pages only say that partial
    outputs and LSEs are merged.
    """
    o_a, lse_a, o_b, lse_b = (_f64(x) for x in (o_a, lse_a, o_b, lse_b))
    mx = np.maximum(lse_a, lse_b)
    both_empty = mx == -np.inf
    mx_safe = np.where(both_empty, 0.0, mx)
    wa = np.exp(lse_a - mx_safe)
    wb = np.exp(lse_b - mx_safe)
    tot = wa + wb
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = np.where(both_empty, -np.inf, mx_safe + np.log(tot))
        ca = np.where(both_empty, 0.0, wa / tot)
        cb = np.where(both_empty, 0.0, wb / tot)
    out = ca[..., None] * o_a + cb[..., None] * o_b
    return out, lse


def chunk_attention(q, k_chunk, v_chunk, *, kv_pos0: int, causal: bool = False,
                    q_pos0: int = 0, scale=None):
    """Partial (O, LSE) of the Q shard against one KV chunk whose row 0 sits at
    global position ``kv_pos0``; rows with no visible key in the chunk get
    O = 0, LSE = -inf."""
    return attention(q, k_chunk, v_chunk, causal=causal, q_pos0=q_pos0,
                     kv_pos0=kv_pos0, scale=scale)


def shifted_attention(q, k, v, *, num_chunks: int, rank: int, causal: bool = False,
                      q_pos0: int = 0, scale=None, order=None):
    """One rank's shifted-chunk attention.

    The KV buffer (global positions ``0 .. Skv-1``) is split into ``J =
    num_chunks`` equal chunks; chunk ``c`` holds positions ``[c*C, (c+1)*C)``.
    Rank ``i = rank`` visits ``c_j = (j + i) % J`` for ``j = 0 .. J-1``,
    computes that chunk's partial (O, LSE) and merges it into the running
    pair.  ``order`` overrides the visit order (for the order-invariance
    property).
    """
    skv = k.shape[2]
    if skv % num_chunks:
        raise ValueError("KV length must be a multiple of the chunk count")
    clen = skv // num_chunks
    bsz, hq, sq, _ = q.shape
    visit = [(j + rank) % num_chunks for j in range(num_chunks)] if order is None else list(order)
    out = np.zeros((bsz, hq, sq, v.shape[3]), dtype=np.float64)
    lse = np.full((bsz, hq, sq), -np.inf, dtype=np.float64)
    for c in visit:
        sl = slice(c * clen, (c + 1) * clen)
        o_c, lse_c = chunk_attention(q, k[:, :, sl], v[:, :, sl], kv_pos0=c * clen,
                                     causal=causal, q_pos0=q_pos0, scale=scale)
        out, lse = lse_merge(out, lse, o_c, lse_c)
    return out, lse
