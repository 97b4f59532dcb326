"""Pins of the fp64 oracle against things other than itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped scale, an
exclusive instead of inclusive causal bound, a wrong GQA head map, a sign or
index error in the merge, a transposed operand) fails at least one of them:

* torch's float64 ``scaled_dot_product_attention`` (a library routine) and
  ``torch.logsumexp`` for J = 1 (catches scale, mask, GQA map, transposes);
* hand-derived closed forms in ``tests/golden/closed_forms.json``;
* the three required properties: rows of the weights sum to 1, chunked-then-
  merged equals monolithic for every chunk order and shift, and a causal first
  query at position 0 attends only to key 0;
* closed forms and invariants: Q = 0 gives the mean of the visible V rows and
  LSE = log n; constant V rows give that row; GQA equals MHA with repeated KV
  heads; joint K/V row permutations and (Q*c, scale/c) change nothing; merging
  with the empty pair is the identity and a self-merge adds log 2.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from long_context_attention_attn_amd.workloads import gen_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa_reference(q, k, v, *, causal, q_pos0, kv_pos0, scale):
    """torch float64 SDPA (with GQA) plus logsumexp of the masked scores."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    sq, skv = q.shape[2], k.shape[2]
    group = q.shape[1] // k.shape[1]
    mask = None
    if causal:
        qp = q_pos0 + torch.arange(sq)
        kp = kv_pos0 + torch.arange(skv)
        mask = kp[None, :] <= qp[:, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                       enable_gqa=group > 1)
    kr = kt.repeat_interleave(group, dim=1)
    s = scale * torch.matmul(qt, kr.transpose(-1, -2))
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("causal,q_pos0", [(False, 0), (True, 0), (True, 7), (True, 29)])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (6, 3), (8, 1)])
def test_matches_torch_sdpa_float64(causal, q_pos0, hq, hkv):
    b, sq, skv, d = 2, 13, 37, 16
    q = _rand((b, hq, sq, d), 1)
    k = _rand((b, hkv, skv, d), 2)
    v = _rand((b, hkv, skv, d), 3)
    scale = 0.37
    o, lse = oracle.attention(q, k, v, causal=causal, q_pos0=q_pos0, scale=scale)
    o_ref, lse_ref = _sdpa_reference(q, k, v, causal=causal, q_pos0=q_pos0, kv_pos0=0,
                                     scale=scale)
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_default_scale_is_inverse_sqrt_head_dim():
    q, k, v = _rand((1, 2, 5, 128), 4), _rand((1, 2, 9, 128), 5), _rand((1, 2, 9, 128), 6)
    o, lse = oracle.attention(q, k, v)
    o_ref, lse_ref = _sdpa_reference(q, k, v, causal=False, q_pos0=0, kv_pos0=0,
                                     scale=1 / math.sqrt(128))
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_golden_closed_forms():
    cases = json.load(open(GOLDEN))["cases"]
    assert cases
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, None]
        v = np.array(c["v"], dtype=np.float64)[None, None]
        o, lse = oracle.attention(q, k, v, causal=c["causal"], q_pos0=c["q_pos0"],
                                  kv_pos0=c["kv_pos0"], scale=c["scale"])
        lse_exp = np.array([float(x) for x in c["lse"]])
        np.testing.assert_allclose(o[0, 0], np.array(c["o"]), atol=1e-14, rtol=0,
                                   err_msg=c["name"])
        np.testing.assert_array_equal(np.isinf(lse[0, 0]), np.isinf(lse_exp), err_msg=c["name"])
        fin = np.isfinite(lse_exp)
        np.testing.assert_allclose(lse[0, 0][fin], lse_exp[fin], atol=1e-14, rtol=0,
                                   err_msg=c["name"])


@pytest.mark.parametrize("causal", [False, True])
def test_property_weights_rows_sum_to_one(causal):
    q, k = _rand((11, 8), 7, 3.0), _rand((19, 8), 8, 3.0)
    qp = 4 + np.arange(11)
    kp = np.arange(19)
    w = oracle.softmax_weights(q, k, qp, kp, causal=causal, scale=0.9)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert (w >= 0).all()
    if causal:
        assert (w[kp[None, :] > qp[:, None]] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_weights_are_the_weights_attention_uses(causal):
    """Binds the rows-sum-to-one property to the oracle's own attention:

    * the weights equal torch's float64 softmax of the masked, scaled scores
      (a library routine; a dropped or wrong scale fails here);
    * they equal exp(scale q.k - LSE) with LSE from :func:`oracle.attention`;
    * W @ V equals :func:`oracle.attention`'s O for a V of full column rank
      (19 keys, head_dim 32), which fixes W uniquely: they are exactly the
      weights the monolithic attention applies, and those rows sum to 1.
    """
    n, m, d, scale = 11, 19, 32, 0.37
    q, k, v = _rand((n, d), 21, 2.0), _rand((m, d), 22, 2.0), _rand((m, d), 23)
    qp = 6 + np.arange(n)
    kp = np.arange(m)
    w = oracle.softmax_weights(q, k, qp, kp, causal=causal, scale=scale)
    s = torch.from_numpy(scale * (q @ k.T))
    if causal:
        s = s.masked_fill(torch.from_numpy(kp[None, :] > qp[:, None]), float("-inf"))
    np.testing.assert_allclose(w, torch.softmax(s, dim=1).numpy(), atol=1e-14, rtol=0)
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], causal=causal,
                              q_pos0=int(qp[0]), scale=scale)
    w_lse = np.exp(scale * (q @ k.T) - lse[0, 0][:, None])
    if causal:
        w_lse = np.where(kp[None, :] <= qp[:, None], w_lse, 0.0)
    np.testing.assert_allclose(w, w_lse, atol=1e-13, rtol=0)
    assert np.linalg.matrix_rank(v) == m
    np.testing.assert_allclose(w @ v, o[0, 0], atol=1e-12, rtol=0)
    # The weights recovered from attention's own output sum to one per row.
    w_attn = o[0, 0] @ np.linalg.pinv(v)
    np.testing.assert_allclose(w_attn.sum(axis=1), 1.0, atol=1e-10, rtol=0)


def _merge_case(causal, q_pos0, skv=24, hq=4, hkv=2, seed=10):
    q = _rand((2, hq, 9, 8), seed, 2.0)
    k = _rand((2, hkv, skv, 8), seed + 1, 2.0)
    v = _rand((2, hkv, skv, 8), seed + 2)
    return q, k, v


@pytest.mark.parametrize("causal,q_pos0", [(False, 0), (True, 0), (True, 11), (True, 20)])
def test_property_chunked_merge_equals_monolithic_all_orders(causal, q_pos0):
    q, k, v = _merge_case(causal, q_pos0)
    o_ref, lse_ref = oracle.attention(q, k, v, causal=causal, q_pos0=q_pos0, scale=0.5)
    for nch in (1, 2, 3, 4):
        for order in itertools.permutations(range(nch)):
            o, lse = oracle.shifted_attention(q, k, v, num_chunks=nch, rank=0, causal=causal,
                                              q_pos0=q_pos0, scale=0.5, order=order)
            np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal,q_pos0", [(False, 0), (True, 3), (True, 15)])
def test_property_chunked_merge_equals_monolithic_every_shift(causal, q_pos0):
    q, k, v = _merge_case(causal, q_pos0, skv=48)
    o_ref, lse_ref = oracle.attention(q, k, v, causal=causal, q_pos0=q_pos0, scale=0.5)
    for nch in (1, 2, 3, 4, 6, 8, 12, 16, 24, 48):  # every divisor of 48
        ranks = range(nch) if nch in (2, 4, 8) else (0, nch - 1)
        for rank in ranks:
            o, lse = oracle.shifted_attention(q, k, v, num_chunks=nch, rank=rank,
                                              causal=causal, q_pos0=q_pos0, scale=0.5)
            np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_shift_order_is_j_plus_i_mod_J(monkeypatch):
    """Rank i visits chunk (j + i) % J at step j: record the chunk positions."""
    import oracle.attention_fp64 as mod

    seen = []
    orig = mod.chunk_attention

    def spy(q, kc, vc, *, kv_pos0, **kw):
        seen.append(kv_pos0)
        return orig(q, kc, vc, kv_pos0=kv_pos0, **kw)

    monkeypatch.setattr(mod, "chunk_attention", spy)
    q, k, v = _merge_case(False, 0, skv=40)
    mod.shifted_attention(q, k, v, num_chunks=5, rank=3)
    assert seen == [8 * c for c in (3, 4, 0, 1, 2)]


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 1), (4, 4)])
def test_property_causal_first_query_attends_only_key0(hq, hkv):
    q, k, v = _rand((1, hq, 6, 16), 20), _rand((1, hkv, 10, 16), 21), _rand((1, hkv, 10, 16), 22)
    scale = 0.25
    o, lse = oracle.attention(q, k, v, causal=True, q_pos0=0, scale=scale)
    grp = hq // hkv
    for h in range(hq):
        np.testing.assert_array_equal(o[0, h, 0], v[0, h // grp, 0])
        assert lse[0, h, 0] == pytest.approx(scale * q[0, h, 0] @ k[0, h // grp, 0], abs=1e-14)
    # Rows are unchanged when keys/values after their position are altered.
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 4:] = 1e3
    v2[:, :, 4:] = -1e3
    o2, lse2 = oracle.attention(q, k2, v2, causal=True, q_pos0=0, scale=scale)
    np.testing.assert_array_equal(o2[:, :, :4], o[:, :, :4])
    np.testing.assert_array_equal(lse2[:, :, :4], lse[:, :, :4])
    assert not np.allclose(o2[:, :, 4:], o[:, :, 4:])


@pytest.mark.parametrize("causal,q_pos0", [(False, 0), (True, 12288 - 1000)])
def test_closed_form_zero_query(causal, q_pos0):
    sq, skv = 7, 12000
    q = np.zeros((1, 2, sq, 8))
    k, v = _rand((1, 1, skv, 8), 30), _rand((1, 1, skv, 8), 31)
    o, lse = oracle.attention(q, k, v, causal=causal, q_pos0=q_pos0)
    for t in range(sq):
        n = min(skv, q_pos0 + t + 1) if causal else skv
        np.testing.assert_allclose(o[0, :, t], np.broadcast_to(v[0, 0, :n].mean(axis=0), (2, 8)),
                                   atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[0, :, t], math.log(n), atol=1e-13, rtol=0)


def test_closed_form_constant_values():
    q, k = _rand((1, 2, 5, 8), 40, 4.0), _rand((1, 2, 30, 8), 41, 4.0)
    u = _rand((8,), 42)
    v = np.broadcast_to(u, (1, 2, 30, 8)).copy()
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, causal=causal, q_pos0=3)
        np.testing.assert_allclose(o, np.broadcast_to(u, o.shape), atol=1e-13, rtol=0)


def test_reduction_gqa_equals_mha_with_repeated_heads():
    q = _rand((2, 8, 5, 8), 50)
    k, v = _rand((2, 2, 12, 8), 51), _rand((2, 2, 12, 8), 52)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal=causal, q_pos0=4)
        o2, lse2 = oracle.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                    causal=causal, q_pos0=4)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, lse2)
        # Head h must not use KV head h % Hkv: that map gives a different answer.
        perm = [0, 1] * 4
        o3, _ = oracle.attention(q, k[:, perm], v[:, perm], causal=causal, q_pos0=4)
        o4, _ = oracle.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                 causal=causal, q_pos0=4)
        assert not np.allclose(o3, o4)


def test_invariants_permutation_and_scale():
    q, k, v = _rand((1, 2, 6, 8), 60), _rand((1, 2, 15, 8), 61), _rand((1, 2, 15, 8), 62)
    o, lse = oracle.attention(q, k, v, scale=0.3)
    perm = np.random.default_rng(63).permutation(15)
    o2, lse2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], scale=0.3)
    np.testing.assert_allclose(o2, o, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-13, rtol=0)
    o3, lse3 = oracle.attention(q * 4.0, k, v, scale=0.3 / 4.0)
    np.testing.assert_allclose(o3, o, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse3, lse, atol=1e-13, rtol=0)


def test_merge_identity_and_self_merge():
    o, lse = _rand((3, 4, 8), 70), _rand((3, 4), 71)
    empty_o, empty_l = np.zeros_like(o), np.full_like(lse, -np.inf)
    for a, b in (((empty_o, empty_l), (o, lse)), ((o, lse), (empty_o, empty_l))):
        om, lm = oracle.lse_merge(*a, *b)
        np.testing.assert_array_equal(om, o)
        np.testing.assert_array_equal(lm, lse)
    om, lm = oracle.lse_merge(o, lse, o, lse)
    np.testing.assert_allclose(om, o, atol=1e-15, rtol=0)
    np.testing.assert_allclose(lm, lse + math.log(2.0), atol=1e-14, rtol=0)
    om, lm = oracle.lse_merge(empty_o, empty_l, empty_o, empty_l)
    assert (om == 0).all() and (lm == -np.inf).all()
    # Unequal weights: closed form for LSEs 0 and log 3 (weights 1/4, 3/4).
    oa, ob = np.array([[4.0, 0.0]]), np.array([[0.0, 4.0]])
    om, lm = oracle.lse_merge(oa, np.array([0.0]), ob, np.array([math.log(3.0)]))
    np.testing.assert_allclose(om, [[1.0, 3.0]], atol=1e-15, rtol=0)
    np.testing.assert_allclose(lm, [math.log(4.0)], atol=1e-15, rtol=0)


def test_masked_chunk_is_empty():
    q, k, v = _rand((1, 2, 4, 8), 80), _rand((1, 1, 6, 8), 81), _rand((1, 1, 6, 8), 82)
    o, lse = oracle.chunk_attention(q, k, v, kv_pos0=100, causal=True, q_pos0=10)
    assert (o == 0).all() and (lse == -np.inf).all()


def test_sampled_rows_match_full():
    q, k, v = gen_qkv(batch=2, heads_q=4, heads_kv=2, seq_q=40, seq_kv=70, head_dim=16,
                      dtype=torch.bfloat16, seed=3)
    o, lse = oracle.attention(q, k, v, causal=True, q_pos0=30)
    rows = [0, 7, 39]
    o_r, lse_r = oracle.attention_rows(q, k, v, 1, 3, rows, causal=True, q_pos0=30)
    np.testing.assert_array_equal(o_r, o[1, 3, rows])
    np.testing.assert_array_equal(lse_r, lse[1, 3, rows])


def test_scalar_loop_tiny():
    """A scalar ``math.exp`` loop agrees with the vectorised oracle on tiny
    shapes (catches broadcasting/axis slips in the numpy code)."""
    for causal, q_pos0, hq, hkv in itertools.product((False, True), (0, 3), (1, 2), (1,)):
        sq, skv, d = 4, 8, 4
        q, k, v = _rand((1, hq, sq, d), 90), _rand((1, hkv, skv, d), 91), _rand((1, hkv, skv, d), 92)
        o, lse = oracle.attention(q, k, v, causal=causal, q_pos0=q_pos0, scale=0.7)
        for h in range(hq):
            for t in range(sq):
                keys = [j for j in range(skv) if not causal or j <= q_pos0 + t]
                sc = [0.7 * sum(q[0, h, t, x] * k[0, 0, j, x] for x in range(d)) for j in keys]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = sum(w)
                for x in range(d):
                    ref = sum(wi * v[0, 0, j, x] for wi, j in zip(w, keys)) / tot
                    assert abs(o[0, h, t, x] - ref) <= 1e-12
                assert abs(lse[0, h, t] - (mx + math.log(tot))) <= 1e-12


def test_nonfinite_value_reaches_only_rows_that_see_it():
    q, k, v = _rand((1, 1, 8, 4), 95), _rand((1, 1, 8, 4), 96), _rand((1, 1, 8, 4), 97)
    v[0, 0, 5, 2] = np.nan
    o, lse = oracle.attention(q, k, v, causal=True, q_pos0=0)
    assert np.isfinite(o[0, 0, :5]).all()
    assert np.isnan(o[0, 0, 5:, 2]).all() and np.isfinite(np.delete(o[0, 0, 5:], 2, axis=1)).all()
    assert np.isfinite(lse).all()
