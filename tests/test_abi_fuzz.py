"""Randomised calls into the C ABI's host-side checks (no GPU).

Thousands of seeded requests go to every entry point: a valid request with
none, one or two of its fields replaced by negative, zero, huge or
overflowing sizes, bad strides, null or misaligned pointers.  Each
call must return one of the four status codes and never crash; a request
the checks let through must satisfy the rules the header states, and, with
no device visible, fails at the launch (SHATTN_EHIP) instead of running.

The calls run in a child process that sees no GPU (HIP_VISIBLE_DEVICES and
ROCR_VISIBLE_DEVICES set to -1), so that even on a machine with a GPU no
request built from fake pointers can reach a kernel.
"""

import json
import os
import subprocess
import sys

import pytest

from long_context_attention_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import ctypes, json, sys
import numpy as np
sys.path.insert(0, sys.argv[1])
from long_context_attention_attn_amd import binding

lib = binding.load_library()
rng = np.random.default_rng(int(sys.argv[2]))
FAKE = 0x10000
S3 = ctypes.c_int64 * 3
SIZES = [-(1 << 62), -7, -1, 0, 1, 2, 3, 4, 7, 8, 16, 64, 100, 128, 255, 256, 1000, 1024,
         4096, 1 << 20, (1 << 31) - 1, 1 << 31, 1 << 40, (1 << 62)]

def pick(values):
    return values[int(rng.integers(len(values)))]

PTRS = [0, FAKE + 2, FAKE + 4, FAKE + 8, FAKE + 16]

out = {"attn": [0, 0, 0, 0], "chunk": [0, 0, 0, 0], "gemm": [0, 0, 0, 0], "merge": [0, 0, 0, 0],
       "violations": []}

def record(kind, st, ok_if_passed, info):
    if st not in (0, 1, 2, 3):
        out["violations"].append((kind, "status", st, info))
        return
    out[kind][st] += 1
    if st in (0, 3) and not ok_if_passed:
        out["violations"].append((kind, "accepted", st, info))

def mutate(base, fields, k):
    # Up to k random fields of a valid request replaced by a random value.
    req = dict(base)
    for _ in range(k):
        name = pick(list(fields))
        req[name] = pick(fields[name])
    return req

STRIDES = [S3(a, b, c) for a, b, c in [(4 * 256 * 128, 256 * 128, 128), (0, 0, 128),
                                        (-128, 128, 128), (1, 1, 129), (0, 0, 1 << 25),
                                        (1 << 62, 1 << 62, 128), (4, 4, 4), (0, 0, 136),
                                        (8, 8, 8), (0, 0, 0)]]
ATTN_BASE = dict(batch=1, heads_q=4, heads_kv=2, head_dim=128, seq_q=256, q_pos0=0, causal=1,
                 scale=0.0, in_dtype=0, out_dtype=0, q_stride=0, k_stride=0, v_stride=0,
                 o_stride=0, total=1024, nch=4, rank=1, kv_len=256, kv_pos0=0,
                 p0=FAKE, p1=FAKE, p2=FAKE, p3=FAKE, p4=FAKE)
ATTN_FIELDS = dict(batch=[-1, 0, 2, 16, (1 << 31) - 1], heads_q=[-1, 0, 3, 8, 64],
                   heads_kv=[-1, 0, 1, 8], head_dim=[-128, 0, 4, 64, 130, 256],
                   seq_q=SIZES, q_pos0=[-1, 5, 1 << 40], causal=[-1, 0, 2],
                   scale=[-1.0, 0.088, float("nan"), float("inf")], in_dtype=[1, 2, -1],
                   out_dtype=[1, 2], q_stride=list(range(len(STRIDES))),
                   k_stride=list(range(len(STRIDES))), v_stride=list(range(len(STRIDES))),
                   o_stride=list(range(len(STRIDES))), total=SIZES, nch=[-1, 0, 1, 3, 8, 64],
                   rank=[-1, 0, 3, 7, 63, 64], kv_len=SIZES, kv_pos0=[-1, 128, 1 << 40],
                   p0=PTRS, p1=PTRS, p2=PTRS, p3=PTRS, p4=PTRS)

def attn_desc(r):
    d = binding.ShattnDesc()
    for name in ("batch", "heads_q", "heads_kv", "head_dim", "seq_q", "q_pos0", "causal",
                 "scale", "in_dtype", "out_dtype"):
        setattr(d, name, r[name])
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        setattr(d, name, STRIDES[r[name]])
    return d

def attn_rules(r, total, nch, rank):
    # What any accepted call must satisfy (a subset of the header's rules).
    if r["batch"] < 0 or r["seq_q"] < 0 or r["heads_q"] <= 0 or r["heads_kv"] <= 0:
        return False
    if r["heads_q"] % r["heads_kv"] or r["head_dim"] != 128 or r["causal"] not in (0, 1):
        return False
    if r["in_dtype"] not in (0, 1) or r["scale"] != r["scale"] or r["scale"] == float("inf"):
        return False
    if nch <= 0 or not (0 <= rank < nch) or total < 0 or total % nch:
        return False
    if r["batch"] == 0 or r["seq_q"] == 0:
        return True
    ptrs = [r["p0"], r["p1"], r["p2"], r["p3"], r["p4"]]
    return all(p != 0 and p % 16 == 0 for p in ptrs[:4]) and ptrs[4] != 0 and ptrs[4] % 4 == 0

for i in range(4000):
    r = mutate(ATTN_BASE, ATTN_FIELDS, i % 3)
    d = attn_desc(r)
    st = lib.attn_shifted_fwd(ctypes.byref(d), r["p0"], r["p1"], r["p2"], r["total"], r["nch"],
                              r["rank"], r["p3"], r["p4"], None)
    record("attn", st, attn_rules(r, r["total"], r["nch"], r["rank"]), r)

for i in range(4000):
    r = mutate(ATTN_BASE, ATTN_FIELDS, i % 3)
    d = attn_desc(r)
    st = lib.attn_chunk_fwd(ctypes.byref(d), r["p0"], r["p1"], r["p2"], r["kv_len"],
                            r["kv_pos0"], r["p3"], r["p4"], None)
    ok = attn_rules(r, 1, 1, 0) and r["kv_len"] >= 0 and r["kv_pos0"] >= 0
    record("chunk", st, ok, r)

GEMM_BASE = dict(m=1024, n=512, k=256, lda=256, ldw=256, ldc=512, out_dtype=0, nch=4, rank=1,
                 a=FAKE, w=FAKE, c=FAKE)
GEMM_FIELDS = dict(m=SIZES, n=SIZES, k=SIZES, lda=SIZES, ldw=SIZES, ldc=SIZES,
                   out_dtype=[1, 2, -1], nch=[-1, 0, 1, 3, 8], rank=[-1, 0, 3, 7, 8],
                   a=PTRS, w=PTRS, c=PTRS)
for i in range(4000):
    r = mutate(GEMM_BASE, GEMM_FIELDS, i % 3)
    g = binding.ShattnGemmDesc()
    for name in ("m", "n", "k", "lda", "ldw", "ldc", "out_dtype"):
        setattr(g, name, r[name])
    st = lib.allgather_gemm_shifted(ctypes.byref(g), r["a"], r["w"], r["c"], r["nch"], r["rank"],
                                    None)
    nch, rank = r["nch"], r["rank"]
    ok = (g.m >= 0 and g.n >= 0 and g.k >= 0 and nch > 0 and 0 <= rank < nch
          and g.out_dtype in (0, 1) and g.m % nch == 0)
    if ok and g.m > 0 and g.n > 0:
        # A and W may be null when K == 0: they are never read.
        used = (r["a"], r["w"], r["c"]) if g.k > 0 else (r["c"],)
        ok = (g.lda >= g.k and g.ldw >= g.k and g.ldc >= g.n and g.k % 64 == 0 and g.n % 8 == 0
              and all(p != 0 and p % 16 == 0 for p in used)
              and all(p % 16 == 0 for p in (r["a"], r["w"])))
    record("gemm", st, ok, r)

# Distinct, far-apart buffers: the two sides of a merge must not alias.
MERGE_BASE = dict(rows=512, hd=128, p0=FAKE, p1=FAKE << 8, p2=FAKE << 12, p3=FAKE << 16)
MERGE_FIELDS = dict(rows=SIZES, hd=[-4, 0, 2, 4, 256, 260], p0=PTRS, p1=PTRS, p2=PTRS, p3=PTRS)
for i in range(3000):
    r = mutate(MERGE_BASE, MERGE_FIELDS, i % 3)
    st = lib.lse_merge(r["rows"], r["hd"], r["p0"], r["p1"], r["p2"], r["p3"], None)
    ptrs = [r["p0"], r["p1"], r["p2"], r["p3"]]
    ok = r["rows"] >= 0 and (r["rows"] == 0 or (r["hd"] % 4 == 0 and 4 <= r["hd"] <= 256
                                                and all(p != 0 for p in ptrs)
                                                and ptrs[0] % 16 == 0 and ptrs[2] % 16 == 0))
    record("merge", st, ok, r)

print(json.dumps(out))
"""


@pytest.mark.parametrize("seed", [1, 2])
def test_random_requests_are_checked_and_never_launch(seed):
    if not os.path.exists(binding.library_path()):
        pytest.skip("libshattn.so not built")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(seed)], capture_output=True,
                         text=True, timeout=600, env=env)
    assert res.returncode == 0, res.stderr[-3000:]
    out = json.loads(res.stdout.strip().splitlines()[-1])
    assert not out["violations"], out["violations"][:5]
    # A third of the requests are valid and reach the launch, which fails
    # with no device; the rest break one or two rules and are refused (or
    # are empty no-ops).
    for kind in ("attn", "chunk", "gemm", "merge"):
        ok, einval, eunsup, ehip = out[kind]
        assert einval > 0 and ehip > 0, (kind, out[kind])
