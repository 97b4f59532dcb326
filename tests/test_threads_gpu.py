"""Concurrent first calls from several host threads.

The library keeps one per-device value (the compute-unit count that sizes the
persistent grid), filled on first use.  A fresh process makes its very first
``attn_shifted_fwd`` calls from 4 threads at once, each on its own stream and
its own inputs, and every result is compared with the oracle.
"""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, threading
import numpy as np
import torch
sys.path.insert(0, ROOT)
import oracle
from long_context_attention_attn_amd import binding
from long_context_attention_attn_amd.workloads import gen_qkv

dev = torch.device("cuda", 0)
cases = [(1, 4, 2, 300, 1024, 4, 1, True, 500), (2, 4, 4, 130, 512, 2, 0, False, 0),
         (1, 8, 2, 520, 2048, 8, 5, True, 1600), (1, 2, 1, 64, 256, 1, 0, True, 192)]
inputs = [gen_qkv(batch=c[0], heads_q=c[1], heads_kv=c[2], seq_q=c[3], seq_kv=c[4],
                  head_dim=128, dtype=torch.bfloat16, device=dev, seed=60 + i)
          for i, c in enumerate(cases)]
streams = [torch.cuda.Stream(dev) for _ in cases]
torch.cuda.synchronize()
start = threading.Barrier(len(cases))
results = [None] * len(cases)
errors = []

def run(i):
    try:
        c = cases[i]
        q, k, v = inputs[i]
        with torch.cuda.stream(streams[i]):
            start.wait()
            o, lse = binding.attn_shifted_fwd(q, k, v, num_chunks=c[5], rank=c[6], causal=c[7],
                                              q_pos0=c[8], out_dtype=torch.float32)
        streams[i].synchronize()
        results[i] = (o.cpu(), lse.cpu())
    except Exception as e:  # reported by the parent
        errors.append(repr(e))

threads = [threading.Thread(target=run, args=(i,)) for i in range(len(cases))]
for t in threads:
    t.start()
for t in threads:
    t.join()
assert not errors, errors
for i, c in enumerate(cases):
    q, k, v = inputs[i]
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), causal=c[7], q_pos0=c[8])
    eo = float(np.max(np.abs(results[i][0].numpy() - o_ref)))
    el = float(np.max(np.abs(results[i][1].numpy() - lse_ref)))
    print("thread", i, c, "max |dO|", eo, "max |dLSE|", el, flush=True)
    assert eo <= 2e-2 and el <= 1e-3, (i, eo, el)
print("THREADS_OK", flush=True)
""".replace("ROOT", repr(ROOT))


def test_first_calls_from_four_threads():
    res = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True,
                         timeout=110, cwd=ROOT)
    print(res.stdout)
    print(res.stderr[-2000:])
    assert res.returncode == 0 and "THREADS_OK" in res.stdout
