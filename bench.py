#!/usr/bin/env python3
"""Throughput of one rank's shifted-chunk attention on one MI355X.

A step is one fused ``attn_shifted_fwd`` launch over the 32K-context GQA rank
shard (Llama-3-8B-like: batch 1, 32 query heads, 8 KV heads, head_dim 128, Q
shard of 4096 rows at global offset 12288, KV of 32768 rows in 8 chunks
visited in order (j + 3) % 8, causal), inputs resident in HBM.  Prints ONE
JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Only one GPU is used: ``--gpus`` above 1 exits with a message.

Extra modes (measurement plumbing, no effect on the default line):
  --calib-copy-mib M   after the timed region, run one plain device copy of
                       M MiB so a hardware-counter run sees a kernel of known
                       traffic next to the attention kernel;
  --summarize-pmc FETCH_CSV WRITE_CSV OUT
                       turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE and
                       WRITE_SIZE runs of this script with the copy) into the
                       traffic summary read back by later runs.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 4096 bf16 flop/clk x 2.4 GHz (AMD's "2.5 PFLOP/s" dense)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# The kernel that dominates each kind of workload: its source (whose hash
# tags a traffic summary) and the name prefix rocprofv3 reports for it.
KERNELS = {
    "attn": ("long_context_attention_attn_amd/csrc/attn_fwd_bf16.hip", "attn_fwd"),
    "attn_f32": ("long_context_attention_attn_amd/csrc/attn_fwd_f32.hip", "attn_fwd_f32"),
    "gemm": ("long_context_attention_attn_amd/csrc/gemm_bf16.hip", "gemm_bf16"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "{prefix}_{workload}_traffic.json")
# torch's negation kernel serves as the calibration copy: it reads and writes
# each element once.
CALIB_KERNEL = "neg_kernel"
METRIC = "attention TFLOP/s per MI355X + % bf16 MFMA peak, 32K-ctx GQA rank shard"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_kind(workload: str) -> str:
    from long_context_attention_attn_amd.workloads import BY_NAME, GEMM_BY_NAME

    if workload in GEMM_BY_NAME:
        return "gemm"
    wl = BY_NAME.get(workload)
    return "attn_f32" if wl is not None and wl.dtype == "f32" else "attn"


def kernel_hash(kind: str = "attn") -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, KERNELS[kind][0]), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was taken on a different kernel source."""
    kind = kernel_kind(workload)
    path = TRAFFIC_FILE.format(prefix=KERNELS[kind][1], workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != kernel_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def _blas_info():
    """Vendor, version and thread count of the BLAS numpy uses."""
    try:
        from threadpoolctl import threadpool_info

        for p in threadpool_info():
            if p.get("user_api") == "blas":
                return {"vendor": p.get("internal_api"), "version": p.get("version"),
                        "threads": p.get("num_threads")}
    except Exception:  # pragma: no cover
        pass
    return {"vendor": None, "version": None, "threads": None}


def cpu_baseline(w, q, k, v, budget_s: float):
    """The fp64 oracle on the host, over whole (batch, head) slices of the
    same workload until ``budget_s`` seconds of oracle time have passed.

    The BLAS pool is set to every core this process may run on.  Moving a
    slice to the host and upcasting it to fp64 is timed apart from the
    oracle call, which then receives fp64 arrays."""
    import numpy as np
    import oracle

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits

        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = None
    group = w.heads_q // w.heads_kv
    done_flops = 0
    slices = 0
    elapsed = 0.0
    prep = 0.0
    nk = w.visible_kv_rows()
    rows = np.arange(w.seq_q)
    kv_cache = {}
    for b in range(w.batch):
        for h in range(w.heads_q):
            hk = h // group
            t0 = time.perf_counter()
            if (b, hk) not in kv_cache:
                kv_cache.clear()
                kv_cache[(b, hk)] = (k[b, hk, :nk].cpu().double().numpy()[None, None],
                                     v[b, hk, :nk].cpu().double().numpy()[None, None])
            ks, vs = kv_cache[(b, hk)]
            qs = q[b, h].cpu().double().numpy()[None, None]
            t1 = time.perf_counter()
            oracle.attention_rows(qs, ks, vs, 0, 0, rows, causal=w.causal, q_pos0=w.q_pos0)
            t2 = time.perf_counter()
            prep += t1 - t0
            elapsed += t2 - t1
            done_flops += 4 * w.head_dim * w.visible_pairs_per_head()
            slices += 1
            if elapsed >= budget_s:
                break
        else:
            continue
        break
    blas = _blas_info()
    if limiter is not None:
        limiter.restore_original_limits()
    return {
        "value": done_flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{slices} of {w.batch * w.heads_q} (batch, query-head) slices, every row, "
                  f"fp64 numpy; oracle {elapsed:.1f} s, host copy + fp64 upcast {prep:.1f} s "
                  "(not in the rate)",
        "blas": blas,
        "oracle_s": round(elapsed, 2),
        "upcast_s": round(prep, 2),
    }


def summarize_pmc(fetch_dir: str, write_dir: str, out: str, workload: str, copy_mib: int):
    """HBM bytes per launch of the attention kernel from two rocprofv3 --pmc
    runs of this script with --calib-copy-mib (FETCH_SIZE, then WRITE_SIZE).

    rocprofv3 writes one CSV row per counter instance; a dispatch's value is
    the sum of its rows (KiB).  The attention kernel's mean per dispatch is
    scaled by bytes / reading of the calibration kernel, which reads and
    writes exactly ``copy_mib`` MiB."""
    import glob

    def per_dispatch(root, counter, needle):
        sums = {}
        for path in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter or needle not in row.get("Kernel_Name", ""):
                        continue
                    key = (path, row["Dispatch_Id"])
                    sums[key] = sums.get(key, 0.0) + float(row["Counter_Value"])
        if not sums:
            raise SystemExit(f"no {counter} rows for a kernel matching {needle!r} under {root}")
        return sum(sums.values()) / len(sums) * 1024.0, len(sums)

    kind = kernel_kind(workload)
    prefix = KERNELS[kind][1]
    f_attn, n_fa = per_dispatch(fetch_dir, "FETCH_SIZE", prefix)
    w_attn, n_wa = per_dispatch(write_dir, "WRITE_SIZE", prefix)
    f_copy, _ = per_dispatch(fetch_dir, "FETCH_SIZE", CALIB_KERNEL)
    w_copy, _ = per_dispatch(write_dir, "WRITE_SIZE", CALIB_KERNEL)
    copy_bytes = copy_mib * 2**20
    f_scale = copy_bytes / f_copy
    w_scale = copy_bytes / w_copy
    rec = {
        "workload": workload,
        "kernel": prefix,
        "kernel_sha": kernel_hash(kind),
        "dispatches": [n_fa, n_wa],
        "fetch_bytes_raw": f_attn,
        "write_bytes_raw": w_attn,
        "copy_bytes": copy_bytes,
        "copy_fetch_raw": f_copy,
        "copy_write_raw": w_copy,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_bytes_per_launch": f_attn * f_scale + w_attn * w_scale,
    }
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def overlap_report(w, q, k, v, steps: int, warmup: int):
    """One JSON line on the overlapped chunk walk: apart from the rank's own
    chunk, K/V start in pinned host memory (standing in for the peers that
    hold the chunks) and each chunk is copied in while the chunks before it
    compute, each chunk's partial merged in its kernel.  Timed beside it on
    the same stream: the same chunk walk with K/V already in HBM, the fused
    one-launch walk, and a plain host-to-device copy of the same bytes."""
    import torch

    from long_context_attention_attn_amd import binding

    dev = q.device
    stream = torch.cuda.current_stream(dev)
    log("bench: pinned host copies of K and V")
    k_src = torch.empty(k.shape, dtype=k.dtype, pin_memory=True)
    k_src.copy_(k)
    v_src = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
    v_src.copy_(v)
    k_dev, v_dev = torch.empty_like(k), torch.empty_like(v)
    own = slice(w.rank * w.chunk_len, (w.rank + 1) * w.chunk_len)
    k_dev[:, :, own] = k[:, :, own]
    v_dev[:, :, own] = v[:, :, own]
    copy_stream = torch.cuda.Stream(dev)
    clen = w.chunk_len
    q_last = w.q_pos0 + w.seq_q - 1
    seen = [c for c in w.visit_order() if not w.causal or c * clen <= q_last]
    o = torch.empty((w.batch, w.heads_q, w.seq_q, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.heads_q, w.seq_q), dtype=torch.float32, device=dev)
    es = k.element_size()
    fetched = [c for c in seen if c != w.rank]
    nbytes = 2 * w.batch * w.heads_kv * len(fetched) * clen * w.head_dim * es
    h_buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d_buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def overlapped():
        binding.attn_shifted_fwd_overlapped(q, k_src, v_src, k_dev, v_dev,
                                            num_chunks=w.num_chunks, rank=w.rank,
                                            causal=w.causal, q_pos0=w.q_pos0,
                                            copy_stream=copy_stream)

    def resident():
        for j, c in enumerate(seen):
            sl = slice(c * clen, (c + 1) * clen)
            if j == 0:
                binding.attn_chunk_fwd(q, k[:, :, sl], v[:, :, sl], kv_pos0=c * clen,
                                       causal=w.causal, q_pos0=w.q_pos0, o_part=o, lse_part=lse)
            else:
                binding.attn_chunk_fwd_accumulate(q, k[:, :, sl], v[:, :, sl], o, lse,
                                                  kv_pos0=c * clen, causal=w.causal,
                                                  q_pos0=w.q_pos0)

    def fused():
        binding.attn_shifted_fwd(q, k, v, num_chunks=w.num_chunks, rank=w.rank, causal=w.causal,
                                 q_pos0=w.q_pos0, out=o, lse=lse)

    def transfer():
        d_buf.copy_(h_buf, non_blocking=True)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / max(steps, 1)

    log("bench: overlapped walk")
    ms_ov = timed(overlapped)
    log("bench: resident walk")
    ms_res = timed(resident)
    log("bench: transfer only")
    ms_tr = timed(transfer)
    log("bench: fused walk (one launch)")
    ms_fused = timed(fused)
    shorter = min(ms_res, ms_tr)
    hidden = (ms_res + ms_tr - ms_ov) / shorter if nbytes and shorter > 0 else None
    rec = {
        "metric": "overlapped chunk walk with K/V arriving from pinned host memory",
        "workload": w.name,
        "steps": steps,
        "warmup": warmup,
        "chunks_computed": len(seen),
        "chunks_fetched": len(fetched),
        "bytes_fetched": nbytes,
        "ms_overlapped": round(ms_ov, 4),
        "ms_compute_resident": round(ms_res, 4),
        "ms_fused_resident": round(ms_fused, 4),
        "ms_transfer_only": round(ms_tr, 4),
        "transfer_GBps": round(nbytes / (ms_tr * 1e-3) / 1e9, 2) if nbytes else None,
        "tflops_overlapped": round(w.flops() / (ms_ov * 1e-3) / 1e12, 3),
        "hidden_fraction_of_shorter_phase": None if hidden is None else round(hidden, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def merge_report(w, steps: int, warmup: int):
    """One JSON line on lse_merge alone, over the workload's rows (B*Hq*Sq
    rows of head_dim fp32): HBM-bound, priced against 8 TB/s with its
    algorithmic bytes (read O_a, O_b and two LSEs, write O and one LSE)."""
    import torch

    from long_context_attention_attn_amd import binding

    dev = torch.device("cuda", 0)
    rows = w.batch * w.heads_q * w.seq_q
    gen = torch.Generator(device=dev).manual_seed(5)
    o_a = torch.randn((rows, w.head_dim), generator=gen, device=dev)
    o_b = torch.randn((rows, w.head_dim), generator=gen, device=dev)
    l_a = torch.randn(rows, generator=gen, device=dev)
    l_b = torch.randn(rows, generator=gen, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        binding.lse_merge(o_a, l_a, o_b, l_b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        binding.lse_merge(o_a, l_a, o_b, l_b)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(steps, 1)
    nbytes = rows * (3 * w.head_dim * 4 + 3 * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "lse_merge HBM throughput", "workload": w.name, "rows": rows,
        "head_dim": w.head_dim, "steps": steps, "warmup": warmup, "ms_per_merge": round(ms, 5),
        "bytes_per_merge": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)},
    }), flush=True)
    return 0


def calibration_copy(mib: int, dev):
    """One launch of the calibration kernel (torch's negation) over ``mib``
    MiB of fp32: it reads and writes each byte once, which fixes the scale
    of the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.empty(mib * 2**20 // 4, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def gemm_report(wl, steps: int, warmup: int, cpu_seconds: float, no_cpu: bool,
                calib_copy_mib: int = 0):
    """One JSON line for the shifted all-gather GEMM workload ``wl``: C = A W^T
    with A's row chunks visited from chunk ``rank`` on, inputs resident.
    Beside it, torch's own bf16 matmul of the same operands (the vendor
    library) is timed on the same stream, as context."""
    import numpy as np
    import torch

    import oracle
    from long_context_attention_attn_amd import binding
    from long_context_attention_attn_amd.workloads import make_gemm_inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"bench: gemm workload {wl.name}: generating inputs")
    a, w = make_gemm_inputs(wl, dev)
    c = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.allgather_gemm_shifted(a, w, num_chunks=wl.num_chunks, rank=wl.rank, out=c)

    def timed(fn, n_warm, n_steps):
        for _ in range(n_warm):
            fn()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
        for i in range(n_steps):
            evs[i].record(stream)
            fn()
        evs[-1].record(stream)
        torch.cuda.synchronize()
        per = sorted(x.elapsed_time(y) for x, y in zip(evs[:-1], evs[1:]))
        return evs[0].elapsed_time(evs[-1]) / max(n_steps, 1), per

    log(f"bench: warmup {warmup}, timing {steps} steps")
    ms, per = timed(step, warmup, steps)
    flops = wl.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"bench: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s")
    if calib_copy_mib:
        calibration_copy(calib_copy_mib, dev)
    wt = w.t()
    ms_lib, _ = timed(lambda: torch.matmul(a, wt, out=c), max(3, warmup // 5), max(5, steps // 2))
    rec = {
        "metric": "shifted all-gather GEMM TFLOP/s per MI355X + % bf16 MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": wl.name, "m": wl.m, "n": wl.n, "k": wl.k,
                   "num_chunks": wl.num_chunks, "rank": wl.rank,
                   "algorithmic_gflop": round(flops / 1e9, 3),
                   "parallelism": "one rank's share on 1 GPU"},
        "launch_ms": {"mean": round(ms, 5), "median": round(per[len(per) // 2], 5),
                      "min": round(per[0], 5), "max": round(per[-1], 5)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(wl.name)},
        "context": {"torch_matmul_ms": round(ms_lib, 5),
                    "torch_matmul_tflops": round(flops / (ms_lib * 1e-3) / 1e12, 1)},
    }
    if not no_cpu:
        log(f"bench: cpu baseline (fp64 oracle, ~{cpu_seconds:.0f} s)")
        cores = len(os.sched_getaffinity(0))
        try:
            from threadpoolctl import threadpool_limits

            limiter = threadpool_limits(limits=cores)
        except Exception:  # pragma: no cover
            limiter = None
        w64 = w.cpu().double().numpy()
        rows_done, elapsed, prep = 0, 0.0, 0.0
        block = 1024
        while elapsed < cpu_seconds and rows_done < wl.m:
            r1 = min(wl.m, rows_done + block)
            t0 = time.perf_counter()
            a64 = a[rows_done:r1].cpu().double().numpy()
            t1 = time.perf_counter()
            oracle.gemm(a64, w64)
            t2 = time.perf_counter()
            prep += t1 - t0
            elapsed += t2 - t1
            rows_done = r1
        blas = _blas_info()
        if limiter is not None:
            limiter.restore_original_limits()
        rec["cpu_baseline"] = {
            "value": 2 * rows_done * wl.n * wl.k / elapsed / 1e12,
            "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows_done} of {wl.m} rows of A, fp64 numpy; oracle {elapsed:.1f} s, "
                      f"host copy + fp64 upcast {prep:.1f} s (not in the rate)",
            "blas": blas, "oracle_s": round(elapsed, 2), "upcast_s": round(prep, 2)}
    del np
    print(json.dumps(rec), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The engine clock takes some 50 back-to-back launches of the default
    # workload (~40 ms of load) to settle; the default warm-up covers that.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="llama3_8b_gqa_32k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0)
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    ap.add_argument("--flush-mib", type=int, default=0)
    ap.add_argument("--lse-merge", action="store_true",
                    help="time lse_merge alone over the workload's rows")
    ap.add_argument("--overlap-from-host", action="store_true",
                    help="time the overlapped chunk walk with K/V in pinned host memory")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, workload=args.workload,
                      copy_mib=args.calib_copy_mib or 1024)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU exchange is not part of this library).", file=sys.stderr)
        return 2

    import torch

    from long_context_attention_attn_amd import binding
    from long_context_attention_attn_amd.workloads import BY_NAME, make_inputs

    from long_context_attention_attn_amd.workloads import GEMM_BY_NAME

    if args.workload in GEMM_BY_NAME:
        return gemm_report(GEMM_BY_NAME[args.workload], args.steps, args.warmup,
                           args.cpu_seconds, args.no_cpu_baseline, args.calib_copy_mib)
    w = BY_NAME[args.workload]
    if args.lse_merge:
        return merge_report(w, args.steps, args.warmup)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"bench: workload {w.name}: generating inputs")
    q, k, v = make_inputs(w, dev)
    if args.overlap_from_host:
        return overlap_report(w, q, k, v, args.steps, args.warmup)
    out = torch.empty((w.batch, w.heads_q, w.seq_q, w.head_dim), dtype=q.dtype, device=dev)
    lse = torch.empty((w.batch, w.heads_q, w.seq_q), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        binding.attn_shifted_fwd(q, k, v, num_chunks=w.num_chunks, rank=w.rank,
                                 causal=w.causal, q_pos0=w.q_pos0, out=out, lse=lse)

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The kernel runs on torch's current stream; events on that same stream
    # bracket exactly the K launches.
    stream = torch.cuda.current_stream(dev)
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    if args.flush_mib:
        scratch = torch.empty(args.flush_mib * 2**20 // 4, dtype=torch.float32, device=dev)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            scratch.fill_(float(i))
            starts[i].record(stream)
            step()
            ends[i].record(stream)
        torch.cuda.synchronize()
        per_launch = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
        ms = sum(per_launch) / max(args.steps, 1)
    else:
        # One event before every launch and one after the last: the first and
        # last bracket the K launches (the mean), neighbours give each
        # launch's own time (median and minimum).
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        for i in range(args.steps):
            evs[i].record(stream)
            step()
        evs[-1].record(stream)
        torch.cuda.synchronize()
        ms = evs[0].elapsed_time(evs[-1]) / max(args.steps, 1)
        per_launch = sorted(a.elapsed_time(b) for a, b in zip(evs[:-1], evs[1:]))
    t_wall = time.perf_counter() - t_wall
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"bench: {ms:.4f} ms/step ({t_wall:.3f} s wall), {tflops:.1f} TFLOP/s")

    if args.calib_copy_mib:
        calibration_copy(args.calib_copy_mib, dev)

    is_f32 = w.dtype == "f32"
    peak = PEAK_F32_TFLOPS if is_f32 else PEAK_BF16_TFLOPS
    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if is_f32 else "bf16",
        "data": "synthetic",
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": w.name,
            "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
            "head_dim": w.head_dim, "seq_q": w.seq_q, "q_pos0": w.q_pos0,
            "seq_kv": w.seq_kv, "num_chunks": w.num_chunks, "rank": w.rank,
            "causal": w.causal, "algorithmic_gflop": round(flops / 1e9, 3),
            "parallelism": "one rank's shard on 1 GPU",
            "cache_flush_mib": args.flush_mib,
        },
        "launch_ms": {
            "mean": round(ms, 5),
            "median": round(per_launch[len(per_launch) // 2], 5) if per_launch else None,
            "min": round(per_launch[0], 5) if per_launch else None,
            "max": round(per_launch[-1], 5) if per_launch else None,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": read_traffic(w.name),
        },
    }
    if not args.no_cpu_baseline:
        log(f"bench: cpu baseline (fp64 oracle, ~{args.cpu_seconds:.0f} s)")
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
