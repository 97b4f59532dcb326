"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and rejects every malformed call on the host before any HIP call.

No case here reaches a kernel launch: each one breaks at least one rule the
host checks, so it runs the same with or without a GPU.
"""

import ctypes
import os
import re

import pytest

from long_context_attention_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shattn.h")

FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def _lib():
    if not os.path.exists(binding.library_path()):
        pytest.skip("libshattn.so not built")
    return binding.load_library()


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^SHATTN_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)


def test_exports_every_declared_symbol():
    lib = _lib()
    names = _declared_functions()
    assert set(names) == {"attn_chunk_fwd", "attn_chunk_fwd_accumulate", "lse_merge",
                          "attn_shifted_fwd",
                          "attn_shifted_fwd_overlapped", "allgather_gemm_shifted",
                          "attn_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    _lib()
    assert binding.attn_status_string(0) == "SHATTN_OK"
    assert binding.attn_status_string(1) == "SHATTN_EINVAL"
    assert binding.attn_status_string(2) == "SHATTN_EUNSUPPORTED"
    assert binding.attn_status_string(3) == "SHATTN_EHIP"
    assert binding.attn_status_string(77) == "SHATTN_UNKNOWN"


def test_desc_layout_matches_header():
    # int32 x4, int64 x2, int32, float, int32 x2, 4 x int64[3]
    assert ctypes.sizeof(binding.ShattnDesc) == 16 + 16 + 16 + 4 * 24
    assert binding.ShattnDesc.q_stride.offset == 48


def _desc(**over):
    d = binding.ShattnDesc()
    d.batch, d.heads_q, d.heads_kv, d.head_dim = 1, 4, 2, 128
    d.seq_q, d.q_pos0, d.causal, d.scale = 256, 0, 1, 0.0
    d.in_dtype, d.out_dtype = binding.BF16, binding.BF16
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        setattr(d, name, (ctypes.c_int64 * 3)(4 * 256 * 128, 256 * 128, 128))
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _shifted(lib, d, q=FAKE, k=FAKE, v=FAKE, total=1024, nch=4, rank=1, o=FAKE, lse=FAKE):
    return lib.attn_shifted_fwd(ctypes.byref(d) if d is not None else None, q, k, v, total, nch,
                                rank, o, lse, None)


def _chunk(lib, d, q=FAKE, k=FAKE, v=FAKE, kv_len=256, kv_pos0=0, o=FAKE, lse=FAKE):
    return lib.attn_chunk_fwd(ctypes.byref(d) if d is not None else None, q, k, v, kv_len,
                              kv_pos0, o, lse, None)


S3 = ctypes.c_int64 * 3


@pytest.mark.parametrize("case,expect", [
    ({"heads_q": 3}, 1),                # heads_q % heads_kv != 0
    ({"heads_kv": 0}, 1),
    ({"heads_q": 0}, 1),
    ({"batch": -1}, 1),
    ({"head_dim": 64}, 2),              # valid shape, not built
    ({"head_dim": 130}, 1),             # not a multiple of 4
    ({"seq_q": -5}, 1),
    ({"q_pos0": -1}, 1),
    ({"causal": 2}, 1),
    ({"scale": float("nan")}, 1),
    ({"scale": float("inf")}, 1),
    ({"in_dtype": 7}, 1),
    ({"out_dtype": 9}, 1),
    ({"q_stride": S3(1, 1, 129)}, 1),   # row stride not a multiple of 16 bytes
    ({"k_stride": S3(-128, 128, 128)}, 1),
    ({"o_stride": S3(4, 4, 4)}, 1),
    ({"k_stride": S3(0, 0, (1 << 24) + 8)}, 2),   # row stride beyond 2^24 elements
    ({"v_stride": S3(0, 0, (1 << 24) + 8)}, 2),
    ({"q_stride": S3(0, 0, (1 << 24) + 8)}, 2),
    ({"o_stride": S3(0, 0, (1 << 24) + 8)}, 2),
])
def test_shifted_rejects_bad_desc(case, expect):
    lib = _lib()
    assert _shifted(lib, _desc(**case)) == expect


def test_shifted_rejects_bad_arguments():
    lib = _lib()
    d = _desc()
    assert _shifted(lib, None) == 1
    assert _shifted(lib, d, rank=4) == 1          # rank >= num_chunks
    assert _shifted(lib, d, rank=-1) == 1
    assert _shifted(lib, d, nch=0) == 1
    assert _shifted(lib, d, total=1000, nch=3) == 1  # not a multiple
    assert _shifted(lib, d, total=-4) == 1
    assert _shifted(lib, d, q=0) == 1             # null pointers
    assert _shifted(lib, d, k=0) == 1
    assert _shifted(lib, d, v=0) == 1
    assert _shifted(lib, d, o=0) == 1
    assert _shifted(lib, d, lse=0) == 1
    assert _shifted(lib, d, q=FAKE + 8) == 1      # misaligned
    assert _shifted(lib, d, o=FAKE + 4) == 1
    assert _shifted(lib, d, lse=FAKE + 2) == 1
    # KV rows are indexed in 32-bit arithmetic: more than 2^31 - 64 is refused.
    assert _shifted(lib, d, total=(1 << 31) - 56, nch=8) == 2
    # Work items beyond 2^31 are refused without overflowing the count
    # (2^44 query tiles times 2^61 (batch, head) pairs; zero batch and head
    # strides keep every tensor's extent in range).
    flat = S3(0, 0, 128)
    big = _desc(batch=(1 << 31) - 1, heads_q=1 << 30, heads_kv=1 << 30, seq_q=1 << 52,
                q_stride=flat, k_stride=flat, v_stride=flat, o_stride=flat)
    assert _shifted(lib, big) == 2
    # With 4 query heads per KV head a bf16 work item is 64 query rows of 4
    # heads, so the item count is bounded with 64-row tiles: 2^35 rows give
    # 2^29 tiles x 4 heads = 2^31 items, one past the limit.  (The same rows
    # in 256-row tiles would pass this check; such a call is not made here
    # because it would be accepted and launched.)
    quad = _desc(heads_q=4, heads_kv=1, seq_q=1 << 35,
                 q_stride=flat, k_stride=flat, v_stride=flat, o_stride=flat)
    assert _shifted(lib, quad) == 2
    assert _chunk(lib, quad) == 2
    # Strides whose last element lies beyond 2^60 elements (64-bit offsets in
    # the kernels would wrap) are refused.
    far = _desc(batch=1 << 20, k_stride=S3(1 << 50, 1 << 20, 128))
    assert _shifted(lib, far) == 1
    assert _shifted(lib, _desc(batch=1 << 20, o_stride=S3(1 << 50, 1 << 20, 128))) == 1


def test_chunk_accumulate_rejects_bad_arguments():
    lib = _lib()
    d = _desc()

    def acc(dd, q=FAKE, k=FAKE, v=FAKE, kv_len=256, kv_pos0=0, o=FAKE, lse=FAKE):
        return lib.attn_chunk_fwd_accumulate(ctypes.byref(dd) if dd is not None else None, q, k,
                                             v, kv_len, kv_pos0, o, lse, None)

    assert acc(None) == 1
    assert acc(d, kv_len=-1) == 1
    assert acc(d, o=0) == 1
    assert acc(d, lse=FAKE + 2) == 1
    assert acc(_desc(head_dim=64)) == 2
    assert acc(_desc(o_stride=S3(6, 6, 6))) == 1


def test_chunk_rejects_bad_arguments():
    lib = _lib()
    d = _desc()
    assert _chunk(lib, None) == 1
    assert _chunk(lib, d, kv_len=-1) == 1
    assert _chunk(lib, d, kv_pos0=-3) == 1
    assert _chunk(lib, d, k=0) == 1
    assert _chunk(lib, d, v=FAKE + 2) == 1
    assert _chunk(lib, _desc(head_dim=256)) == 2
    assert _chunk(lib, d, kv_len=(1 << 31) - 63) == 2
    # o_part is fp32: a row stride of 6 floats (24 bytes) is not 16-byte aligned.
    assert _chunk(lib, _desc(o_stride=S3(6, 6, 6)), kv_len=256) == 1


S1, S2 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)  # stream handles, never used


def _overlapped(lib, d, q=FAKE, ksrc=FAKE, vsrc=FAKE, k=FAKE, v=FAKE, total=1024, nch=4, rank=1,
                o=0x1000000, lse=0x2000000, cs=S1, ps=S2):
    return lib.attn_shifted_fwd_overlapped(ctypes.byref(d) if d is not None else None, q, ksrc,
                                           vsrc, k, v, total, nch, rank, o, lse, cs, ps)


def test_overlapped_rejects_bad_arguments():
    lib = _lib()
    d = _desc()  # O strides are the contiguous [1, 4, 256, 128] ones
    assert _overlapped(lib, None) == 1
    assert _overlapped(lib, d, rank=4) == 1
    assert _overlapped(lib, d, total=1000, nch=3) == 1
    assert _overlapped(lib, d, cs=None, ps=None) == 1          # one stream for both
    assert _overlapped(lib, d, cs=S1, ps=S1) == 1
    assert _overlapped(lib, d, ksrc=0) == 1
    assert _overlapped(lib, d, vsrc=0) == 1
    assert _overlapped(lib, d, k=0) == 1
    assert _overlapped(lib, d, o=0) == 1
    assert _overlapped(lib, d, o=0x1000000 + 4) == 1            # misaligned O
    assert _overlapped(lib, d, lse=0x1000000 + 4096) == 1       # LSE inside O
    assert _overlapped(lib, d, lse=0x2000000 + 2) == 1          # misaligned LSE
    assert _overlapped(lib, _desc(o_stride=S3(2 * 4 * 256 * 128, 256 * 128, 128))) == 1
    assert _overlapped(lib, _desc(head_dim=64)) == 2
    assert _overlapped(lib, _desc(k_stride=S3(4 * 256 * 128, 256 * 128, 64))) == 1  # rows overlap
    assert _overlapped(lib, d, total=(1 << 31) - 56, nch=8) == 2
    # No query rows: nothing to do, nothing enqueued.
    empty = _desc(seq_q=0, o_stride=S3(0, 0, 128))
    assert _overlapped(lib, empty, q=0, o=0, lse=0) == 0


def test_merge_rejects_bad_arguments():
    lib = _lib()
    a, b = 0x100000, 0x200000
    la, lb = 0x300000, 0x400000
    assert lib.lse_merge(-1, 128, a, la, b, lb, None) == 1
    assert lib.lse_merge(10, 130, a, la, b, lb, None) == 1
    assert lib.lse_merge(10, 0, a, la, b, lb, None) == 1
    assert lib.lse_merge(10, 512, a, la, b, lb, None) == 1
    assert lib.lse_merge(10, 128, 0, la, b, lb, None) == 1
    assert lib.lse_merge(10, 128, a + 4, la, b, lb, None) == 1
    assert lib.lse_merge(10, 128, a, la + 1, b, lb, None) == 1
    assert lib.lse_merge(10, 128, a, la, a + 16, lb, None) == 1  # O sides overlap
    assert lib.lse_merge(10, 128, a, la, b, la, None) == 1       # LSE sides alias
    assert lib.lse_merge(10, 128, a, a + 64, b, lb, None) == 1   # LSE inside O
    assert lib.lse_merge(0, 128, 0, 0, 0, 0, None) == 0          # empty: a no-op


def test_python_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 2, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.attn_shifted_fwd(q, q, q, num_chunks=1, rank=0)


def _gdesc(**over):
    d = binding.ShattnGemmDesc()
    d.m, d.n, d.k = 1024, 256, 512
    d.lda, d.ldw, d.ldc = 512, 512, 256
    d.out_dtype = binding.BF16
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _gemm(lib, d, a=FAKE, w=FAKE, c=FAKE, nch=4, rank=1):
    return lib.allgather_gemm_shifted(ctypes.byref(d) if d is not None else None, a, w, c, nch,
                                      rank, None)


def test_gemm_desc_layout():
    assert ctypes.sizeof(binding.ShattnGemmDesc) == 6 * 8 + 8
    assert binding.ShattnGemmDesc.out_dtype.offset == 48


@pytest.mark.parametrize("case,expect", [
    ({"m": -1}, 1),
    ({"n": -8}, 1),
    ({"k": -64}, 1),
    ({"m": 1001}, 1),             # not a multiple of the chunk count
    ({"k": 96}, 2),               # valid, not built (k % 64)
    ({"n": 100, "ldc": 104}, 2),  # valid, not built (n % 8)
    ({"lda": 256}, 1),            # row stride below k
    ({"ldw": 500}, 1),
    ({"ldc": 200}, 1),
    ({"lda": 516}, 1),            # not a multiple of 8 elements
    ({"ldc": 260}, 1),            # bf16 C rows must stay 16-byte aligned
    ({"out_dtype": 5}, 1),
    ({"lda": (1 << 22) + 8}, 2),  # 32-bit tile addressing
])
def test_gemm_rejects_bad_desc(case, expect):
    lib = _lib()
    assert _gemm(lib, _gdesc(**case)) == expect


def test_gemm_rejects_bad_arguments():
    lib = _lib()
    d = _gdesc()
    assert _gemm(lib, None) == 1
    assert _gemm(lib, d, rank=4) == 1
    assert _gemm(lib, d, rank=-1) == 1
    assert _gemm(lib, d, nch=0) == 1
    assert _gemm(lib, d, a=0) == 1
    assert _gemm(lib, d, w=0) == 1
    assert _gemm(lib, d, c=0) == 1
    assert _gemm(lib, d, a=FAKE + 2) == 1
    assert _gemm(lib, d, c=FAKE + 8) == 1
    # fp32 C: a row stride of 260 floats (1040 bytes) is 16-byte aligned.
    assert _gemm(lib, _gdesc(out_dtype=binding.F32, ldc=260, n=256), a=0, nch=4) == 1
    # A grid beyond 2^31 workgroups (2^22 x 2^22 tiles; every extent within
    # 2^60 elements) is refused.
    assert _gemm(lib, _gdesc(m=1 << 30, n=1 << 30, k=64, lda=64, ldw=64, ldc=1 << 30)) == 2
    # Rows whose last element lies beyond 2^60 elements are refused.
    assert _gemm(lib, _gdesc(m=1 << 40, lda=1 << 21, ldw=512)) == 1
    # K == 0 writes zeros: A and W are never read and may be null.
    assert _gemm(lib, _gdesc(k=0, lda=0, ldw=0), a=0, w=0, c=0) == 1   # C is still needed
    # Nothing to compute: a no-op that touches no pointer.
    assert _gemm(lib, _gdesc(m=0), a=0, w=0, c=0) == 0
    assert _gemm(lib, _gdesc(n=0, ldc=0), a=0, w=0, c=0) == 0
