"""ctypes binding of libshattn.so (C-ABI declared in include/shattn.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: without the built library, or with CPU tensors, every
call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "ShattnError",
    "ShattnDesc",
    "library_path",
    "load_library",
    "attn_chunk_fwd",
    "attn_chunk_fwd_accumulate",
    "lse_merge",
    "attn_shifted_fwd",
    "attn_shifted_fwd_overlapped",
    "attn_status_string",
    "allgather_gemm_shifted",
    "ShattnGemmDesc",
    "DTYPE_CODES",
]

OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
BF16, F32 = 0, 1
DTYPE_CODES = {torch.bfloat16: BF16, torch.float32: F32}


class ShattnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {attn_status_string(status)} ({status})")


class ShattnDesc(ctypes.Structure):
    """Mirror of ``shattn_desc``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seq_q", ctypes.c_int64),
        ("q_pos0", ctypes.c_int64),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
    ]


class ShattnGemmDesc(ctypes.Structure):
    """Mirror of ``shattn_gemm_desc``."""

    _fields_ = [
        ("m", ctypes.c_int64),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("lda", ctypes.c_int64),
        ("ldw", ctypes.c_int64),
        ("ldc", ctypes.c_int64),
        ("out_dtype", ctypes.c_int32),
    ]


_LIB = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libshattn.so")


def load_library():
    """Load libshattn.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m long_context_attention_attn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    dp = ctypes.POINTER(ShattnDesc)
    lib.attn_chunk_fwd.argtypes = [dp, vp, vp, vp, i64, i64, vp, vp, vp]
    lib.attn_chunk_fwd.restype = ctypes.c_int
    lib.attn_chunk_fwd_accumulate.argtypes = [dp, vp, vp, vp, i64, i64, vp, vp, vp]
    lib.attn_chunk_fwd_accumulate.restype = ctypes.c_int
    lib.lse_merge.argtypes = [i64, i32, vp, vp, vp, vp, vp]
    lib.lse_merge.restype = ctypes.c_int
    lib.attn_shifted_fwd.argtypes = [dp, vp, vp, vp, i64, i32, i32, vp, vp, vp]
    lib.attn_shifted_fwd.restype = ctypes.c_int
    lib.attn_shifted_fwd_overlapped.argtypes = [dp, vp, vp, vp, vp, vp, i64, i32, i32, vp, vp,
                                                vp, vp]
    lib.attn_shifted_fwd_overlapped.restype = ctypes.c_int
    lib.allgather_gemm_shifted.argtypes = [ctypes.POINTER(ShattnGemmDesc), vp, vp, vp, i32, i32,
                                           vp]
    lib.allgather_gemm_shifted.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != OK:
        raise ShattnError(fn, status)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("shattn operates on GPU tensors only (no CPU path)")


def _strides(t: torch.Tensor):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a 4-D [B, H, S, D] tensor with a contiguous last axis")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _check_shapes(q, k, v, o, lse):
    """The C ABI sees pointers and strides only: every size it derives from
    ``q`` must hold for the other tensors, or a kernel would run past one of
    them.  K/V: [B, Hkv, Skv, D] with Hq % Hkv == 0; O: q's shape; LSE:
    [B, Hq, Sq]."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", o)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, S, D], got {tuple(t.shape)}")
    b, hq, sq, dim = q.shape
    if k.shape != v.shape:
        raise ValueError(f"K {tuple(k.shape)} and V {tuple(v.shape)} differ in shape")
    if k.shape[0] != b or k.shape[3] != dim:
        raise ValueError(f"K/V {tuple(k.shape)} do not match Q {tuple(q.shape)} in batch "
                         "or head_dim")
    if k.shape[1] < 1 or hq % k.shape[1] != 0:
        raise ValueError(f"query heads {hq} are not a multiple of KV heads {k.shape[1]}")
    if tuple(o.shape) != (b, hq, sq, dim):
        raise ValueError(f"output {tuple(o.shape)} does not match Q {tuple(q.shape)}")
    if lse is not None and tuple(lse.shape) != (b, hq, sq):
        raise ValueError(f"LSE {tuple(lse.shape)} is not [B, Hq, Sq] = {(b, hq, sq)}")


def make_desc(q, k, v, o, *, causal: bool, q_pos0: int, scale, out_dtype, lse=None) -> ShattnDesc:
    if q.dtype not in DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("Q, K, V must share one dtype: bfloat16 or float32")
    _check_shapes(q, k, v, o, lse)
    d = ShattnDesc()
    d.batch, d.heads_q, d.seq_q, d.head_dim = q.shape[0], q.shape[1], q.shape[2], q.shape[3]
    d.heads_kv = k.shape[1]
    d.q_pos0 = int(q_pos0)
    d.causal = 1 if causal else 0
    d.scale = 0.0 if scale is None else float(scale)
    d.in_dtype = DTYPE_CODES[q.dtype]
    d.out_dtype = DTYPE_CODES[out_dtype]
    d.q_stride = _strides(q)
    d.k_stride = _strides(k)
    d.v_stride = _strides(v)
    d.o_stride = _strides(o)
    return d


def attn_chunk_fwd(q, k_chunk, v_chunk, *, kv_pos0: int, causal: bool = False, q_pos0: int = 0,
                   scale=None, o_part=None, lse_part=None):
    """Partial (O fp32, LSE fp32) of ``q`` against one KV chunk at ``kv_pos0``."""
    _require_cuda(q, k_chunk, v_chunk, o_part, lse_part)
    b, hq, sq, dim = q.shape
    if k_chunk.shape[2] != v_chunk.shape[2]:
        raise ValueError("K and V chunks differ in length")
    if o_part is None:
        o_part = torch.empty((b, hq, sq, dim), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32 \
            or not lse_part.is_contiguous():
        raise ValueError("o_part/lse_part must be float32 (lse_part contiguous)")
    desc = make_desc(q, k_chunk, v_chunk, o_part, causal=causal, q_pos0=q_pos0, scale=scale,
                     out_dtype=torch.float32, lse=lse_part)
    lib = load_library()
    st = lib.attn_chunk_fwd(ctypes.byref(desc), q.data_ptr(), k_chunk.data_ptr(),
                            v_chunk.data_ptr(), k_chunk.shape[2], int(kv_pos0),
                            o_part.data_ptr(), lse_part.data_ptr(), _stream(q))
    _check("attn_chunk_fwd", st)
    return o_part, lse_part


def attn_chunk_fwd_accumulate(q, k_chunk, v_chunk, o_acc, lse_acc, *, kv_pos0: int,
                              causal: bool = False, q_pos0: int = 0, scale=None):
    """In place: (o_acc, lse_acc) <- merge((o_acc, lse_acc), partial of ``q``
    against one KV chunk at ``kv_pos0``), the merge done in the kernel."""
    _require_cuda(q, k_chunk, v_chunk, o_acc, lse_acc)
    if o_acc.dtype != torch.float32 or lse_acc.dtype != torch.float32 \
            or not lse_acc.is_contiguous():
        raise ValueError("o_acc/lse_acc must be float32 (lse_acc contiguous)")
    desc = make_desc(q, k_chunk, v_chunk, o_acc, causal=causal, q_pos0=q_pos0, scale=scale,
                     out_dtype=torch.float32, lse=lse_acc)
    st = load_library().attn_chunk_fwd_accumulate(
        ctypes.byref(desc), q.data_ptr(), k_chunk.data_ptr(), v_chunk.data_ptr(),
        k_chunk.shape[2], int(kv_pos0), o_acc.data_ptr(), lse_acc.data_ptr(), _stream(q))
    _check("attn_chunk_fwd_accumulate", st)
    return o_acc, lse_acc


def lse_merge(o_acc, lse_acc, o_part, lse_part):
    """In place: (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_part, lse_part))."""
    _require_cuda(o_acc, lse_acc, o_part, lse_part)
    for t in (o_acc, lse_acc, o_part, lse_part):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("lse_merge takes contiguous float32 tensors")
    dim = o_acc.shape[-1]
    rows = lse_acc.numel()
    if o_part.shape != o_acc.shape or lse_part.shape != lse_acc.shape \
            or tuple(o_acc.shape[:-1]) != tuple(lse_acc.shape):
        raise ValueError("O tensors must share one shape [..., D] and LSE tensors its [...]")
    if o_acc.numel() != rows * dim:
        raise ValueError("shape mismatch between O and LSE tensors")
    st = load_library().lse_merge(rows, dim, o_acc.data_ptr(), lse_acc.data_ptr(),
                                  o_part.data_ptr(), lse_part.data_ptr(), _stream(o_acc))
    _check("lse_merge", st)


def attn_shifted_fwd(q, k, v, *, num_chunks: int, rank: int, causal: bool = False,
                     q_pos0: int = 0, scale=None, out_dtype=None, out=None, lse=None):
    """Fused shifted-chunk attention of rank ``rank`` of ``num_chunks``.

    Returns (O in ``out_dtype`` (default: the input dtype), LSE float32).
    """
    _require_cuda(q, k, v, out, lse)
    b, hq, sq, dim = q.shape
    if k.shape[2] != v.shape[2]:
        raise ValueError("K and V differ in length")
    if out_dtype is None:
        out_dtype = q.dtype if out is None else out.dtype
    if out is None:
        out = torch.empty((b, hq, sq, dim), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    if out.dtype != out_dtype or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("bad output tensors")
    desc = make_desc(q, k, v, out, causal=causal, q_pos0=q_pos0, scale=scale,
                     out_dtype=out_dtype, lse=lse)
    st = load_library().attn_shifted_fwd(ctypes.byref(desc), q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), k.shape[2], int(num_chunks), int(rank),
                                         out.data_ptr(), lse.data_ptr(), _stream(q))
    _check("attn_shifted_fwd", st)
    return out, lse


def attn_shifted_fwd_overlapped(q, k_src, v_src, k, v, *, num_chunks: int, rank: int,
                                causal: bool = False, q_pos0: int = 0, scale=None,
                                copy_stream=None):
    """Shifted chunk walk with each chunk's K/V rows copied from ``k_src`` /
    ``v_src`` (pinned host tensors, or another device's) into the device
    tensors ``k`` / ``v`` on ``copy_stream`` while earlier chunks compute on
    the current stream.

    Returns (O float32, LSE float32).  ``copy_stream`` defaults to a new
    stream of default priority.
    """
    _require_cuda(q, k, v)
    for src, dst in ((k_src, k), (v_src, v)):
        if src.shape != dst.shape or src.dtype != dst.dtype or src.stride() != dst.stride():
            raise ValueError("source and device K/V tensors must match in shape and layout")
        if not src.is_cuda and not src.is_pinned():
            raise ValueError("a host source must be pinned memory")
    b, hq, sq, dim = q.shape
    if k.shape[2] != v.shape[2]:
        raise ValueError("K and V differ in length")
    o = torch.empty((b, hq, sq, dim), dtype=torch.float32, device=q.device)
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=q.device)
    desc = make_desc(q, k, v, o, causal=causal, q_pos0=q_pos0, scale=scale,
                     out_dtype=torch.float32, lse=lse)
    st = load_library().attn_shifted_fwd_overlapped(
        ctypes.byref(desc), q.data_ptr(), k_src.data_ptr(), v_src.data_ptr(), k.data_ptr(),
        v.data_ptr(), k.shape[2], int(num_chunks), int(rank), o.data_ptr(), lse.data_ptr(),
        _stream(q), copy_stream.cuda_stream)
    _check("attn_shifted_fwd_overlapped", st)
    # The sources must stay alive until the current stream has passed this
    # call's work (the caller's references do that); the device K/V are
    # ordered by the current stream, which ends after the copies.
    return o, lse


def _row_stride(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major matrix (contiguous rows)")
    return t.stride(0)


def allgather_gemm_shifted(a, w, *, num_chunks: int, rank: int, out_dtype=None, out=None):
    """C = A W^T with A's row chunks visited from chunk ``rank`` on.

    ``a`` [M, K] bf16 (the gathered activation, M a multiple of
    ``num_chunks``), ``w`` [N, K] bf16 (the rank's weight shard).  Returns C
    [M, N] in ``out_dtype`` (default bf16) or into ``out``.
    """
    _require_cuda(a, w, out)
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("A and W must be bfloat16")
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[1]:
        raise ValueError(f"A {tuple(a.shape)} and W {tuple(w.shape)} must be [M, K] and [N, K]")
    m, k = a.shape
    n = w.shape[0]
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    if out_dtype not in DTYPE_CODES:
        raise ValueError("C must be bfloat16 or float32")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    if out.dtype != out_dtype or tuple(out.shape) != (m, n):
        raise ValueError(f"C must be [M, N] = {(m, n)} of {out_dtype}")
    d = ShattnGemmDesc()
    d.m, d.n, d.k = m, n, k
    d.lda, d.ldw, d.ldc = _row_stride(a, "A"), _row_stride(w, "W"), _row_stride(out, "C")
    if k == 0:  # an empty contraction has no rows to step over
        d.lda = d.ldw = 0
    d.out_dtype = DTYPE_CODES[out_dtype]
    st = load_library().allgather_gemm_shifted(ctypes.byref(d), a.data_ptr(), w.data_ptr(),
                                               out.data_ptr(), int(num_chunks), int(rank),
                                               _stream(a))
    _check("allgather_gemm_shifted", st)
    return out
