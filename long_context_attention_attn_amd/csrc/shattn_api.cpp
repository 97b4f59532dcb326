// C-ABI entry points declared in include/shattn.h.
//
// Every argument is checked on the host before any HIP runtime call, so the
// error paths need no GPU.  Each successful kernel call enqueues exactly one
// kernel on the caller's stream and returns the launch status; the
// overlapped walk enqueues copies, events and those kernels on two streams.
// Nothing synchronizes and no memory is allocated.

#include <math.h>
#include <stdint.h>

#include "../../include/shattn.h"
#include "kernels.h"

namespace {

using shattn::DType;
using shattn::FwdParams;

constexpr int32_t kSupportedHeadDim = 128;
constexpr int64_t kPosLimit = (int64_t)1 << 60;  // keeps position arithmetic far from overflow
// The kernels address rows within one 64-row tile in 32-bit arithmetic
// (row * seq_stride + column), so a sequence stride must stay below 2^24
// elements.  Real layouts ([B, H, S, D] or [B, S, H, D]) are far below it.
constexpr int64_t kSeqStrideLimit = (int64_t)1 << 24;
// Key rows of one call: the kernels index them in 32-bit arithmetic.
constexpr int64_t kKvRowLimit = ((int64_t)1 << 31) - 64;

bool valid_dtype(int32_t d) { return d == SHATTN_BF16 || d == SHATTN_F32; }

int64_t elem_size(int32_t d) { return d == SHATTN_F32 ? 4 : 2; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A (batch, head, seq) stride triple: non-negative and a multiple of 16 bytes.
bool strides_ok(const int64_t s[3], int64_t esize) {
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0 || s[i] > kPosLimit) return false;
    if ((s[i] * esize) % 16 != 0) return false;
  }
  return true;
}

int status_of(hipError_t e) { return e == hipSuccess ? SHATTN_OK : SHATTN_EHIP; }

// The element offset of the last element of a [n0, n1, n2, inner] tensor with
// strides s (a non-empty one), computed without overflow, must stay within
// kPosLimit: the kernels address elements in 64-bit arithmetic.
bool extent_ok(const int64_t s[3], int64_t n0, int64_t n1, int64_t n2, int64_t inner) {
  const __int128 last = (__int128)(n0 - 1) * s[0] + (__int128)(n1 - 1) * s[1] +
                        (__int128)(n2 - 1) * s[2] + inner;
  return last <= kPosLimit;
}

// Checks shared by attn_chunk_fwd and attn_shifted_fwd.  `o_esize` is the
// element size of the O tensor of the call.
int check_desc(const shattn_desc* d, const void* q, const void* k, const void* v, const void* o,
               const float* lse, int64_t kv_rows, int64_t o_esize) {
  if (d == nullptr) return SHATTN_EINVAL;
  if (d->batch < 0 || d->heads_q < 1 || d->heads_kv < 1) return SHATTN_EINVAL;
  if (d->heads_q % d->heads_kv != 0) return SHATTN_EINVAL;
  if (d->head_dim <= 0 || d->head_dim % 4 != 0) return SHATTN_EINVAL;
  if (d->head_dim != kSupportedHeadDim) return SHATTN_EUNSUPPORTED;
  if (d->seq_q < 0 || d->seq_q > kPosLimit) return SHATTN_EINVAL;
  if (d->q_pos0 < 0 || d->q_pos0 > kPosLimit) return SHATTN_EINVAL;
  if (d->causal != 0 && d->causal != 1) return SHATTN_EINVAL;
  if (!isfinite(d->scale)) return SHATTN_EINVAL;
  if (!valid_dtype(d->in_dtype)) return SHATTN_EINVAL;
  const int64_t es = elem_size(d->in_dtype);
  if (!strides_ok(d->q_stride, es) || !strides_ok(d->k_stride, es) ||
      !strides_ok(d->v_stride, es) || !strides_ok(d->o_stride, o_esize))
    return SHATTN_EINVAL;
  if (d->q_stride[2] > kSeqStrideLimit || d->k_stride[2] > kSeqStrideLimit ||
      d->v_stride[2] > kSeqStrideLimit || d->o_stride[2] > kSeqStrideLimit)
    return SHATTN_EUNSUPPORTED;
  const bool q_empty = d->batch == 0 || d->seq_q == 0;
  const bool kv_empty = d->batch == 0 || kv_rows == 0;
  if (!q_empty && (!extent_ok(d->q_stride, d->batch, d->heads_q, d->seq_q, d->head_dim) ||
                   !extent_ok(d->o_stride, d->batch, d->heads_q, d->seq_q, d->head_dim)))
    return SHATTN_EINVAL;
  if (!kv_empty && (!extent_ok(d->k_stride, d->batch, d->heads_kv, kv_rows, d->head_dim) ||
                    !extent_ok(d->v_stride, d->batch, d->heads_kv, kv_rows, d->head_dim)))
    return SHATTN_EINVAL;
  if (!q_empty && (q == nullptr || o == nullptr || lse == nullptr)) return SHATTN_EINVAL;
  if (!kv_empty && (k == nullptr || v == nullptr)) return SHATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SHATTN_EINVAL;
  if (((uintptr_t)lse & 3u) != 0) return SHATTN_EINVAL;
  // Work items: item_rows query rows of item_heads query heads (the bf16
  // kernel walks them with at most one workgroup per CU, the fp32 kernel
  // launches one workgroup per item).  The count is bounded by tiles x heads.
  const int64_t bm =
      shattn::item_rows((DType)d->in_dtype, (int64_t)d->heads_q / d->heads_kv);
  const int64_t tiles = (d->seq_q + bm - 1) / bm;
  // Each factor is bounded first, so that no product overflows.
  const int64_t heads = (int64_t)d->batch * d->heads_q;  // < 2^62
  if (tiles > INT32_MAX || heads > INT32_MAX || tiles * heads > INT32_MAX)
    return SHATTN_EUNSUPPORTED;
  return SHATTN_OK;
}

FwdParams make_params(const shattn_desc* d, const void* q, const void* k, const void* v,
                      void* o, float* lse) {
  FwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.q_sb = d->q_stride[0];
  p.q_sh = d->q_stride[1];
  p.q_ss = d->q_stride[2];
  p.k_sb = d->k_stride[0];
  p.k_sh = d->k_stride[1];
  p.k_ss = d->k_stride[2];
  p.v_sb = d->v_stride[0];
  p.v_sh = d->v_stride[1];
  p.v_ss = d->v_stride[2];
  p.o_sb = d->o_stride[0];
  p.o_sh = d->o_stride[1];
  p.o_ss = d->o_stride[2];
  p.seq_q = d->seq_q;
  p.q_pos0 = d->q_pos0;
  p.batch = d->batch;
  p.heads_q = d->heads_q;
  p.heads_kv = d->heads_kv;
  p.group = d->heads_q / d->heads_kv;
  p.causal = d->causal;
  const double scale = d->scale > 0.f ? (double)d->scale : 1.0 / sqrt((double)d->head_dim);
  p.scale_log2 = (float)(scale * 1.4426950408889634074);
  const DType in = (DType)d->in_dtype;
  const int64_t bm = shattn::item_rows(in, p.group);
  p.num_q_tiles = (int32_t)((d->seq_q + bm - 1) / bm);
  p.quad_heads = shattn::quad_heads(in, p.group) ? 1 : 0;
  return p;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// attn_chunk_fwd, writing (accumulate = 0) or merging into (accumulate = 1)
// the fp32 pair (o, lse).
int chunk_fwd(const shattn_desc* desc, const void* q, const void* k, const void* v,
              int64_t kv_len, int64_t kv_pos0, float* o, float* lse, int accumulate,
              hipStream_t stream) {
  if (kv_len < 0 || kv_len > kPosLimit || kv_pos0 < 0 || kv_pos0 > kPosLimit)
    return SHATTN_EINVAL;
  int st = check_desc(desc, q, k, v, o, lse, kv_len, 4);
  if (st != SHATTN_OK) return st;
  if (kv_len > kKvRowLimit) return SHATTN_EUNSUPPORTED;
  FwdParams p = make_params(desc, q, k, v, o, lse);
  p.kv_pos0 = kv_pos0;
  p.chunk_len = kv_len;
  p.num_chunks = 1;
  p.rank = 0;
  p.kv_rows = (int32_t)kv_len;
  p.seg_a0 = 0;
  p.q_rel0 = desc->q_pos0 - kv_pos0;
  p.accumulate = accumulate;
  if (desc->batch == 0 || desc->seq_q == 0) return SHATTN_OK;
  return status_of(shattn::launch_attn_fwd(p, (DType)desc->in_dtype, DType::F32, stream));
}

}  // namespace

extern "C" {

int attn_chunk_fwd(const shattn_desc* desc, const void* q, const void* k, const void* v,
                   int64_t kv_len, int64_t kv_pos0, float* o_part, float* lse_part,
                   hipStream_t stream) {
  return chunk_fwd(desc, q, k, v, kv_len, kv_pos0, o_part, lse_part, 0, stream);
}

int attn_chunk_fwd_accumulate(const shattn_desc* desc, const void* q, const void* k,
                              const void* v, int64_t kv_len, int64_t kv_pos0, float* o_acc,
                              float* lse_acc, hipStream_t stream) {
  return chunk_fwd(desc, q, k, v, kv_len, kv_pos0, o_acc, lse_acc, 1, stream);
}

}  // extern "C"

namespace {

// Argument checks of lse_merge for rows > 0.
int check_merge(int64_t rows, int32_t head_dim, const float* o_acc, const float* lse_acc,
                const float* o_part, const float* lse_part) {
  if (!o_acc || !lse_acc || !o_part || !lse_part) return SHATTN_EINVAL;
  if (!aligned16(o_acc) || !aligned16(o_part)) return SHATTN_EINVAL;
  if ((((uintptr_t)lse_acc) & 3u) || (((uintptr_t)lse_part) & 3u)) return SHATTN_EINVAL;
  // The accumulator must not overlap the partial it reads.
  const uintptr_t oa = (uintptr_t)o_acc, ob = (uintptr_t)o_part;
  const uintptr_t la = (uintptr_t)lse_acc, lb = (uintptr_t)lse_part;
  const uintptr_t obytes = (uintptr_t)rows * (uintptr_t)head_dim * 4u;
  const uintptr_t lbytes = (uintptr_t)rows * 4u;
  if (oa < ob + obytes && ob < oa + obytes) return SHATTN_EINVAL;
  if (la < lb + lbytes && lb < la + lbytes) return SHATTN_EINVAL;
  if (oa < la + lbytes && la < oa + obytes) return SHATTN_EINVAL;
  return SHATTN_OK;
}

}  // namespace

extern "C" {

int lse_merge(int64_t rows, int32_t head_dim, float* o_acc, float* lse_acc, const float* o_part,
              const float* lse_part, hipStream_t stream) {
  if (rows < 0 || rows > kPosLimit) return SHATTN_EINVAL;
  if (head_dim < 4 || head_dim > 256 || head_dim % 4 != 0) return SHATTN_EINVAL;
  if (rows == 0) return SHATTN_OK;
  const int st = check_merge(rows, head_dim, o_acc, lse_acc, o_part, lse_part);
  if (st != SHATTN_OK) return st;
  return status_of(
      shattn::launch_lse_merge(rows, head_dim, o_acc, lse_acc, o_part, lse_part, stream));
}

int attn_shifted_fwd(const shattn_desc* desc, const void* q, const void* k, const void* v,
                     int64_t kv_len_total, int32_t num_chunks, int32_t rank, void* o, float* lse,
                     hipStream_t stream) {
  if (num_chunks < 1 || rank < 0 || rank >= num_chunks) return SHATTN_EINVAL;
  if (kv_len_total < 0 || kv_len_total > kPosLimit || kv_len_total % num_chunks != 0)
    return SHATTN_EINVAL;
  if (desc == nullptr || !valid_dtype(desc->out_dtype)) return SHATTN_EINVAL;
  int st = check_desc(desc, q, k, v, o, lse, kv_len_total, elem_size(desc->out_dtype));
  if (st != SHATTN_OK) return st;
  if (kv_len_total > kKvRowLimit) return SHATTN_EUNSUPPORTED;
  FwdParams p = make_params(desc, q, k, v, o, lse);
  p.kv_pos0 = 0;
  p.chunk_len = kv_len_total / num_chunks;
  p.num_chunks = num_chunks;
  p.rank = rank;
  p.kv_rows = (int32_t)kv_len_total;
  p.seg_a0 = (int32_t)(p.chunk_len * rank);
  p.q_rel0 = desc->q_pos0;
  if (desc->batch == 0 || desc->seq_q == 0) return SHATTN_OK;
  return status_of(shattn::launch_attn_fwd(p, (DType)desc->in_dtype, (DType)desc->out_dtype,
                                           stream));
}

int attn_shifted_fwd_overlapped(const shattn_desc* desc, const void* q, const void* k_src,
                                const void* v_src, void* k, void* v, int64_t kv_len_total,
                                int32_t num_chunks, int32_t rank, float* o, float* lse,
                                hipStream_t compute_stream, hipStream_t copy_stream) {
  if (num_chunks < 1 || rank < 0 || rank >= num_chunks) return SHATTN_EINVAL;
  if (kv_len_total < 0 || kv_len_total > kPosLimit || kv_len_total % num_chunks != 0)
    return SHATTN_EINVAL;
  if (desc == nullptr) return SHATTN_EINVAL;
  int st = check_desc(desc, q, k, v, o, lse, kv_len_total, 4);
  if (st != SHATTN_OK) return st;
  if (kv_len_total > kKvRowLimit) return SHATTN_EUNSUPPORTED;
  if (compute_stream == copy_stream) return SHATTN_EINVAL;
  const bool q_empty = desc->batch == 0 || desc->seq_q == 0;
  const bool kv_empty = desc->batch == 0 || kv_len_total == 0;
  if (!kv_empty && (k_src == nullptr || v_src == nullptr)) return SHATTN_EINVAL;
  // Rows must not overlap: each chunk is copied row by row at most.
  if (desc->k_stride[2] < desc->head_dim || desc->v_stride[2] < desc->head_dim)
    return SHATTN_EINVAL;
  // O is contiguous [B, Hq, Sq, D] and must not overlap LSE.
  const int64_t dim = desc->head_dim;
  const int64_t rows = (int64_t)desc->batch * desc->heads_q * desc->seq_q;
  if (desc->o_stride[2] != dim || desc->o_stride[1] != desc->seq_q * dim ||
      desc->o_stride[0] != desc->heads_q * desc->seq_q * dim)
    return SHATTN_EINVAL;
  if (q_empty) return SHATTN_OK;
  {
    const uintptr_t oa = (uintptr_t)o, la = (uintptr_t)lse;
    const uintptr_t ob = (uintptr_t)rows * (uintptr_t)dim * 4u, lb = (uintptr_t)rows * 4u;
    if (oa < la + lb && la < oa + ob) return SHATTN_EINVAL;
  }

  const int64_t es = elem_size(desc->in_dtype);
  const int64_t clen = kv_len_total / num_chunks;
  // Position of the last query: a causal chunk starting after it is seen by
  // no query, so it is neither fetched nor computed.
  const int64_t q_last = desc->q_pos0 + desc->seq_q - 1;
  auto chunk_ptr = [&](const void* base, const int64_t* stride, int64_t c) {
    return (const char*)base + c * clen * stride[2] * es;
  };
  hipError_t e = hipSuccess;
  auto ok = [&](hipError_t r) {
    if (e == hipSuccess) e = r;
    return e == hipSuccess;
  };
  // The copies overwrite k and v: they wait for the work already on the
  // compute stream, which may still read them.
  hipEvent_t ev;
  if (!ok(hipEventCreateWithFlags(&ev, hipEventDisableTiming))) return SHATTN_EHIP;
  ok(hipEventRecord(ev, compute_stream));
  ok(hipStreamWaitEvent(copy_stream, ev, 0));
  ok(hipEventDestroy(ev));
  auto copy_chunk = [&](const void* src, void* dst, const int64_t* st, int64_t c) {
    const int64_t row_b = dim * es, pitch = st[2] * es;
    const char* s0 = chunk_ptr(src, st, c);
    char* d0 = (char*)chunk_ptr(dst, st, c);
    if (st[2] == dim) {
      const int64_t block = clen * row_b;
      const int32_t nb = desc->batch, nh = desc->heads_kv;
      if ((int64_t)nb * nh == 1) {
        ok(hipMemcpyAsync(d0, s0, block, hipMemcpyDefault, copy_stream));
      } else if ((nb == 1 || st[0] == nh * st[1]) && st[1] * es >= block) {
        ok(hipMemcpy2DAsync(d0, st[1] * es, s0, st[1] * es, block, (size_t)nb * nh,
                            hipMemcpyDefault, copy_stream));
      } else {
        for (int32_t b = 0; b < nb && e == hipSuccess; ++b)
          for (int32_t hk = 0; hk < nh && e == hipSuccess; ++hk) {
            const int64_t off = (b * st[0] + hk * st[1]) * es;
            ok(hipMemcpyAsync(d0 + off, s0 + off, block, hipMemcpyDefault, copy_stream));
          }
      }
      return;
    }
    for (int32_t b = 0; b < desc->batch && e == hipSuccess; ++b)
      for (int32_t hk = 0; hk < desc->heads_kv && e == hipSuccess; ++hk) {
        const int64_t off = (b * st[0] + hk * st[1]) * es;
        ok(hipMemcpy2DAsync(d0 + off, pitch, s0 + off, pitch, row_b, clen, hipMemcpyDefault,
                            copy_stream));
      }
  };
  bool first = true;
  for (int32_t j = 0; j < num_chunks && e == hipSuccess && !kv_empty; ++j) {
    const int64_t c = (j + rank) % num_chunks;
    if (desc->causal && c * clen > q_last) continue;
    // Chunk c's rows of every (batch, KV head) slice, at the same offsets in
    // source and destination, in as few copies as the layout allows: with
    // rows back to back (sequence stride == head_dim) one slice's chunk is a
    // single block, and evenly spaced slices make one 2-D copy of blocks.
    // Chunk `rank` (j = 0) is the rank's own: it is already in k, v.
    if (j > 0) {
      copy_chunk(k_src, k, desc->k_stride, c);
      copy_chunk(v_src, v, desc->v_stride, c);
      if (!ok(hipEventCreateWithFlags(&ev, hipEventDisableTiming))) break;
      ok(hipEventRecord(ev, copy_stream));
      ok(hipStreamWaitEvent(compute_stream, ev, 0));
      ok(hipEventDestroy(ev));
      if (e != hipSuccess) break;
    }
    // Partial of Q against chunk c: the first one written to (o, lse), each
    // later one merged into them in the kernel's epilogue, in visit order.
    st = chunk_fwd(desc, q, chunk_ptr(k, desc->k_stride, c), chunk_ptr(v, desc->v_stride, c),
                   clen, c * clen, o, lse, first ? 0 : 1, compute_stream);
    if (st != SHATTN_OK) return st;
    first = false;
  }
  if (e != hipSuccess) return SHATTN_EHIP;
  // No chunk visible to any query: O = 0, LSE = -inf.
  if (first) return attn_chunk_fwd(desc, q, k, v, 0, 0, o, lse, compute_stream);
  return SHATTN_OK;
}

int allgather_gemm_shifted(const shattn_gemm_desc* desc, const void* a, const void* w, void* c,
                           int32_t num_chunks, int32_t rank, hipStream_t stream) {
  if (desc == nullptr) return SHATTN_EINVAL;
  const shattn_gemm_desc& d = *desc;
  if (num_chunks < 1 || rank < 0 || rank >= num_chunks) return SHATTN_EINVAL;
  if (d.m < 0 || d.n < 0 || d.k < 0 || d.m > kPosLimit || d.n > kPosLimit || d.k > kPosLimit)
    return SHATTN_EINVAL;
  if (d.m % num_chunks != 0) return SHATTN_EINVAL;
  if (!valid_dtype(d.out_dtype)) return SHATTN_EINVAL;
  if (d.k % 64 != 0 || d.n % 8 != 0) return SHATTN_EUNSUPPORTED;
  const bool empty = d.m == 0 || d.n == 0;
  if (!empty && (a == nullptr && d.k > 0)) return SHATTN_EINVAL;
  if (!empty && ((w == nullptr && d.k > 0) || c == nullptr)) return SHATTN_EINVAL;
  if (d.lda < d.k || d.ldw < d.k || d.ldc < d.n) return SHATTN_EINVAL;
  if (!empty) {  // the last element of A, W and C within 64-bit element offsets
    const int64_t ra[3] = {0, 0, d.lda}, rw[3] = {0, 0, d.ldw}, rc[3] = {0, 0, d.ldc};
    if (!extent_ok(ra, 1, 1, d.m, d.k) || !extent_ok(rw, 1, 1, d.n, d.k) ||
        !extent_ok(rc, 1, 1, d.m, d.n))
      return SHATTN_EINVAL;
  }
  if (d.lda % 8 != 0 || d.ldw % 8 != 0 || d.ldc % (d.out_dtype == SHATTN_F32 ? 4 : 8) != 0)
    return SHATTN_EINVAL;
  if (!aligned16(a) || !aligned16(w) || !aligned16(c)) return SHATTN_EINVAL;
  // A tile's copies address up to 256 rows in 32-bit byte offsets.
  if (d.lda > kSeqStrideLimit / 4 || d.ldw > kSeqStrideLimit / 4) return SHATTN_EUNSUPPORTED;
  const int64_t chunk_rows = d.m / num_chunks;
  const int64_t tiles_per_chunk = (chunk_rows + 255) / 256;
  const int64_t tiles_m = tiles_per_chunk * num_chunks;
  const int64_t tiles_n = (d.n + 255) / 256;
  // The launch's grid is one of two shapes (the XCDs all on every column
  // tile, or split into row groups and column halves); each factor is
  // bounded first, so that no product overflows.
  if (tiles_m > INT32_MAX / 8 || tiles_n > INT32_MAX) return SHATTN_EUNSUPPORTED;
  const int64_t grid_all_columns = ((tiles_m + 7) / 8) * 8 * tiles_n;
  const int64_t grid_split = 8 * ((tiles_m + 3) / 4) * ((tiles_n + 1) / 2);
  if (grid_all_columns > INT32_MAX || grid_split > INT32_MAX) return SHATTN_EUNSUPPORTED;
  if (empty) return SHATTN_OK;
  shattn::GemmParams p = {};
  p.a = a;
  p.w = w;
  p.c = c;
  p.m = d.m;
  p.n = d.n;
  p.k = d.k;
  p.lda = d.lda;
  p.ldw = d.ldw;
  p.ldc = d.ldc;
  p.chunk_rows = chunk_rows;
  p.num_chunks = num_chunks;
  p.rank = rank;
  p.tiles_per_chunk = (int32_t)tiles_per_chunk;
  p.n_tiles_m = (int32_t)tiles_m;
  p.n_tiles_n = (int32_t)tiles_n;
  return status_of(shattn::launch_gemm_bf16(p, (DType)d.out_dtype, stream));
}

const char* attn_status_string(int status) {
  switch (status) {
    case SHATTN_OK:
      return "SHATTN_OK";
    case SHATTN_EINVAL:
      return "SHATTN_EINVAL";
    case SHATTN_EUNSUPPORTED:
      return "SHATTN_EUNSUPPORTED";
    case SHATTN_EHIP:
      return "SHATTN_EHIP";
    default:
      return "SHATTN_UNKNOWN";
  }
}

}  // extern "C"
