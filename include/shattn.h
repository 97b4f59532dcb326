/*
 * shattn — shifted-chunk long-context attention for AMD MI355X (gfx950).
 *
 * One rank's share of ring/shifted long-context attention: a local query
 * shard attends to a KV buffer split into J equal chunks that are visited in
 * the rank-shifted order c_j = (j + i) % J, each chunk's partial output and
 * log-sum-exp being merged online.  The shift order is the one CommIR's
 * `shift` primitive introduces (papers.lqhl.me summary "Mercury (SOSP 2025)",
 * section 核心方法 / core method); staggering the chunk order by rank is the
 * temporal decoupling of the Silicon & Systems digest of Mercury, section
 * "The hidden cost of synchronized operators".  The local attention itself
 * is the kernel Mercury keeps as a "patch" (digest, section "CommIR makes
 * communication transformable"); the pages do not write its arithmetic out,
 * so the definitions below are the textbook ones.
 *
 * Common rules for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller (the
 *    overlapped walk's sources may also be pinned host memory).  The
 *    library never allocates, frees or retains user memory.
 *  - Calls only enqueue work on their stream(s) (0 = the null stream) and
 *    never synchronize; outputs are valid once the stream reaches that
 *    point.
 *  - Every argument is validated on the host before anything is launched; on
 *    failure the call returns a non-zero status and launches nothing.  Among
 *    the checks: the last element of every tensor, from its sizes and
 *    strides, must lie within 2^60 elements of its base pointer (kernels
 *    address elements in 64-bit arithmetic), else SHATTN_EINVAL.  No
 *    exceptions cross this boundary and nothing aborts.
 *  - NaN/Inf in inputs propagate to the outputs; they are never masked.  In
 *    the bf16 path they can also reach a few rows that do not see them:
 *    with a NaN/Inf in V, the rows of a 64-row query group that reads the
 *    64-key tile holding it get NaN in that column (0 * NaN in P V); with a
 *    NaN/Inf score (from Q or K), query t +- 16 of t's 32-row block gets a
 *    NaN output row (the sum of rounded probabilities that divides O is
 *    taken for both rows in one matrix op).  LSE is unaffected by either.
 *  - Range (bf16 inputs): the softmax keeps a per-row reference that moves
 *    only when a score exceeds it by more than 64 in log2 units, so an
 *    unnormalised output element can reach n * 2^64 * max|v| for a row with
 *    n visible keys.  Outputs are finite whenever max|v| * n < 2^64 (fp32
 *    accumulators overflow at 2^128); beyond that an output may become inf
 *    where the exact result is finite.  The fp32 path keeps a true running
 *    max and has no such limit.
 *  - Calls are thread-safe.  The only state kept between calls is a cache of
 *    each device's compute-unit count, filled on first use with atomic
 *    stores of the same value.
 */
#ifndef SHATTN_H
#define SHATTN_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define SHATTN_API __attribute__((visibility("default")))
#else
#define SHATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SHATTN_OK = 0,
  SHATTN_EINVAL = 1,       /* bad pointer, size, stride, alignment or rank  */
  SHATTN_EUNSUPPORTED = 2, /* valid request this build does not implement   */
  SHATTN_EHIP = 3          /* the HIP runtime reported an error at launch   */
} shattn_status;

typedef enum { SHATTN_BF16 = 0, SHATTN_F32 = 1 } shattn_dtype;

/*
 * Problem description shared by attn_chunk_fwd and attn_shifted_fwd.
 *
 * Q is [batch, heads_q, seq_q, head_dim]; K and V are
 * [batch, heads_kv, seq_kv, head_dim]; O is [batch, heads_q, seq_q, head_dim].
 * Strides are in ELEMENTS of the tensor's own dtype, for the (batch, head,
 * sequence) axes; the head_dim axis must be contiguous (stride 1).  A
 * sequence stride above 2^24 elements, more than 2^31 - 64 key rows in one
 * call (kv_len, kv_len_total), or ceil(seq_q / R) * batch * heads_q above
 * 2^31 - 1 (R = 64 for bf16 inputs with heads_q / heads_kv a multiple of 4,
 * 256 for other bf16 inputs, 128 for fp32) is refused with
 * SHATTN_EUNSUPPORTED.
 *
 * Query head h reads KV head h / (heads_q / heads_kv) (contiguous GQA
 * groups; heads_q == heads_kv is MHA).
 *
 * Query row t sits at global position q_pos0 + t.  With causal != 0, the key
 * at global position p is visible to it iff p <= q_pos0 + t (inclusive).
 * Scores are scale * (q . k); scale <= 0 selects 1/sqrt(head_dim).
 * LSE values are natural logarithms of sum_k exp(score_k).
 */
typedef struct {
  int32_t batch, heads_q, heads_kv, head_dim; /* head_dim must be 128       */
  int64_t seq_q;                              /* Q-shard rows, >= 0         */
  int64_t q_pos0;                             /* global position of Q row 0 */
  int32_t causal;                             /* 0 or 1                     */
  float scale;                                /* <= 0: 1/sqrt(head_dim)     */
  int32_t in_dtype;                           /* shattn_dtype of Q, K, V    */
  int32_t out_dtype;                          /* O dtype (attn_shifted_fwd) */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
} shattn_desc;

/*
 * attn_chunk_fwd — partial attention of the Q shard against ONE KV chunk.
 *
 * k, v point at the chunk's row 0 (global position kv_pos0); the chunk has
 * kv_len rows (>= 0).  Writes the chunk's normalized partial output
 * o_part (fp32, strided by desc->o_stride in fp32 elements) and its LSE
 * lse_part (fp32, contiguous [batch, heads_q, seq_q]).  A row with no
 * visible key in the chunk (kv_len == 0, or every key causally after it)
 * gets O = 0 and LSE = -inf: the identity of lse_merge.
 * desc->out_dtype is ignored (o_part is always fp32).
 *
 * Requirements: 16-byte aligned q, k, v, o_part; every (b, h, s) stride a
 * multiple of 16 bytes; in_dtype BF16 or F32.
 */
SHATTN_API int attn_chunk_fwd(const shattn_desc* desc, const void* q, const void* k, const void* v,
                   int64_t kv_len, int64_t kv_pos0, float* o_part, float* lse_part,
                   hipStream_t stream);

/*
 * attn_chunk_fwd_accumulate — attn_chunk_fwd merged into a running pair.
 *
 * The same partial as attn_chunk_fwd, merged in the kernel's epilogue into
 * (o_acc, lse_acc) with lse_merge's arithmetic instead of being written out:
 * (o_acc, lse_acc) <- merge((o_acc, lse_acc), (O_c, LSE_c)).  A chunk
 * consumed this way is never written as a separate fp32 partial and merged
 * by a second pass: the running result moves where it is needed (digest,
 * section "The hidden cost of synchronized operators"; summary, section
 * 核心方法).  o_acc is fp32, strided by desc->o_stride in fp32 elements;
 * lse_acc fp32 contiguous [batch, heads_q, seq_q]; an accumulator row with
 * LSE -inf is empty (its O must be 0).  A row with no visible key in the
 * chunk keeps its accumulator (the merge identity).  Requirements as
 * attn_chunk_fwd.  Calls that merge into the same rows must be ordered on
 * one stream.
 */
SHATTN_API int attn_chunk_fwd_accumulate(const shattn_desc* desc, const void* q, const void* k,
                                         const void* v, int64_t kv_len, int64_t kv_pos0,
                                         float* o_acc, float* lse_acc, hipStream_t stream);

/*
 * lse_merge — in place, row by row:
 *   (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_part, lse_part))
 * with M = max(L_a, L_b), L = M + log(exp(L_a - M) + exp(L_b - M)),
 * O = exp(L_a - L) O_a + exp(L_b - L) O_b.  Two empty rows (both LSE -inf)
 * give O = 0, LSE = -inf; an empty side contributes nothing.  This is the
 * exact decomposition of softmax over a disjoint union of key sets; the
 * pages only say that each chunk's partial output and LSE are merged.
 *
 * o_acc/o_part are contiguous fp32 [rows, head_dim]; lse_acc/lse_part are
 * contiguous fp32 [rows].  head_dim must be a multiple of 4 in [4, 256];
 * all pointers 16-byte aligned (LSE pointers 4-byte).  The two sides must
 * not alias.  rows == 0 is a valid no-op.
 */
SHATTN_API int lse_merge(int64_t rows, int32_t head_dim, float* o_acc, float* lse_acc,
              const float* o_part, const float* lse_part, hipStream_t stream);

/*
 * attn_shifted_fwd — rank `rank` of `num_chunks`, in ONE fused launch.
 *
 * k, v hold the whole KV buffer: row p is global position p, for
 * p in [0, kv_len_total).  kv_len_total must be a multiple of num_chunks;
 * chunk c covers [c*C, (c+1)*C) with C = kv_len_total / num_chunks.  Chunks
 * are visited in the order c_j = (j + rank) % num_chunks, j = 0..J-1; chunks
 * (or parts of chunks) that are causally invisible to a query tile are
 * skipped; each visited chunk's softmax partial is merged into the running
 * state with the same arithmetic as lse_merge.
 *
 * Writes O (desc->out_dtype: BF16 rounded to nearest even, or F32; strided by
 * desc->o_stride) and LSE (fp32, contiguous [batch, heads_q, seq_q]).
 * Rows with no visible key at all get O = 0, LSE = -inf.
 *
 * Requirements: as attn_chunk_fwd, plus 0 <= rank < num_chunks.
 */
SHATTN_API int attn_shifted_fwd(const shattn_desc* desc, const void* q, const void* k, const void* v,
                     int64_t kv_len_total, int32_t num_chunks, int32_t rank, void* o,
                     float* lse, hipStream_t stream);

/*
 * attn_shifted_fwd_overlapped — the chunk walk of attn_shifted_fwd with each
 * chunk's K/V rows fetched while the chunks before it compute: the shifted
 * schedule's overlap of the next chunk's transfer with local attention
 * (Silicon & Systems digest of Mercury, section "The hidden cost of
 * synchronized operators"; papers.lqhl.me summary, section 核心方法: remote
 * chunks are moved when their consumer needs them).  On one GPU the source
 * stands in for the peer that holds the chunk.
 *
 * k, v: the device KV buffers (whole length), which on entry hold the
 * rank's own chunk, chunk `rank`.  k_src, v_src: where the other chunks'
 * rows come from: pinned host memory (hipHostMalloc) or memory of another
 * device, laid out with desc->k_stride / v_stride like k, v (sequence
 * strides >= head_dim).  The own chunk is computed first, at once; for
 * j = 1..J-1 and c = (j + rank) % num_chunks, the call enqueues on
 * copy_stream the copy of chunk c's rows of every (batch, KV head) slice,
 * and on compute_stream, behind an event on those copies, the partial of Q
 * against chunk c merged into (o, lse) in the kernel's epilogue
 * (attn_chunk_fwd_accumulate): the copy of each chunk runs while the chunks
 * before it compute, and no partial is written or merged separately.  A causal
 * chunk that starts after the last query's position is neither copied nor
 * computed (its rows of k, v are left as they were).
 *
 * Outputs: o, fp32, contiguous [batch, heads_q, seq_q, head_dim] (so
 * desc->o_stride must be the contiguous strides; desc->out_dtype is
 * ignored), and lse, fp32 [batch, heads_q, seq_q], which must not overlap.
 * Results equal attn_chunk_fwd over the first visited chunk followed by
 * attn_chunk_fwd_accumulate over the others in visit order, which equals
 * attn_shifted_fwd up to rounding.
 *
 * Streams: copy_stream first waits for the work already enqueued on
 * compute_stream (which may still read k, v); compute_stream ends after all
 * of the call's work.  The two streams must differ (two null streams are
 * rejected).  The call creates and destroys HIP events; it allocates no
 * memory and never synchronizes.  Arguments are checked before anything is
 * enqueued; a HIP error while enqueuing returns SHATTN_EHIP, with the work
 * enqueued before it left in the streams.
 */
SHATTN_API int attn_shifted_fwd_overlapped(const shattn_desc* desc, const void* q,
                                const void* k_src, const void* v_src, void* k, void* v,
                                int64_t kv_len_total, int32_t num_chunks, int32_t rank,
                                float* o, float* lse, hipStream_t compute_stream,
                                hipStream_t copy_stream);

/*
 * Shifted all-gather GEMM: one rank's share of a tensor-parallel product
 * whose shared operand stays sharded and is consumed piece by piece in a
 * rank-staggered order (Silicon & Systems digest of Mercury, section "The
 * hidden cost of synchronized operators": each rank owns a slice of one
 * matrix, all ranks need the other, and the schedule shifts the order in
 * which ranks consume the shared buffer; measured as the all-gather GEMM in
 * section "What Mercury finds that templates miss").  The shift order is
 * CommIR's (j + i) % J (papers.lqhl.me summary, section 核心方法).
 *
 * A [m, k]: the gathered activation, bf16, row-major (row stride lda
 * elements); its rows form num_chunks equal chunks, chunk c being rows
 * [c*m/J, (c+1)*m/J) (the piece rank c holds).  W [n, k]: the rank's weight
 * shard, bf16, row-major out x in (row stride ldw).  C [m, n] = A W^T,
 * row-major (row stride ldc), in out_dtype (bf16 rounded to nearest even
 * from the fp32 accumulator, or fp32).  Chunks are visited in the order
 * c_j = (j + rank) % num_chunks: output tiles of chunk c_j are started
 * before those of c_{j+1}.  The result does not depend on the order.
 */
typedef struct {
  int64_t m, n, k;       /* C [m, n] = A [m, k] W [n, k]^T; k == 0 writes zeros */
  int64_t lda, ldw, ldc; /* row strides in elements (>= k, k, n)             */
  int32_t out_dtype;     /* shattn_dtype of C                                */
} shattn_gemm_desc;

/*
 * allgather_gemm_shifted — C = A W^T in one launch, A's chunks visited from
 * chunk `rank` on.
 *
 * Requirements: 0 <= rank < num_chunks; m a multiple of num_chunks; k a
 * multiple of 64 and n of 8 (else SHATTN_EUNSUPPORTED); lda, ldw multiples
 * of 8 and ldc of 8 (bf16 C) or 4 (fp32 C); a, w, c 16-byte aligned; lda,
 * ldw at most 2^22 (SHATTN_EUNSUPPORTED beyond).  m == 0 or n == 0 is a
 * successful no-op.  Pointers are device memory owned by the caller; the
 * call enqueues one kernel on `stream` and allocates nothing.
 */
SHATTN_API int allgather_gemm_shifted(const shattn_gemm_desc* desc, const void* a, const void* w,
                                      void* c, int32_t num_chunks, int32_t rank,
                                      hipStream_t stream);

/* attn_status_string — static, NUL-terminated name of a status code. */
SHATTN_API const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SHATTN_H */
