// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace shattn {

// Everything one forward launch needs.  Positions are global token positions.
// Key row r of the K/V buffers sits at global position kv_pos0 + r.  The
// buffer is walked as num_chunks chunks of chunk_len rows, chunk c covering
// [kv_pos0 + c*chunk_len, kv_pos0 + (c+1)*chunk_len), visited in the order
// (j + rank) % num_chunks.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sh, q_ss;  // element strides (batch, head, seq)
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t seq_q;
  int64_t q_pos0;
  int64_t kv_pos0;
  int64_t chunk_len;
  int32_t batch, heads_q, heads_kv, group;  // group = heads_q / heads_kv
  int32_t num_chunks, rank;
  int32_t causal;
  float scale_log2;  // softmax scale times log2(e)
  int32_t num_q_tiles;
  // The same walk relative to key row 0 of the buffer: its row count
  // (< 2^31), the first row of the visit order (rank * chunk_len), and
  // q_pos0 - kv_pos0 (the position of query row 0 relative to key row 0).
  int32_t kv_rows;
  int32_t seg_a0;
  int64_t q_rel0;
  // With fp32 output only: merge the result into (o, lse), which hold a
  // running (O, LSE) pair, instead of overwriting them (lse_merge's
  // arithmetic, in the kernel's epilogue).
  int32_t accumulate;
  // bf16 kernel: 1 if a work item is 64 query rows of 4 query heads that
  // share a KV head (one head per wave), 0 if it is 256 rows of one head.
  int32_t quad_heads;
};

// Weights and LSE of the merge of (O_a, L_a) with (O_b, L_b):
// O = wa O_a + wb O_b, L = lse; two empty sides (-inf) give wa = wb = 0 and
// lse = -inf.  The same operations as the standalone merge kernel.
__device__ __forceinline__ void merge_weights(float la, float lb, float& wa, float& wb,
                                              float& lse) {
  const float mx = fmaxf(la, lb);
  const bool both_empty = (mx == -INFINITY);
  const float ms = both_empty ? 0.f : mx;
  const float ea = __expf(la - ms);
  const float eb = __expf(lb - ms);
  const float tot = ea + eb;
  wa = both_empty ? 0.f : ea / tot;
  wb = both_empty ? 0.f : eb / tot;
  lse = both_empty ? -INFINITY : ms + __logf(tot);
}

enum class DType : int { BF16 = 0, F32 = 1 };

// Query rows of a one-head work item of the forward kernels, per input type.
constexpr int kBlockMBf16 = 256;
constexpr int kBlockMF32 = 128;
inline int block_m(DType in) { return in == DType::BF16 ? kBlockMBf16 : kBlockMF32; }

// The bf16 kernel's work items.  When every KV head serves a multiple of 4
// query heads, an item is 64 query rows of 4 of them (one per wave): all four
// waves then share their causal limits, so an item's diagonal band spans one
// or two 64-key tiles instead of four, and no wave computes tiles none of its
// queries sees.  Otherwise an item is 256 rows of one head, 64 per wave.
inline bool quad_heads(DType in, int64_t group) { return in == DType::BF16 && group % 4 == 0; }
// Query rows per work item, and query heads per work item.
inline int item_rows(DType in, int64_t group) { return quad_heads(in, group) ? 64 : block_m(in); }
inline int item_heads(DType in, int64_t group) { return quad_heads(in, group) ? 4 : 1; }

// Launches the fused forward kernel on `stream`; returns the HIP launch status.
// p.num_q_tiles must equal ceil(seq_q / item_rows(in, group)), and
// p.quad_heads quad_heads(in, group).
hipError_t launch_attn_fwd(const FwdParams& p, DType in, DType out, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const FwdParams& p, DType out, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const FwdParams& p, DType out, hipStream_t stream);

// Launches the row-wise (O, LSE) merge; rows > 0, head_dim % 4 == 0, <= 256.
hipError_t launch_lse_merge(int64_t rows, int32_t head_dim, float* o_acc, float* lse_acc,
                            const float* o_part, const float* lse_part, hipStream_t stream);

// One rank's share of the shifted all-gather GEMM: C [m, n] = A [m, k] W [n, k]^T,
// A's rows in num_chunks chunks of chunk_rows visited (j + rank) % num_chunks.
// Row strides in elements; k a multiple of 64, n of 8.
struct GemmParams {
  const void* a;
  const void* w;
  void* c;
  int64_t m, n, k;
  int64_t lda, ldw, ldc;
  int64_t chunk_rows;
  int32_t num_chunks, rank;
  int32_t tiles_per_chunk;  // ceil(chunk_rows / 256)
  int32_t n_tiles_m;        // num_chunks * tiles_per_chunk
  int32_t n_tiles_n;        // ceil(n / 256)
};

hipError_t launch_gemm_bf16(const GemmParams& p, DType out, hipStream_t stream);

}  // namespace shattn
