// Row-wise merge of two partial attention results (O, LSE) over disjoint key
// sets, in place into the accumulator pair:
//   M = max(L_a, L_b), L = M + log(exp(L_a - M) + exp(L_b - M)),
//   O = exp(L_a - L) O_a + exp(L_b - L) O_b,
// with two empty rows (LSE -inf) staying empty.  This is how each chunk's
// partial output and log-sum-exp are merged online in a shifted schedule
// (papers.lqhl.me summary "Mercury (SOSP 2025)", section 核心方法; the pages
// leave the arithmetic to the reader, this is the exact decomposition).
//
// HBM-bound elementwise work: every row is owned by exactly one wave and each
// lane moves 16 bytes of O_a, O_b and the result, so the loads of lse_acc by
// a row's lanes all precede the single store of that row's new LSE.
//
// A merge larger than the 256 MB Infinity Cache streams from HBM: there the
// kernel loads and stores O non-temporally (3 GiB merge: 5.85 -> 6.52 TB/s;
// non-temporal loads or stores alone gave nothing).  A smaller one is left
// to the caches, which may still hold the accumulator from the previous
// merge (194 MiB merge: 6.85 TB/s cached, 6.46 non-temporal).  The result is
// bitwise the same either way.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace shattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;
constexpr int64_t kInfinityCacheBytes = 256ll << 20;

template <bool kStream>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(
    int64_t rows, int32_t head_dim, int32_t rows_per_wave, float* __restrict__ o_acc,
    float* __restrict__ lse_acc, const float* __restrict__ o_part,
    const float* __restrict__ lse_part) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kMergeThreads + threadIdx.x) >> 6;
  const int pieces = head_dim >> 2;  // 16-byte pieces per row
  const int r_local = lane / pieces;
  const int c = lane - r_local * pieces;
  const int64_t row = wave * rows_per_wave + r_local;
  if (r_local >= rows_per_wave || row >= rows) return;

  float ca, cb, lse;
  merge_weights(lse_acc[row], lse_part[row], ca, cb, lse);

  const int64_t off = row * head_dim + c * 4;
  if constexpr (kStream) {
    const f32x4 a = __builtin_nontemporal_load((const f32x4*)(o_acc + off));
    const f32x4 bv = __builtin_nontemporal_load((const f32x4*)(o_part + off));
    __builtin_nontemporal_store(a * ca + bv * cb, (f32x4*)(o_acc + off));
  } else {
    const f32x4 a = *(const f32x4*)(o_acc + off);
    const f32x4 bv = *(const f32x4*)(o_part + off);
    *(f32x4*)(o_acc + off) = a * ca + bv * cb;
  }
  if (c == 0) lse_acc[row] = lse;
}

}  // namespace

hipError_t launch_lse_merge(int64_t rows, int32_t head_dim, float* o_acc, float* lse_acc,
                            const float* o_part, const float* lse_part, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int32_t pieces = head_dim / 4;
  const int32_t rows_per_wave = 64 / pieces;
  const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
  const int64_t blocks = (waves * 64 + kMergeThreads - 1) / kMergeThreads;
  int32_t hd = head_dim, rpw = rows_per_wave;
  int64_t r = rows;
  void* args[] = {&r, &hd, &rpw, &o_acc, &lse_acc, (void*)&o_part, (void*)&lse_part};
  // Bytes of the merge: O_a, O_b and the result, three LSEs.
  const int64_t bytes = rows * (3 * (int64_t)head_dim * 4 + 3 * 4);
  const void* fn = bytes > kInfinityCacheBytes ? (const void*)&lse_merge_kernel<true>
                                               : (const void*)&lse_merge_kernel<false>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kMergeThreads), args, 0, stream);
}

}  // namespace shattn
