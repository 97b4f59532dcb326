// Shifted all-gather GEMM, bf16 inputs, fp32 accumulate, for gfx950 (CDNA4).
//
// One rank's share of a tensor-parallel matrix product whose shared operand
// is sharded over the ranks: the gathered activation A [M, K] arrives as J
// row chunks, consumed in the rank-shifted order c_j = (j + rank) % J (the
// `shift` primitive of CommIR, papers.lqhl.me summary "Mercury (SOSP 2025)",
// section 核心方法; the staggered consumption of a sharded buffer is the
// temporal decoupling of the Silicon & Systems digest, section "The hidden
// cost of synchronized operators").  Each chunk's rows times the local
// weight shard W [N, K] (stored out x in) fill C's rows of that chunk:
// C = A W^T.  On one GPU every chunk is already resident; the visit order
// fixes which output tiles are produced first.
//
// Work split.  A workgroup (4 waves, one per SIMD) computes a 256 x 256 tile
// of C; wave w owns rows 128 * (w >> 1) and columns 128 * (w & 1) of it, as
// 4 x 4 blocks of 32 x 32 in accumulator registers.  Tiles never straddle a
// chunk: each chunk's rows are tiled on their own, and tiles are numbered in
// visit order.  The hardware deals workgroups round-robin to the 8 XCDs;
// XCD x takes the row tiles x, x + 8, ... of that order, each with all its
// column tiles, so one XCD's L2 serves an A tile to every workgroup that
// reads it.
//
// Matrix cores: v_mfma_f32_32x32x16_bf16 with A-operand = W rows and
// B-operand = A rows, so each 32 x 32 result block is C^T: lane l holds C
// row l % 32 of the block, columns 8 g + 4 (l / 32) .. + 3 in registers
// 4 g .. 4 g + 3, written as 8- or 16-byte pieces of C's rows.
//
// Data movement.  K advances 32 at a time through a 5-deep LDS ring per
// operand (global_load_lds_dwordx4 straight from global memory; a slot is
// 256 rows of 64 bytes, 16 KB; the two rings fill the 160 KB of LDS), so the
// copies of a step are issued four steps (about 4 K cycles) before it runs:
// with one wave per SIMD nothing else hides the memory latency.  16-byte
// chunks are XOR-swizzled by (row >> 2) & 3 so that the operand reads (one
// 16-byte chunk per lane, 32 rows by 2 chunks per wave) meet no bank
// conflicts.  A step runs 2 k-substeps of 16 matrix ops with the copies of
// step + 4 spread among the second; one barrier per step, between them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace shattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kTileK = 32;                    // K per ring slot
constexpr int kRowBytes = kTileK * 2;         // 64 bytes per operand row in LDS
constexpr int kSlotBytes = 256 * kRowBytes;   // 16 KB per operand per slot
constexpr int kStages = 5;                    // ring depth
constexpr int kSubsteps = kTileK / 16;        // matrix-op k-steps per slot
constexpr int kCopies = 8;                    // 1 KB copies per wave per step
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// Physical 16-byte chunk of logical chunk c in row r (an involution).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }

// One 1 KB global->LDS copy: 16 rows of 64 bytes.  M0 holds the LDS
// destination, the source is an SGPR base plus a per-lane byte offset.  As
// inline assembly the compiler does not make later LDS reads wait for it;
// the kernel waits explicitly before the barrier that publishes a slot.
__device__ __forceinline__ void copy_1k(uint32_t lds_dst, const void* gbase, uint32_t off) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_dst), "v"(off), "s"(gbase)
      : "memory", "m0");
}

__device__ __forceinline__ const void* uniform(const void* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Waits until at most 24 (16) of this wave's copies are in flight.
__device__ __forceinline__ void wait_copies_24() { __builtin_amdgcn_s_waitcnt(0x4F78); }
__device__ __forceinline__ void wait_copies_16() { __builtin_amdgcn_s_waitcnt(0x4F70); }

// Workgroup barrier; the wave's own LDS reads are complete before it arrives.
__device__ __forceinline__ void barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename TOut>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) char lds_a[kStages][kSlotBytes];
  __shared__ __attribute__((aligned(16))) char lds_w[kStages][kSlotBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // Workgroup -> tile.  Row tiles in visit order: chunk j-th visited is
  // c = (j + rank) % J, tiled on its own into ceil(clen / 256) row tiles.
  const int bid = (int)blockIdx.x;
  const int xcd = bid & 7;
  const int local = bid >> 3;
  const int group = local / p.n_tiles_n;
  const int nt = local - group * p.n_tiles_n;
  const int mt_seq = 8 * group + xcd;  // position of the row tile in visit order
  if (mt_seq >= p.n_tiles_m) return;   // whole workgroup: uniform exit
  const int j = mt_seq / p.tiles_per_chunk;
  const int mt = mt_seq - j * p.tiles_per_chunk;
  const int chunk = (j + p.rank) % p.num_chunks;
  const int64_t row0 = (int64_t)chunk * p.chunk_rows + (int64_t)mt * kTileM;
  const int rows = (int)min((int64_t)kTileM, (int64_t)p.chunk_rows - (int64_t)mt * kTileM);
  const int64_t col0 = (int64_t)nt * kTileN;
  const int cols = (int)min((int64_t)kTileN, p.n - col0);

  // Copies: wave w fills rows 64 w .. 64 w + 63 of both operand slots, 16
  // per instruction; lane i writes LDS row 16 n + i / 4, physical chunk
  // i % 4, which holds logical chunk swz(row, i % 4).  Rows past the tile's
  // end copy its last row (their results are never stored).
  const __bf16* abase = (const __bf16*)p.a + row0 * p.lda;
  const __bf16* wbase = (const __bf16*)p.w + col0 * p.ldw;
  const uint32_t lda_b = (uint32_t)(p.lda * 2), ldw_b = (uint32_t)(p.ldw * 2);
  uint32_t a_off[4], w_off[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = 64 * wave + 16 * n + (lane >> 2);
    const int c = swz(r, lane & 3);
    a_off[n] = (uint32_t)min(r, rows - 1) * lda_b + (uint32_t)c * 16u;
    w_off[n] = (uint32_t)min(r, cols - 1) * ldw_b + (uint32_t)c * 16u;
  }
  const uint32_t a_dst0 = lds_addr(&lds_a[0][0]) + (uint32_t)(64 * wave) * kRowBytes;
  const uint32_t w_dst0 = lds_addr(&lds_w[0][0]) + (uint32_t)(64 * wave) * kRowBytes;
  // Copy instruction n (0..7: A rows, then W rows) of K-step ks into a slot.
  auto copy_n = [&](int ks, int slot, int n) {
    if (n < 4)
      copy_1k(a_dst0 + (uint32_t)slot * kSlotBytes + 1024u * n,
              uniform(abase + (int64_t)ks * kTileK), a_off[n]);
    else
      copy_1k(w_dst0 + (uint32_t)slot * kSlotBytes + 1024u * (n - 4),
              uniform(wbase + (int64_t)ks * kTileK), w_off[n - 4]);
  };

  // Operand reads: block b of this wave, k-substep kk: row 32 b + lane % 32
  // of the wave's 128 rows, logical chunk 2 kk + lane / 32.
  const int wm = wave >> 1, wn = wave & 1;
  int rd_off[4][kSubsteps];  // [block][kk] byte offset within a slot (A and W alike)
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int kk = 0; kk < kSubsteps; ++kk) {
      const int r = 32 * b + (lane & 31);
      rd_off[b][kk] = r * kRowBytes + swz(r, 2 * kk + (lane >> 5)) * 16;
    }
  const char* a_rd = &lds_a[0][0] + wm * 128 * kRowBytes;
  const char* w_rd = &lds_w[0][0] + wn * 128 * kRowBytes;

  f32x16 acc[4][4];  // [a block (C rows)][w block (C columns)], each C^T
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = (f32x16){};

  // K loop.  Step ks sits in slot ks % 5 and runs 2 k-substeps of 16 matrix
  // ops.  The barrier sits between them: once this wave's copies of step
  // ks + 1 are in (the two later steps' copies may still fly), a barrier
  // makes everyone's visible and frees the slot of step ks - 1 (every wave is
  // past its reads).  After it the wave issues the copies of step ks + 4
  // into that slot, one after every 2 ops of the second substep, and reads
  // step ks + 1's first operands, so that the next step starts on operands
  // already in registers.  Operands are read one substep ahead throughout.
  // Past the last step the copies repeat it into slots nothing reads, so
  // every step issues the same copies and the wait counts stay constant.
  const int nk = (int)(p.k / kTileK);
  bf16x8 av[2][4], wv[2][4];
  if (nk > 0) {
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
#pragma unroll
      for (int n = 0; n < kCopies; ++n) copy_n(min(st, nk - 1), st, n);
    wait_copies_24();
    barrier();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      av[0][b] = *(const bf16x8*)(a_rd + rd_off[b][0]);
      wv[0][b] = *(const bf16x8*)(w_rd + rd_off[b][0]);
    }
  }
  int slot = 0;
  for (int ks = 0; ks < nk; ++ks) {
    const int fill = slot == 0 ? kStages - 1 : slot - 1;
    const int next = slot == kStages - 1 ? 0 : slot + 1;
    const int ks_fill = min(ks + kStages - 1, nk - 1);
    const char* ab = a_rd + slot * kSlotBytes;
    const char* wb = w_rd + slot * kSlotBytes;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      av[1][b] = *(const bf16x8*)(ab + rd_off[b][1]);
      wv[1][b] = *(const bf16x8*)(wb + rd_off[b][1]);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        acc[q4][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[0][jj], av[0][q4],
                                                              acc[q4][jj], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_copies_16();
    barrier();
    if (ks + 1 < nk) {
      const char* an = a_rd + next * kSlotBytes;
      const char* wn = w_rd + next * kSlotBytes;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        av[0][b] = *(const bf16x8*)(an + rd_off[b][0]);
        wv[0][b] = *(const bf16x8*)(wn + rd_off[b][0]);
      }
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        acc[q4][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[1][jj], av[1][q4],
                                                              acc[q4][jj], 0, 0, 0);
        if (jj & 1) copy_n(ks_fill, fill, 2 * q4 + (jj >> 1));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    slot = next;
  }
  // The repeated copies of the last steps land before the workgroup's LDS
  // can be handed to another workgroup.
  __builtin_amdgcn_s_waitcnt(0xF70);

  // Epilogue: C[row][col .. col + 3] from registers 4 g .. 4 g + 3 of block
  // (i, jj): row = 128 wm + 32 i + lane % 32, col = 128 wn + 32 jj + 8 g +
  // 4 (lane / 32).  N is a multiple of 8, so a 4-column piece is all in or
  // all out.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 128 * wm + 32 * i + (lane & 31);
    if (r >= rows) continue;
    TOut* crow = (TOut*)p.c + (row0 + r) * p.ldc + col0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cc = 128 * wn + 32 * jj + 8 * g + 4 * (lane >> 5);
        if (cc >= cols) continue;
        const f32x4 v = {acc[i][jj][4 * g], acc[i][jj][4 * g + 1], acc[i][jj][4 * g + 2],
                         acc[i][jj][4 * g + 3]};
        if constexpr (sizeof(TOut) == 2) {
          const bf16x4 x = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
          *(bf16x4*)(crow + cc) = x;
        } else {
          *(f32x4*)(crow + cc) = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, DType out, hipStream_t stream) {
  if (p.n_tiles_m == 0 || p.n_tiles_n == 0) return hipSuccess;
  const int64_t groups = (p.n_tiles_m + 7) / 8;
  const int64_t blocks = 8 * groups * p.n_tiles_n;
  GemmParams arg = p;
  void* args[] = {&arg};
  const void* fn = out == DType::BF16 ? (const void*)&gemm_bf16_kernel<__bf16>
                                      : (const void*)&gemm_bf16_kernel<float>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0, stream);
}

}  // namespace shattn
