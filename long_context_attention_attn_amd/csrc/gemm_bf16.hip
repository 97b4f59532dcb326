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
// 8 x 8 blocks of 16 x 16 in accumulator registers.  Tiles never straddle a
// chunk: each chunk's rows are tiled on their own, and tiles are numbered in
// visit order.  The hardware deals workgroups round-robin to the 8 XCDs.
// With 8 or more column tiles the XCDs form 4 row groups x 2 column halves:
// XCD x takes the row tiles x / 2, x / 2 + 4, ... of that order, each with
// the column tiles of half x % 2, so one XCD's L2 serves an A tile to the
// workgroups of its half and each XCD streams only half of W (about 30 %
// fewer L2 fills than every XCD taking all columns; 3 % faster).  With fewer
// column tiles XCD x takes the row tiles x, x + 8, ... with all columns.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16 with A-operand = W rows and
// B-operand = A rows, so each 16 x 16 result block is C^T: lane l holds C
// row l % 16 of the block, columns 4 (l / 16) .. + 3.  On this chip the
// engine clock is held down by power under a dense product, and the
// 16 x 16 x 32 ops cost less energy per flop than 32 x 32 x 16 ones (a
// quarter of the accumulator registers per op for half the flops): the same
// loop with the larger ops ran at a clock about 12 % lower for the same
// cycles.  The ops are inline assembly so that each accumulator stays in
// one AGPR quad; with the compiler's builtin the register allocator moved
// accumulators between registers around every op.
//
// Data movement.  K advances 32 at a time through a 5-deep LDS ring per
// operand (global_load_lds_dwordx4 straight from global memory; a slot is
// 256 rows of 64 bytes, 16 KB; the two rings fill the 160 KB of LDS), so the
// copies of a step are issued four steps ahead: with one wave per SIMD
// nothing else hides the memory latency.  16-byte chunks are XOR-swizzled by
// (row >> 2) & 3 so that the operand reads (one 16-byte chunk per lane, 16
// rows by 4 chunks per instruction) meet no bank conflicts.  A step is 64
// matrix ops in two halves with one barrier between them; each half issues
// 4 of the 8 copies of step + 4, and the second half reads all of step + 1's
// operands, so a step's ops never wait on LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace shattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kTileK = 32;                    // K per ring slot
constexpr int kRowBytes = kTileK * 2;         // 64 bytes per operand row in LDS
constexpr int kSlotBytes = 256 * kRowBytes;   // 16 KB per operand per slot
constexpr int kStages = 5;                    // ring depth
constexpr int kCopies = 8;                    // 1 KB copies per wave per step
constexpr int kThreads = 256;
constexpr int kSplitColsFrom = 8;  // column tiles from which the XCDs split the columns

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

// One 16x16x32 bf16 matrix op into an accumulator held in AGPRs.  As inline
// assembly the accumulator cannot be moved between registers around it.
__device__ __forceinline__ void mfma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ const void* uniform(const void* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Waits until at most 24 (20) of this wave's copies are in flight.
__device__ __forceinline__ void wait_copies_24() { __builtin_amdgcn_s_waitcnt(0x4F78); }
__device__ __forceinline__ void wait_copies_20() { __builtin_amdgcn_s_waitcnt(0x4F74); }

// Workgroup barrier; the wave's own LDS reads are complete before it arrives.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), seen by the compiler's wait tracking
  __builtin_amdgcn_s_barrier();
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
  // Within an XCD, consecutive workgroups take the column tiles of one row
  // tile, row tile after row tile.
  const int bid = (int)blockIdx.x;
  const int xcd = bid & 7;
  const int local = bid >> 3;
  int mt_seq, nt;  // position of the row tile in visit order; column tile
  if (p.n_tiles_n >= kSplitColsFrom) {
    // 4 row groups x 2 column halves: XCD x takes the row tiles x / 2,
    // x / 2 + 4, ... and the columns of half x % 2.
    const int xr = xcd >> 1, xc = xcd & 1;
    const int half0 = (p.n_tiles_n + 1) >> 1;
    const int ncols = xc == 0 ? half0 : p.n_tiles_n - half0;
    const int group = local / ncols;
    nt = (xc == 0 ? 0 : half0) + (local - group * ncols);
    mt_seq = 4 * group + xr;
  } else {
    const int group = local / p.n_tiles_n;
    nt = local - group * p.n_tiles_n;
    mt_seq = 8 * group + xcd;
  }
  if (mt_seq >= p.n_tiles_m) return;  // whole workgroup: uniform exit
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

  // Operand reads (16x16x32 ops): block b of this wave, row 16 b + lane % 16
  // of the wave's 128 rows, logical chunk lane / 16 (the whole 32-deep step).
  const int wm = wave >> 1, wn = wave & 1;
  int rd_off[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int r = 16 * b + (lane & 15);
    rd_off[b] = r * kRowBytes + swz(r, lane >> 4) * 16;
  }
  const char* a_rd = &lds_a[0][0] + wm * 128 * kRowBytes;
  const char* w_rd = &lds_w[0][0] + wn * 128 * kRowBytes;

  f32x4 acc[8][8];  // [a block (C rows)][w block (C columns)], each C^T
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[i][jj] = (f32x4){};

  const int nk = (int)(p.k / kTileK);
  bf16x8 av[2][8], wv[2][8];
  if (nk > 0) {
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
#pragma unroll
      for (int n = 0; n < kCopies; ++n) copy_n(min(st, nk - 1), st, n);
    wait_copies_24();
    barrier();
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      av[0][b] = *(const bf16x8*)(a_rd + rd_off[b]);
      wv[0][b] = *(const bf16x8*)(w_rd + rd_off[b]);
    }
  }
  // K loop.  Step ks sits in slot ks % 5; its operands are already in
  // registers (buffer ks & 1), read during step ks - 1.  Slot ks - 1 was last
  // read before the previous barrier, so both halves of step ks refill it
  // with the copies of step ks + 4.  At the barrier this wave's copies of
  // step ks + 1 have landed (at most the later steps' 8 + 8 and this step's
  // first 4 are in flight); the barrier makes everyone's visible, and the
  // second half reads them.  Past the last step the copies repeat it into
  // slots nothing reads, so every step issues the same copies and the wait
  // counts stay constant.  K is a multiple of 64: steps come in pairs.
  int slot = 0;
  auto step = [&](int ks, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr int nxt = cur ^ 1;
    const int fill = slot == 0 ? kStages - 1 : slot - 1;
    const int next = slot == kStages - 1 ? 0 : slot + 1;
    const int ks_fill = min(ks + kStages - 1, nk - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        mfma16(acc[q][jj], wv[cur][jj], av[cur][q]);
        if (jj == 4) copy_n(ks_fill, fill, q);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_copies_20();
    barrier();
    const char* an = a_rd + next * kSlotBytes;
    const char* wn_ = w_rd + next * kSlotBytes;
#pragma unroll
    for (int q = 4; q < 8; ++q) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        mfma16(acc[q][jj], wv[cur][jj], av[cur][q]);
        // The next step's W operands first (its first ops need all of them),
        // then its A operands in the order its ops use them.
        if (jj % 2 == 1) {
          const int r = 4 * (q - 4) + jj / 2;  // 0..15 over the half
          if (r < 8)
            wv[nxt][r] = *(const bf16x8*)(wn_ + rd_off[r]);
          else
            av[nxt][r - 8] = *(const bf16x8*)(an + rd_off[r - 8]);
        }
        if (jj == 4) copy_n(ks_fill, fill, q);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    slot = next;
  };
  for (int ks = 0; ks < nk; ks += 2) {
    step(ks, std::integral_constant<int, 0>{});
    step(ks + 1, std::integral_constant<int, 1>{});
  }
  // The repeated copies of the last steps land before the workgroup's LDS
  // can be handed to another workgroup.
  __builtin_amdgcn_s_waitcnt(0xF70);
  // The last matrix ops' results settle before vector code reads them (the
  // compiler does not see the latency of the assembly ops).
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) asm volatile("" : "+a"(acc[i][jj]));

  // Epilogue.  C is written once and never read here: non-temporal stores keep
  // it from displacing A and W tiles from L2 (-3.8 % launch time).  Block
  // (i, jj) holds C rows 128 wm + 16 i + lane % 16 and
  // columns 128 wn + 16 jj + 4 (lane / 16) .. + 3 in its 4 registers.
  if constexpr (sizeof(TOut) == 2) {
    // bf16 C goes through LDS (the ring is idle: every copy has landed and,
    // after the barrier, every wave is past its operand reads) and leaves as
    // 16-byte pieces of whole rows: 4 rows of 256 bytes per store.  Each
    // wave stages its 128 x 128 quarter in its own area, rows padded to 272
    // bytes (conflict-free for both the 8-byte writes and 16-byte reads).
    barrier();
    constexpr int kStageRow = 272;
    char* stage = (wave < 2 ? &lds_a[0][0] : &lds_w[0][0]) + (wave & 1) * (128 * kStageRow);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const f32x4 v = acc[i][jj];
        const bf16x4 x = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *(bf16x4*)(stage + (16 * i + (lane & 15)) * kStageRow + (16 * jj + 4 * (lane >> 4)) * 2) = x;
      }
    const int cc = 128 * wn + 8 * (lane & 15);
#pragma unroll
    for (int s4 = 0; s4 < 32; ++s4) {
      const int r = 4 * s4 + (lane >> 4);
      const u32x4 x = *(const u32x4*)(stage + r * kStageRow + (lane & 15) * 16);
      if (128 * wm + r < rows && cc < cols)
        __builtin_nontemporal_store(x, (u32x4*)((TOut*)p.c + (row0 + 128 * wm + r) * p.ldc + col0 + cc));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 128 * wm + 16 * i + (lane & 15);
      if (r >= rows) continue;
      TOut* crow = (TOut*)p.c + (row0 + r) * p.ldc + col0;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int cc = 128 * wn + 16 * jj + 4 * (lane >> 4);
        if (cc >= cols) continue;
        __builtin_nontemporal_store(acc[i][jj], (f32x4*)(crow + cc));
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, DType out, hipStream_t stream) {
  if (p.n_tiles_m == 0 || p.n_tiles_n == 0) return hipSuccess;
  const int64_t blocks = p.n_tiles_n >= kSplitColsFrom
                             ? 8 * (int64_t)((p.n_tiles_m + 3) / 4) * ((p.n_tiles_n + 1) / 2)
                             : 8 * (int64_t)((p.n_tiles_m + 7) / 8) * p.n_tiles_n;
  GemmParams arg = p;
  void* args[] = {&arg};
  const void* fn = out == DType::BF16 ? (const void*)&gemm_bf16_kernel<__bf16>
                                      : (const void*)&gemm_bf16_kernel<float>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0, stream);
}

}  // namespace shattn
