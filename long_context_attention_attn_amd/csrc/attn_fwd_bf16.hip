// Fused shifted-chunk attention forward, bf16 inputs, for gfx950 (CDNA4).
//
// A work item is four waves, one per SIMD, of 64 query rows each (two
// 32-row query blocks): 256 rows of one (batch, query head), or, when each KV
// head serves a multiple of 4 query heads, the same 64 rows of 4 query heads
// that share one KV head (the waves then share their causal limits, so an
// item's diagonal band is one or two 64-key tiles, not four, and no wave
// computes tiles none of its queries sees).  The grid has at most
// one workgroup per CU, each working through a fixed list of items (see the
// block -> item mapping in the kernel): the hardware hands out waiting
// workgroups in bursts to whichever CUs are free, which pairs heavy causal
// items with heavy ones; a fixed list pairs heavy with light.  An item
// walks the KV chunks in the rank-shifted order c_j = (j + rank) % J (the
// `shift` primitive of CommIR, papers.lqhl.me summary "Mercury (SOSP
// 2025)", section 核心方法), 64 keys per tile, and carries the
// online-softmax state in registers across chunk boundaries.  Rescaling
// that state when a chunk starts is exactly the log-sum-exp merge of the
// chunk's partial result, so one launch computes what attn_chunk_fwd
// followed by lse_merge computes chunk by chunk.  Chunk ranges that no
// query of the workgroup can see (causal) are skipped without touching
// memory.
//
// Matrix cores (v_mfma_f32_32x32x16_bf16), per wave, query block qb and
// 64-key tile:
//   S^T[key][q] = sum_d K[key][d] Q[q][d]          2 key blocks x 8 steps
//     A = K rows from LDS (ds_read_b128), B = Q^T resident in registers.
//   O^T[d][q] += sum_key V^T[d][key] P^T[key][q]   4 d blocks x 4 steps
//     A = V^T, read from row-major V in LDS with the transposing
//         ds_read_b64_tr_b16, B = P^T taken straight from the S^T accumulator.
// In the main walk a K operand read from LDS feeds both query blocks, and so
// does a V operand (the masked tiles run one query block at a time and read
// them once per block): LDS traffic per flop is well below that of 32-row
// waves, which is what bounds the matrix cores when they are fed from LDS.
// Each lane owns one query column of S^T per query block, so the softmax
// row max/sum are in-lane reductions plus one v_permlane32_swap with the
// lane holding the other half of the keys.  Accumulator layout (lane l,
// register r): column = l % 32, row = 8*(r/4) + 4*(l/32) + (r%4).
//
// One wave per SIMD, so the overlap of matrix-core work and softmax work
// comes from one instruction stream, which issues at most one instruction
// every few cycles.  Tile j is processed in 64 half steps of one matrix-core
// op each (two ops back to back would leave the vector work behind the
// second one waiting for the matrix pipe), the two query blocks alternating;
// the softmax work rides along:
//   Q1: S of tile j, key block 0   + exp of tile j-1, key block 1 (both qb)
//   Q2: S of tile j, key block 1   + max of tile j, key block 0; all copies
//   Q3: O += P V, tile j-1, keys 0-31  + max of key block 1, reference check;
//                                        exp of tile j, key block 0, qb 1
//   Q4: O += P V, tile j-1, keys 32-63 + exp of tile j, key block 0, qb 0
// An exponential is rounded to bf16 and summed one half step after it is
// issued, so that no vector op waits on a transcendental result; K and V
// operands are read three steps ahead (the first V operands of Q3 in the
// last steps of Q2).  Scheduling barriers fix the order, and the loop is
// unrolled by the ring depth so that ring slots are compile-time constants.

// K and V tiles stream straight from global memory into a 4-deep LDS ring
// per tensor (global_load_lds_dwordx4, no registers involved): each wave
// copies 16 rows of K tile j+3 and of V tile j+2 in Q2 (past the end of
// the walk, the last tile again into a slot nothing reads, so every tile
// issues the same copies), waits for its own copies of the tiles the next
// tile needs, then all waves meet at one barrier per tile.  A slot is
// refilled only after every read of its old tile has passed that barrier.
// Tiles sit in LDS unpadded with XOR-swizzled 16-byte chunks (K: chunk ^
// (row & 15); V: chunk ^ 4*(row & 3)) so that the K reads and the
// transposing V reads are free of bank conflicts.
//
// Which tiles go where.  The hot loop (the main walk) takes, in visit order,
// the full tiles that every query of the workgroup sees: no masking.  The
// causal diagonal band and ragged ends (a few tiles per workgroup) follow in
// a second loop, one tile at a time, masked.  Softmax partials merge the
// same way in any order, so taking those tiles last changes only rounding.
//
// Reference max.  Exponentials use a per-row reference m_ref, set by the
// first tile and left alone in the hot loop while no score exceeds it by
// more than 64 (log2 units): p then stays below 2^64, and O and the row
// sums stay multiples of the same exp2(-m_ref), so the common path never
// rescales (O is modified only by matrix-core ops there).  A tile with a
// score beyond that (rare even in data with outlier keys) moves its rows'
// reference up to the tile max, in a branch: the tile's scores are shifted,
// the row sums shrink by exp2(old - new) at once and O at the end of the
// tile, after the previous tile's P V (computed in the old scale) is in.
// Each wave does this for its own rows, without waiting for the others.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "kernels.h"

namespace shattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kBlockMBf16;  // query rows of a one-head work item (4 waves x 64)
constexpr int kN = 64;                // keys per tile
constexpr int kTile = kN * 128;       // elements of one K or V tile (16 KB, unpadded)
constexpr int kTileBytes = kTile * 2;
constexpr int kRing = 4;              // LDS ring depth per stream
// The reference max of a row moves (which needs the accumulated O and l
// rescaled) only when a score exceeds it by more than this, in log2 units.
// Until then every p <= 2^64, so with n visible keys the row sum stays below
// n * 2^64 and each unnormalised output element below n * 2^64 * max|v|.
// fp32 overflows at 2^128: results are finite while max|v| * n < 2^64 (for
// example |v| < 2^33 at the 2^31-row limit of a call).  A running max would
// allow max|v| * n up to 2^128; the header states the narrower range.
constexpr float kRescaleSlack = 64.0f;
static_assert(kBlockM == kWaves * 64, "64 query rows per wave");

// The tiles a workgroup visits.  Chunk c covers key rows [c*C, (c+1)*C) of
// the buffer; visiting chunks in the order (j + rank) % J walks rows
// [rank*C, J*C) and then [0, rank*C).  With the causal limit (one past the
// workgroup's last query position, relative to row 0) that is two
// contiguous ranges, each cut into 64-row tiles from its start.  Tile
// boundaries need not fall on chunk boundaries: the keys are taken in
// exactly the visit order either way.
template <int N>
struct SlotC {
  static constexpr int value = N;
};

struct Walk {
  int a0, a_end, b0, b_end, n_a, n;
};

__device__ __forceinline__ Walk make_walk(int a0, int a_end, int b0, int b_end) {
  Walk w;
  w.a0 = a0;
  w.a_end = a_end;
  w.b0 = b0;
  w.b_end = b_end;
  w.n_a = a_end > a0 ? (a_end - a0 + kN - 1) / kN : 0;
  w.n = w.n_a + (b_end > b0 ? (b_end - b0 + kN - 1) / kN : 0);
  return w;
}

// Start row and end row (exclusive) of tile `it` of the walk.
__device__ __forceinline__ void tile_bounds(const Walk& w, int it, int& t0, int& t_end) {
  if (it < w.n_a) {
    t0 = w.a0 + kN * it;
    t_end = min(t0 + kN, w.a_end);
  } else {
    t0 = w.b0 + kN * (it - w.n_a);
    t_end = min(t0 + kN, w.b_end);
  }
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Waits until at most n (a multiple of 4 in [0, 16]) of this wave's
// global->LDS copies are still in flight.
__device__ __forceinline__ void wait_copies(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0xF70); break;   // vmcnt(0)
    case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;   // vmcnt(4)
    case 8: __builtin_amdgcn_s_waitcnt(0xF78); break;   // vmcnt(8)
    case 12: __builtin_amdgcn_s_waitcnt(0xF7C); break;  // vmcnt(12)
    default: __builtin_amdgcn_s_waitcnt(0x4F70); break; // vmcnt(16)
  }
}

// Workgroup barrier without the release fence __syncthreads() adds: that
// fence would wait for every global->LDS copy in flight, including the
// prefetches of later tiles.  Copies a barrier must publish are waited for
// explicitly with wait_copies().  The wave's own LDS reads are complete
// before it arrives.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Global -> LDS copy of one 64-row tile of K or V by the four waves.  Wave w
// copies rows 16*w .. 16*w+15 with four 1 KB instructions; lane i of
// instruction n writes LDS chunk i of rows 16*w + 4*n + i/16, i.e. physical
// 16-byte chunk i%16 of that row, which holds logical chunk (i%16) ^ swz(row).
// The source address is a wave-uniform base in SGPRs plus a per-lane 32-bit
// byte offset.  K (swz = row & 15) keeps one offset per instruction; for V
// (swz = 4*(row & 3) = 4*(i/16)) the offset is the same for all four and the
// row step goes into the base.  In a ragged tile, rows past its end copy its
// last row instead (in bounds; their keys are masked and their P is 0).
struct CopyLanes {
  uint32_t k_off[4];  // K: byte offset of instruction n's source in a full tile
  uint32_t v_off;     // V: byte offset within 4 rows, same for every n
  uint32_t v_offn[4]; // V: v_off plus 4 n rows (full tiles)
};

__device__ __forceinline__ uint32_t k_chunk(int row, int lane) {
  return (uint32_t)((lane & 15) ^ (row & 15)) * 16u;
}
__device__ __forceinline__ uint32_t v_chunk(int row, int lane) {
  return (uint32_t)((lane & 15) ^ (4 * (row & 3))) * 16u;
}

__device__ __forceinline__ void copy_lanes_init(CopyLanes& cl, int w, int lane, uint32_t k_stride_b,
                                                uint32_t v_stride_b) {
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 16 * w + 4 * n + (lane >> 4);
    cl.k_off[n] = (uint32_t)row * k_stride_b + k_chunk(row, lane);
  }
  const int row0 = 16 * w + (lane >> 4);
  cl.v_off = (uint32_t)row0 * v_stride_b + v_chunk(row0, lane);
#pragma unroll
  for (int n = 0; n < 4; ++n) cl.v_offn[n] = cl.v_off + (uint32_t)(4 * n) * v_stride_b;
}

// One 1 KB copy instruction.  Written as inline assembly on purpose: through
// the builtin, the compiler cannot tell which LDS bytes a copy writes and
// makes every later LDS read wait for all copies in flight, prefetches
// included.  Here every wait is explicit (wait_copies before the barrier
// that publishes a tile).  M0 holds the LDS destination; one wait state must
// separate its scalar write from the copy that reads it.  Nothing else in
// the kernel uses M0.
__device__ __forceinline__ void copy_one(uint32_t lds_addr, const __bf16* gbase, uint32_t off) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_addr), "v"(off), "s"(gbase)
      : "memory", "m0");
}

// The same copy in two parts, for the hot loop: M0 is written one schedule
// step before the load that reads it (no wait states to fill).
__device__ __forceinline__ void set_m0(uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0" : : "s"(lds_addr) : "m0");
}
// M0 = base + off, off a constant once the caller is unrolled.
__device__ __forceinline__ void set_m0_add(uint32_t base, uint32_t off) {
  asm volatile("s_add_u32 m0, %0, %1" : : "s"(base), "i"(off) : "m0");
}
__device__ __forceinline__ void copy_at_m0(const __bf16* gbase, uint32_t off) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(gbase) : "memory");
}

// A wave-uniform pointer, kept in SGPRs (the copy instructions take their
// base address from SGPRs).
__device__ __forceinline__ const __bf16* uniform_ptr(const __bf16* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const __bf16*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// One tile copy of this wave: LDS byte address of the wave's first row in the
// slot, global address of tile row 0, valid rows, row stride.
struct TileCopy {
  uint32_t dst;
  const __bf16* src;
  int rows;
  uint32_t stride_b;
};

// Instruction n (0..3) of a K tile copy.
__device__ __forceinline__ void copy_k(const TileCopy& tc, const CopyLanes& cl, int n, int w,
                                       int lane) {
  uint32_t off = cl.k_off[n];
  if (tc.rows < kN) {  // rare: ragged tile
    const int row = 16 * w + 4 * n + (lane >> 4);
    const int r = min(row, tc.rows - 1);
    off = (uint32_t)r * tc.stride_b + k_chunk(row, lane);
  }
  copy_one(tc.dst + 1024u * n, tc.src, off);
}

// Instruction n (0..3) of a V tile copy.
__device__ __forceinline__ void copy_v(const TileCopy& tc, const CopyLanes& cl, int n, int w,
                                       int lane) {
  uint32_t off = cl.v_off;
  const __bf16* base = tc.src + (size_t)(4 * n) * (tc.stride_b >> 1);
  if (tc.rows < kN) {  // rare: ragged tile
    const int row = 16 * w + 4 * n + (lane >> 4);
    const int r = min(row, tc.rows - 1);
    off = (uint32_t)r * tc.stride_b + v_chunk(row, lane);
    base = tc.src;
  }
  copy_one(tc.dst + 1024u * n, base, off);
}

// K operand of step kk of key block kb: this lane's row is kb*32 + lq, its
// logical chunk 2*kk + hh, physical chunk logical ^ (lq & 15).  koff[kk] is
// the byte offset for key block 0; key block 1 is 32 rows (8 KB) further.
__device__ __forceinline__ bf16x8 read_k(const __bf16* ktile, const int (&koff)[8], int kb,
                                         int kk) {
  return *(const bf16x8*)((const char*)ktile + koff[kk] + kb * 8192);
}

// V^T operand of 16-key step ks, d block db: two transposing reads 8 rows
// apart.  voff[db] is this lane's byte address for step 0; step ks is 16
// rows (4 KB) further.
// The same read from a per-lane LDS byte address computed once per tile
// (the tile base plus voff[db]); the step goes into the instruction offset.
__device__ __forceinline__ bf16x8 read_v_at(uint32_t addr, int ks) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(addr + ks * 4096));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(addr + ks * 4096 + 2048));
  bf16x8 a;
  a.lo = __builtin_bit_cast(bf16x4, lo);
  a.hi = __builtin_bit_cast(bf16x4, hi);
  return a;
}

// The same read for any V tile: vrel is the tile's LDS address minus that
// of V ring slot 0 (wrapping), vaddr0[db] this lane's address in slot 0.
__device__ __forceinline__ bf16x8 read_v(uint32_t vrel, const uint32_t (&vaddr0)[4], int ks,
                                         int db) {
  return read_v_at(vaddr0[db] + vrel, ks);
}

// S^T += K Q^T for one 16-deep d step, Q^T taken from AGPRs (qk_mfma0: the
// first step, accumulator starting at zero).  All matrix-core ops are
// written as assembly: the compiler otherwise places every accumulator in
// AGPRs (scores included, which the softmax then has to copy out) and keeps
// Q^T in VGPRs.  Hazards are handled by construction: an accumulator is
// read only by the next op on it or, by vector ALU code, at least eight
// matrix-core ops later; the few places that read sooner call
// matrix_settle() first.
__device__ __forceinline__ void qk_mfma(f32x16& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "a"(q));
}
__device__ __forceinline__ void qk_mfma0(f32x16& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "a"(q));
}

// O^T += V^T P^T with the accumulator in AGPRs: O is touched only by these
// ops inside the loop.  P is written by vector ALU code a quarter tile
// before the op that reads it; V comes from an LDS read the compiler waits
// for.
__device__ __forceinline__ void pv_mfma(f32x16& o, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}

// Row sums of the bf16-rounded probabilities, on the matrix cores.  O is
// divided by the sum of the very weights P V multiplied (the fp32 sum of the
// unrounded values gives the LSE): every output is then an exact convex
// combination of V rows, and the bf16 rounding of p_k moves it by
// sum_k w_k d_k (v_k - O) rather than sum_k w_k d_k v_k (d_k the relative
// rounding error), so rows dominated by a few keys keep their values.
// One 16x16x32 op per query block and 16-key step: A is a constant 0/1
// pattern, B the P^T operand of the 32x32x16 P V op.  Read with the 16x16x32
// layout (lane l: column l % 16, keys 8 * (l / 16) .. + 7), lanes c and c + 32
// hold query c's 16 keys and lanes c + 16, c + 48 query c + 16's; A row 0 is
// one on key groups 0 and 2, row 1 on groups 1 and 3.  Result: lane c < 16
// holds query c's sum in register 0 and query c + 16's in register 1
// (accumulated in fp32 over the whole walk; every other element stays 0).
// Adding the rounded values with vector instructions instead would cost
// four more per probability pair in a loop whose vector issue is the limit.
// The zeros of A still multiply the other query's probabilities: a
// non-finite probability of query t (from a NaN or Inf in Q or K) also makes
// the sum, hence the output row, of query t +- 16 of its 32-row block NaN.
__device__ __forceinline__ void psum_mfma(f32x4& acc, const bf16x8& ones, const bf16x8& p) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "a"(ones), "v"(p));
}

// O and Q^T live in AGPRs.  Reading or rescaling O goes through a VGPR
// copy made by these empty statements, so that O itself is never used by a
// vector ALU instruction: otherwise the compiler keeps O in VGPRs and copies
// it into AGPRs around every O^T op.
template <typename T>
__device__ __forceinline__ T agpr_get(const T& o) {
  T t;
  asm volatile("" : "=v"(t) : "0"(o));
  return t;
}
template <typename T>
__device__ __forceinline__ void agpr_set(T& o, const T& t) {
  asm volatile("" : "=a"(o) : "0"(t));
}

// Wait states between a matrix-core op and another instruction that reads
// or writes its result (a 32x32x16 op runs 16 passes).
__device__ __forceinline__ void matrix_settle() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Two probabilities p = exp2(s*c - m) of scores s[r], s[r+1], rounded to
// bf16 into P operand slots x, x+1 of `dst`; their fp32 values are added to
// `acc`.  (Summing the bf16 values instead would leave rows with few keys
// with a relative error of up to 2^-9 in the sum, i.e. in the LSE.)
__device__ __forceinline__ float exp_one(const f32x16& s, int r, float c, float m) {
  return exp2_fast(fmaf(s[r], c, -m));
}
// Stores two probabilities as bf16 into P^T (elements x, x+1) and adds them
// to this lane's row sum (fp32, unrounded).
__device__ __forceinline__ void store_pair(float e0, float e1, bf16x8& dst, int x, float& acc) {
  const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
  uint32_t u = __builtin_bit_cast(uint32_t, pr);
  asm volatile("" : "+v"(u));  // round here, not where the matrix op reads it
  u32x4 d = __builtin_bit_cast(u32x4, dst);
  d[x >> 1] = u;
  dst = __builtin_bit_cast(bf16x8, d);
  acc += e0 + e1;
  asm volatile("" : "+v"(acc));
}
// Exponentials of scores already scaled and shifted in place (s*c - m).
__device__ __forceinline__ float exp_s(const f32x16& s, int r) { return exp2_fast(s[r]); }

__device__ __forceinline__ void exp_pair(const f32x16& s, int r, float c, float m, bf16x8& dst,
                                         int x, float& acc) {
  const float e0 = exp_one(s, r, c, m);
  const float e1 = exp_one(s, r + 1, c, m);
  store_pair(e0, e1, dst, x, acc);
}

// NaN-propagating maximum (v_maximum3_f32 on gfx950; unlike fmaxf it needs
// no operand canonicalisation).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float lane_swap32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_swap32_add(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait states for the matrix ops writing acc to retire, as an asm statement
// that names acc: no read of it can be scheduled ahead of the wait.
__device__ __forceinline__ void settle_acc(f32x4& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc) : : "memory");
}

// Scales the rounded-P sums of a query block by a per-query factor f (lane
// l holds query l % 32's): lane c < 16 keeps query c in register 0 and query
// c + 16 in register 1.
__device__ __forceinline__ void scale_lr(f32x4& acc, float f) {
  const float f16 = __shfl_down(f, 16);
  settle_acc(acc);
  f32x4 t = agpr_get(acc);
  t[0] *= f;
  t[1] *= f16;
  agpr_set(acc, t);
}

// The rounded-P sum of this lane's query (l % 32), from psum_mfma's layout.
__device__ __forceinline__ float lr_total(f32x4& acc, int lq) {
  settle_acc(acc);
  const f32x4 t = agpr_get(acc);
  const float a = __shfl(t[0], lq & 15);
  const float b = __shfl(t[1], lq & 15);
  return lq < 16 ? a : b;
}

template <typename TOut>
__device__ __forceinline__ void store4(TOut* dst, const f32x4& v);

template <>
__device__ __forceinline__ void store4<float>(float* dst, const f32x4& v) {
  *(f32x4*)dst = v;
}

template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, const f32x4& v) {
  bf16x4 x = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  *(bf16x4*)dst = x;
}

// Makes the compiler wait for outstanding loads into v before going on.
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

// kQuad: an item is 64 query rows of 4 query heads of one KV head's group (wave
// w takes head 4 g + w), else 256 rows of one head (wave w takes rows
// 64 w .. 64 w + 63).  A compile-time choice: chosen at run time, the
// register allocator spilled per-lane constants to scratch.
template <typename TOut, bool kQuad>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_bf16_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 lds_k[kRing][kTile];
  __shared__ __attribute__((aligned(16))) __bf16 lds_v[kRing][kTile];
  // All zeros: the V tile P V reads when every query of the wave is past
  // the tile (P known to be zero), so that non-finite values in a V tile no
  // query of the wave can see never reach it through 0 * NaN.
  __shared__ __attribute__((aligned(16))) __bf16 lds_vzero[kTile];
  // Wave 3's staging area for its Q rows (waves 0-2 stage theirs in K ring
  // slot 3, V ring slot 2 and the zero tile, all free at an item's start).
  __shared__ __attribute__((aligned(16))) __bf16 lds_qx[kTile];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in [0, 4)
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hh = lane >> 5;

  // Blocks -> work items (b, kv head, query head of its group or group of 4
  // of them, query tile).
  // The grid holds at most one block per CU; each block walks a list of
  // items.  The hardware deals consecutive blocks round-robin to the 8 XCDs:
  // when the KV heads split evenly, the blocks of XCD x share the items of
  // KV heads x, x+8, ... (its L2 then serves their common K/V tiles).  A
  // list runs KV head by KV head, each head's items heaviest (latest query
  // tile, for causal) first, and is dealt to the blocks sharing it in rounds
  // of alternating direction, so that heavy and light items pair up.
  const int n_blocks = (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  const int nkv = p.batch * p.heads_kv;
  const int per_tile = kQuad ? p.group >> 2 : p.group;  // items per query tile and KV head
  const int per_head = per_tile * p.num_q_tiles;
  const bool by_xcd = (nkv & 7) == 0 && (n_blocks & 7) == 0;
  const int lanes = by_xcd ? (n_blocks >> 3) : n_blocks;
  const int lidx = by_xcd ? (bid >> 3) : bid;
  const int xcd = by_xcd ? (bid & 7) : 0;
  const int n_list = (by_xcd ? (nkv >> 3) : nkv) * per_head;
  for (int round = 0;; ++round) {
  const int item = round * lanes + ((round & 1) ? lanes - 1 - lidx : lidx);
  if (item >= n_list) break;
  const int kvi = (by_xcd ? xcd + 8 * (item / per_head) : item / per_head);
  const int i_in = item % per_head;
  const int qt = p.num_q_tiles - 1 - i_in / per_tile;
  const int g = i_in % per_tile;
  const int hk = kvi % p.heads_kv;
  const int b = kvi / p.heads_kv;
  const int h = hk * p.group + (kQuad ? 4 * g + wave : g);  // this wave's query head
  // Every wave is done with the previous item's LDS tiles.
  if (round > 0) __syncthreads();

  constexpr int rows_item = kQuad ? 64 : kBlockM;
  const int64_t q_start = (int64_t)qt * rows_item;
  const int64_t q_rows_wg = min((int64_t)rows_item, p.seq_q - q_start);
  const int64_t wave_q0 = q_start + (kQuad ? 0 : wave * 64);
  // Query positions relative to key row 0, clamped to [-1, kv_rows]: -1 sees
  // no key, kv_rows sees every key.
  const int kv_rows = p.kv_rows;
  auto rel = [&](int64_t q_index) {
    return (int)max((int64_t)-1, min(p.q_rel0 + q_index, (int64_t)kv_rows));
  };
  // The same for the first query of a 32-row block, clamped no higher than
  // -kN below, so that adding the row index keeps every row's own limit
  // exact (a row left of key 0 stays left of it).
  auto rel_block = [&](int64_t q_index) {
    return (int)max((int64_t)-kN, min(p.q_rel0 + q_index, (int64_t)kv_rows));
  };
  // One past the last key any query of the workgroup can see, and one past
  // the last key every query of it sees.
  const int limit = p.causal ? rel(q_start + q_rows_wg - 1) + 1 : kv_rows;
  const int ulim = p.causal ? rel(q_start) + 1 : kv_rows;
  // The main walk takes the full tiles every query sees, in visit order; the
  // rest (the causal diagonal band, ragged ends: at most a few tiles) comes
  // after it, with masking.  The softmax merge does not depend on the order.
  const int a0 = p.seg_a0;
  const int a_lim = min(kv_rows, limit);
  const int b_lim = min(a0, limit);
  const int a_main = a0 + kN * (max(0, min(a_lim, ulim) - a0) / kN);
  const int b_main = kN * (max(0, min(b_lim, ulim)) / kN);
  const Walk walk = make_walk(a0, a_main, 0, b_main);
  const Walk rest_walk = make_walk(a_main, a_lim, b_main, b_lim);
  const int n_tiles = walk.n;
  // Last query of the wave (below its first, rel(wave_q0), if the wave has
  // no rows).
  const int wave_q_max = rel(min(wave_q0 + 63, p.seq_q - 1));

  const __bf16* qbase = (const __bf16*)p.q + b * p.q_sb + h * p.q_sh;
  const __bf16* kbase = (const __bf16*)p.k + b * p.k_sb + hk * p.k_sh;
  const __bf16* vbase = (const __bf16*)p.v + b * p.v_sb + hk * p.v_sh;
  // The sequence strides are below 2^24 elements (checked on the host), so a
  // tile spans < 2^31 bytes.
  const uint32_t k_stride_b = (uint32_t)p.k_ss * 2u;
  const uint32_t v_stride_b = (uint32_t)p.v_ss * 2u;
  // LDS byte address of this wave's first row in ring slot 0.
  const uint32_t k_ring = lds_address(&lds_k[0][0]) + (uint32_t)(16 * wave) * 256u;
  const uint32_t v_ring = lds_address(&lds_v[0][0]) + (uint32_t)(16 * wave) * 256u;
  CopyLanes cl;
  copy_lanes_init(cl, wave, lane, k_stride_b, v_stride_b);
  auto k_copy = [&](const Walk& wk, int it, int slot) {
    TileCopy tc;
    int t0, te;
    tile_bounds(wk, it, t0, te);
    tc.dst = k_ring + (uint32_t)slot * kTileBytes;
    tc.src = kbase + (int64_t)t0 * p.k_ss;
    tc.rows = te - t0;
    tc.stride_b = k_stride_b;
    return tc;
  };
  auto v_copy = [&](const Walk& wk, int it, int slot) {
    TileCopy tc;
    int t0, te;
    tile_bounds(wk, it, t0, te);
    tc.dst = v_ring + (uint32_t)slot * kTileBytes;
    tc.src = vbase + (int64_t)t0 * p.v_ss;
    tc.rows = te - t0;
    tc.stride_b = v_stride_b;
    return tc;
  };
  auto copy_tile_k = [&](const TileCopy& tc) {
#pragma unroll
    for (int n = 0; n < 4; ++n) copy_k(tc, cl, n, wave, lane);
  };
  auto copy_tile_v = [&](const TileCopy& tc) {
#pragma unroll
    for (int n = 0; n < 4; ++n) copy_v(tc, cl, n, wave, lane);
  };

  // Q rows of the wave go through LDS: 16 copies of four whole rows each
  // (laid out and swizzled like a K tile), read back below as the Q^T
  // operands.  Rows past the end of the shard copy its last row (their
  // results are never stored).
  const __bf16* const q_stage = wave == 0 ? &lds_k[kRing - 1][0]
                              : wave == 1 ? &lds_v[2][0]
                              : wave == 2 ? lds_vzero
                                          : lds_qx;
  {
    const int64_t q_hi = p.seq_q - 1;
    const uint32_t q_stride_b = (uint32_t)p.q_ss * 2u;
    const uint32_t qdst = lds_address(q_stage);
    if (wave_q0 + 63 <= q_hi) {
      // All 64 rows exist: instruction n copies rows 4n..4n+3; the row step
      // goes into the (scalar) base, the lane offset repeats every 4 n.
      uint32_t off[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        off[m] = (uint32_t)(lane >> 4) * q_stride_b + k_chunk(4 * m + (lane >> 4), lane);
#pragma unroll
      for (int n = 0; n < 16; ++n)
        copy_one(qdst + 1024u * n, uniform_ptr(qbase + (wave_q0 + 4 * n) * p.q_ss), off[n & 3]);
    } else {
      // The shard's last rows: rows past its end copy row q_hi.
      const int64_t q_w = min(wave_q0, q_hi);
      const __bf16* qsrc = uniform_ptr(qbase + q_w * p.q_ss);
      const int r_lim = __builtin_amdgcn_readfirstlane((int)min(q_hi - q_w, (int64_t)63));
      for (int n = 0; n < 16; ++n) {
        const int row = 4 * n + (lane >> 4);
        const uint32_t r = (uint32_t)min(row, r_lim);
        copy_one(qdst + 1024u * n, qsrc, r * q_stride_b + k_chunk(row, lane));
      }
    }
  }
  // Q^T operands of both query blocks, resident in AGPRs for the whole kernel.
  bf16x8 qv[2][8];

  // Per-lane LDS byte offsets of the matrix-core operands (see read_k, read_v).
  int koff[8];
  uint32_t voff[4];  // V^T reads: this lane's LDS byte address in V ring slot 0
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = lq * 256 + (((2 * kk + hh) ^ (lq & 15)) * 16);
  {
    const int t = (lane >> 2) & 3, gq = (lane >> 4) & 1, u = lane & 3;
    const int row = 4 * hh + t;  // row & 3 == t
#pragma unroll
    for (int db = 0; db < 4; ++db)
      voff[db] = lds_address(&lds_v[0][0]) +
                 (uint32_t)(row * 256 + (((db * 4 + 2 * gq + (u >> 1)) ^ (4 * t)) * 16) + (u & 1) * 8);
  }

  const float c = p.scale_log2;
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // The main walk's first tile multiplies P = 0 into V ring slot 3 (the
    // slot of "tile -1"), which no copy writes before tile 1.  (The zero
    // tile is refilled below, once wave 2 has read its Q rows from it.)
    for (int i = tid; i < kTile / 8; i += kThreads)
      *(u32x4*)(&lds_v[kRing - 1][0] + 8 * i) = zero;
  }
  f32x16 o[2][4];
  float m_ref[2], m_use[2];  // reference max; m_use = m_ref, or 0 while it is -inf
  // In the hot loop the scores are scaled and shifted in place, s*c - m_use,
  // before their maxima are taken: a shifted score above t_far = m_ref +
  // slack - m_use is far (-inf before the first tile, which so always
  // takes the rare branch).
  float t_far[2];
  float l_run[2];            // this lane's half of the row sums (fp32 p: the LSE)
  // Sums of the rounded P (divide O), see psum_mfma; and its constant A.
  f32x4 lr[2];
  bf16x8 ones;
  // P^T operands: pb[qb][ks] holds keys 16*ks .. 16*ks+15 of the tile being
  // multiplied into O (ks 0-1: key block 0, ks 2-3: key block 1).
  bf16x8 pb[2][4];
  // Scores of the current tile; s[1][*] of tile j-1 lives on into Q1/Q2 of
  // tile j, which take its exponentials.
  f32x16 s[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int db = 0; db < 4; ++db) agpr_set(o[qb][db], (f32x16){});
    agpr_set(lr[qb], (f32x4){0.f, 0.f, 0.f, 0.f});
    m_ref[qb] = -INFINITY;
    m_use[qb] = 0.f;
    t_far[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int x = 0; x < 8; ++x) pb[qb][ks][x] = (__bf16)0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][qb][r] = -INFINITY;
  }
  {
    const int row = lane & 15, grp = lane >> 4;
    const bool one = (row == 0 && (grp & 1) == 0) || (row == 1 && (grp & 1) == 1);
    bf16x8 t;
#pragma unroll
    for (int x = 0; x < 8; ++x) t[x] = (__bf16)(one ? 1.0f : 0.0f);
    agpr_set(ones, t);
  }
  // The compiler must not know P's starting value: a known constant gets
  // rebuilt by vector moves right in front of the asm matrix ops, which do
  // not see the wait states such a move needs before a matrix-core read.
  asm volatile("" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[0][2]), "+v"(pb[0][3]),
               "+v"(pb[1][0]), "+v"(pb[1][1]), "+v"(pb[1][2]), "+v"(pb[1][3]));

  // ---- Main walk.  The first tile sets each row's reference (nothing is
  // accumulated yet); a later tile with a score more than the slack above it
  // moves the reference of the rows concerned (rare branch below).
  if (n_tiles > 0) {
    copy_tile_k(k_copy(walk, 0, 0));
    copy_tile_v(v_copy(walk, 0, 0));
  }
  if (n_tiles > 1) {
    copy_tile_k(k_copy(walk, 1, 1));
    copy_tile_v(v_copy(walk, 1, 1));
  }
  if (n_tiles > 2) copy_tile_k(k_copy(walk, 2, 2));
  wait_copies(0);
  // This wave's Q rows are in: take the operands.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) agpr_set(qv[qb][kk], read_k(q_stage, koff, qb, kk));
  if (wave == 2) {
    // Wave 2 staged its Q in the zero tile: zero it again.
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kTile / 8 / 64; ++i) *(u32x4*)(lds_vzero + 8 * (64 * i + lane)) = zero;
  }
  __syncthreads();

  int slot = 0;
  float rs_pend[2] = {0.f, 0.f};  // key-block-0 sums of tile j-1
  int it = 0;
  // Per-row factor that tile j's far-score branch leaves for O (tile j-1's
  // P V, still running then, completes in the old scale).
  float o_scale[2] = {1.f, 1.f};
  // First key rows of the next copies: K takes tile it+3, V tile it+2, both
  // clamped to the last tile; V's row is the one K took a tile earlier.
  auto main_row = [&](int i) { return i < walk.n_a ? walk.a0 + kN * i : kN * (i - walk.n_a); };
  int k_i = min(3, n_tiles - 1);
  int k_row = main_row(max(k_i, 0));
  int v_row = main_row(max(min(2, n_tiles - 1), 0));
  // The hot loop's body for a tile whose ring slot (its index mod 4) is a
  // compile-time constant: every LDS address below is then a register plus
  // an immediate.
  auto tile_body = [&](auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    // This tile copies K tile j+3 and V tile j+2 (main-walk tiles are full:
    // no row clamping).  Past the end of the walk the last tile is copied
    // again, into a ring slot no later read uses.
    const __bf16* ksrc =
        uniform_ptr((const __bf16*)((const char*)kbase + (uint64_t)(uint32_t)k_row * k_stride_b));
    const __bf16* vsrc =
        uniform_ptr((const __bf16*)((const char*)vbase + (uint64_t)(uint32_t)v_row * v_stride_b));
    const __bf16* ktile = &lds_k[slot][0];
    // Tile j-1's V^T: slot 0's read addresses plus a constant (it goes into
    // the instruction offset).
    constexpr uint32_t v_slot_off = (uint32_t)((slot + kRing - 1) & (kRing - 1)) * kTileBytes;
    bool rescale = false;  // a far score in this tile: O gets o_scale at its end
    float rh[2] = {0.f, 0.f};  // sums of tile j-1, key block 1
    float mx[2] = {-INFINITY, -INFINITY};

    // ---- Q1, Q2: S of tile j in 32 half steps of one matrix op each, the
    // two query blocks alternating on one K read.  Q1 (t < 8): key block 0,
    // with the exponentials of tile j-1's key block 1 (both query blocks, one
    // pair per half step; Q2 overwrites those scores).  Q2 (t >= 8): key
    // block 1, with the key-block-0 maxima and the copies of K tile j+3 and
    // V tile j+2 (one copy instruction per half step).
    bf16x8 va[4];
    bf16x8 ka[4];
    ka[0] = read_k(ktile, koff, 0 >> 3, 0 & 7);
    ka[1] = read_k(ktile, koff, 1 >> 3, 1 & 7);
    ka[2] = read_k(ktile, koff, 2 >> 3, 2 & 7);
    float pe0 = 0.f, pe1 = 0.f;  // exponentials issued, not yet rounded and summed
    auto copy_step = [&](int h) {  // h = 0..15: K copies 0..3, then V copies 0..3
      if (h < 8) {
        if (!(h & 1)) set_m0_add(k_ring, (uint32_t)((slot + 3) & (kRing - 1)) * kTileBytes + 1024u * (h >> 1));
        else copy_at_m0(ksrc, cl.k_off[h >> 1]);
      } else {
        if (!(h & 1)) set_m0_add(v_ring, (uint32_t)((slot + 2) & (kRing - 1)) * kTileBytes + 1024u * ((h - 8) >> 1));
        else copy_at_m0(vsrc, cl.v_offn[(h - 8) >> 1]);
      }
    };
    // Key-block-0 max of query block qb, score pair p (2 scores per lane).
    auto max_pair = [&](int qb, int p) {
      s[0][qb][2 * p] = fmaf(s[0][qb][2 * p], c, -m_use[qb]);
      s[0][qb][2 * p + 1] = fmaf(s[0][qb][2 * p + 1], c, -m_use[qb]);
      mx[qb] = vmax(vmax(mx[qb], s[0][qb][2 * p]), s[0][qb][2 * p + 1]);
    };
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int kb = t >> 3, kk = t & 7;
      // Half step A: query block 0.
      __builtin_amdgcn_sched_barrier(0);
      if (t + 3 < 16) {
        const int u = t + 3;
        ka[u % 4] = read_k(ktile, koff, u >> 3, u & 7);
      }
      // One LDS wait per two steps: step t (even) also waits for step t+1's
      // operand (read a step later than its own).
      if (!(t & 1)) asm volatile("" : : "v"(ka[(t + 1) % 4]));
      if (kk == 0) qk_mfma0(s[kb][0], ka[t % 4], qv[0][kk]);
      else qk_mfma(s[kb][0], ka[t % 4], qv[0][kk]);
      if (t < 8) {
        // Exponentials of pair kk (qb 0) now, rounding and sums of the pair
        // before it (qb 1, kk - 1) after them: an exponential's result is
        // first used a half step later.
        const float n0 = exp_s(s[1][0], 2 * kk);
        const float n1 = exp_s(s[1][0], 2 * kk + 1);
        if (t > 0) store_pair(pe0, pe1, pb[1][2 + ((kk - 1) >> 2)], (2 * (kk - 1)) & 7, rh[1]);
        pe0 = n0;
        pe1 = n1;
      } else {
        if (t == 8) store_pair(pe0, pe1, pb[1][3], 6, rh[1]);
        copy_step(2 * (t - 8));
        // qb 0's key-block-0 scores were last written in half step 7A; the
        // first read waits for two full steps.
        if (t >= 10) max_pair(0, t - 10);
        if (t >= 14) max_pair(0, t - 8);
      }
      // Half step B: query block 1.
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) qk_mfma0(s[kb][1], ka[t % 4], qv[1][kk]);
      else qk_mfma(s[kb][1], ka[t % 4], qv[1][kk]);
      if (t < 8) {
        const float n0 = exp_s(s[1][1], 2 * kk);
        const float n1 = exp_s(s[1][1], 2 * kk + 1);
        store_pair(pe0, pe1, pb[0][2 + (kk >> 2)], (2 * kk) & 7, rh[0]);
        pe0 = n0;
        pe1 = n1;
      } else {
        copy_step(2 * (t - 8) + 1);
        if (t >= 11) max_pair(1, t - 11);
        if (t >= 13) max_pair(1, t - 8);
        // The first V^T operands of Q3, three steps ahead (ka[(t+3)%4] is
        // no longer read from t = 13 on).
        if (t >= 13) {
          const int n = t - 13;
          va[n] = read_v_at(voff[n & 3] + v_slot_off, n >> 2);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- Q3, Q4: O += P V of tile j-1 (step st: keys 16*(st/4).., d
    // block st%4) ------------------------------------------------------
    //  Q3: max of key block 1 (then the reference); exp of tile j, key
    //      block 0, qb 1 (into pn: pb[1][0..1] is still being read).
    //  Q4: exp of tile j, key block 0, qb 0.
    // Key-block-1 maxima: qb 0 first (its scores were final 8 ops before the
    // end of Q2), qb 1 from the fifth half step on (its last op then lies
    // four matrix ops and their vector work back).
    // Key block 1, half steps 4..11: scale and shift two scores per query
    // block, then take their max.
    auto scale_max_kb1 = [&](int h) {
      if (h >= 4 && h < 12) {
        const int r = 2 * (h - 4);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[1][qb][r] = fmaf(s[1][qb][r], c, -m_use[qb]);
          s[1][qb][r + 1] = fmaf(s[1][qb][r + 1], c, -m_use[qb]);
          mx[qb] = vmax(vmax(mx[qb], s[1][qb][r]), s[1][qb][r + 1]);
        }
      }
    };
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      const int n = st + 3;
      va[n % 4] = read_v_at(voff[n & 3] + v_slot_off, n >> 2);
      if (!(st & 1)) asm volatile("" : : "v"(va[(st + 1) % 4]));
      pv_mfma(o[0][st & 3], va[st % 4], pb[0][st >> 2]);
      if ((st & 3) == 3) psum_mfma(lr[0], ones, pb[0][st >> 2]);
      scale_max_kb1(2 * st);
      __builtin_amdgcn_sched_barrier(0);
      pv_mfma(o[1][st & 3], va[st % 4], pb[1][st >> 2]);
      if ((st & 3) == 3) psum_mfma(lr[1], ones, pb[1][st >> 2]);
      scale_max_kb1(2 * st + 1);
      if (st == 0) {
        // Tile j-1's sums join the row sums.
        l_run[0] += rs_pend[0] + rh[0];
        l_run[1] += rs_pend[1] + rh[1];
        asm volatile("" : "+v"(l_run[0]), "+v"(l_run[1]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Common case: no lane's partial max exceeds its row's threshold.
    if (__builtin_amdgcn_ballot_w64(mx[0] > t_far[0] || mx[1] > t_far[1]) != 0) {
      bool far = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m_old = m_use[qb];
        const float m_tile = lane_swap32_max(mx[qb]) + m_old;  // max of s*c
        // No reference yet (the first tile): set it, nothing to rescale (O
        // and the row sums are zero).  A far score: the row's reference
        // moves up to it; the row sums so far (through tile j-1) shrink by
        // exp2(old - new) now, O once tile j-1's P V is in (end of tile).
        const bool first = m_ref[qb] == -INFINITY;
        const bool far_q = !first && m_tile > m_ref[qb] + kRescaleSlack;
        o_scale[qb] = far_q ? exp2_fast(m_ref[qb] - m_tile) : 1.f;
        l_run[qb] *= o_scale[qb];
        m_ref[qb] = (first || far_q) ? m_tile : m_ref[qb];
        m_use[qb] = m_ref[qb] == -INFINITY ? 0.f : m_ref[qb];
        t_far[qb] = m_ref[qb] + kRescaleSlack - m_use[qb];
        // The tile's scores were shifted by the old m_use: shift them to the
        // new one.
        const float d = m_old - m_use[qb];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[0][qb][r] += d;
          s[1][qb][r] += d;
        }
        far = far || far_q;
      }
      rescale = __builtin_amdgcn_ballot_w64(far) != 0;
    }
    bf16x8 pn[2];  // P of tile j, key block 0, qb 1
    rs_pend[0] = 0.f;
    rs_pend[1] = 0.f;
    // Exponentials of tile j, key block 0, one pair per half step from half
    // step 12 (qb 1: pairs 0..7 into pn; qb 0 from half step 20: pb[0][0..1]
    // was last read in step 7), each rounded and summed a half step later.
    auto exp_job = [&](int h) {
      const int j = h - 12;  // job index 0..15
      float n0 = 0.f, n1 = 0.f;
      if (j >= 0 && j < 16) {
        const int qb = j < 8 ? 1 : 0, i = j & 7;
        n0 = exp_s(s[0][qb], 2 * i);
        n1 = exp_s(s[0][qb], 2 * i + 1);
      }
      if (j >= 1 && j <= 16) {
        const int i = j - 1;  // commit job i
        if (i < 8) store_pair(pe0, pe1, pn[i >> 2], (2 * i) & 7, rs_pend[1]);
        else store_pair(pe0, pe1, pb[0][(i - 8) >> 2], (2 * (i - 8)) & 7, rs_pend[0]);
      }
      pe0 = n0;
      pe1 = n1;
    };
#pragma unroll
    for (int st = 6; st < 16; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      if (st + 3 < 16) {
        const int n = st + 3;
        va[n % 4] = read_v_at(voff[n & 3] + v_slot_off, n >> 2);
      }
      if (!(st & 1)) asm volatile("" : : "v"(va[(st + 1) % 4]));
      pv_mfma(o[0][st & 3], va[st % 4], pb[0][st >> 2]);
      if ((st & 3) == 3) psum_mfma(lr[0], ones, pb[0][st >> 2]);
      exp_job(2 * st);
      __builtin_amdgcn_sched_barrier(0);
      pv_mfma(o[1][st & 3], va[st % 4], pb[1][st >> 2]);
      if ((st & 3) == 3) psum_mfma(lr[1], ones, pb[1][st >> 2]);
      exp_job(2 * st + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    pb[1][0] = pn[0];
    pb[1][1] = pn[1];
    if (rescale) {
      // Rare: tile j-1's P V (old scale) is complete once its ops retire.
      matrix_settle();
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int db = 0; db < 4; ++db) agpr_set(o[qb][db], agpr_get(o[qb][db]) * o_scale[qb]);
        scale_lr(lr[qb], o_scale[qb]);
      }
    }
    {
      v_row = k_row;
      const int kn = k_i + 1;
      const bool kmore = kn < n_tiles;
      k_row = kmore ? (kn == walk.n_a ? 0 : k_row + kN) : k_row;
      k_i = kmore ? kn : k_i;
    }

    // Copies still allowed in flight: those issued after K[j+1] and V[j],
    // i.e. K[j+2], V[j+1], K[j+3], V[j+2].
    wait_copies(16);
    asm volatile("" : "+v"(pb[0][0]), "+v"(pb[0][1]), "+v"(pb[1][0]), "+v"(pb[1][1]),
                 "+v"(rs_pend[0]), "+v"(rs_pend[1])
                 :
                 : "memory");
    tile_barrier();
  };
  while (it < n_tiles) {
    tile_body(SlotC<0>());
    if (++it >= n_tiles) break;
    tile_body(SlotC<1>());
    if (++it >= n_tiles) break;
    tile_body(SlotC<2>());
    if (++it >= n_tiles) break;
    tile_body(SlotC<3>());
    ++it;
  }
  // The slot after the last tile.
  slot = n_tiles & (kRing - 1);
  wait_copies(0);
  // The rest tiles (below) continue the ring: rest tile r sits in slot
  // (n_tiles + r) mod 4.  The first two are fetched now, under the last
  // main tile's P V: no wave reads K any more (every wave passed the last
  // tile's barrier), and that P V reads only the V slot before `slot`.
  const int n_rest = rest_walk.n;
  auto copy_rest = [&](int r) {
    copy_tile_k(k_copy(rest_walk, r, (slot + r) & (kRing - 1)));
    copy_tile_v(v_copy(rest_walk, r, (slot + r) & (kRing - 1)));
  };
  if (n_rest > 0) copy_rest(0);
  if (n_rest > 1) copy_rest(1);

  // The last tile of the main walk: its key-block-1 probabilities, then its
  // P V (its V sits in the slot before `slot`; with no main walk at all P
  // is zero and that slot is the zeroed slot 3).
  {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float rh = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        store_pair(exp_s(s[1][qb], 2 * i), exp_s(s[1][qb], 2 * i + 1), pb[qb][2 + (i >> 2)],
                   (2 * i) & 7, rh);
      l_run[qb] += rs_pend[qb] + rh;
    }
    const uint32_t vrel = (uint32_t)((slot + kRing - 1) & (kRing - 1)) * kTileBytes;
    bf16x8 va[3];  // V operands two steps ahead
    va[0] = read_v(vrel, voff, 0, 0);
    va[1] = read_v(vrel, voff, 0, 1);
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      if (st + 2 < 16) va[(st + 2) % 3] = read_v(vrel, voff, (st + 2) >> 2, (st + 2) & 3);
      pv_mfma(o[0][st & 3], va[st % 3], pb[0][st >> 2]);
      pv_mfma(o[1][st & 3], va[st % 3], pb[1][st >> 2]);
      if ((st & 3) == 3) {
        psum_mfma(lr[0], ones, pb[0][st >> 2]);
        psum_mfma(lr[1], ones, pb[1][st >> 2]);
      }
    }
  }

  // ---- The rest, one tile at a time, with masking: the causal diagonal
  // band and ragged ends.  Two tiles ahead in flight.
  for (int xt = 0; xt < n_rest; ++xt) {
    int t0, t_end;
    tile_bounds(rest_walk, xt, t0, t_end);
    const int rslot = (slot + xt) & (kRing - 1);
    // This wave's copies of tile xt are in (tile xt+1's may still fly) ...
    if (xt + 1 < n_rest) wait_copies(8);
    else wait_copies(0);
    // ... and everyone's; every wave is done with tile xt-1, so tile xt+2
    // may take the slot of tile xt-2.
    tile_barrier();
    if (xt + 2 < n_rest) copy_rest(xt + 2);
    const __bf16* ktile = &lds_k[rslot][0];
    const int last = t_end - 1 - t0;
    const bool dead = (p.causal && t0 > wave_q_max) || wave_q0 >= p.seq_q;
    // P V; a wave none of whose queries sees the tile reads the zero tile.
    const uint32_t vrel =
        lds_address(dead ? lds_vzero : &lds_v[rslot][0]) - lds_address(&lds_v[0][0]);
    // Four phases of 16 matrix ops: S of query block 0, S of block 1, P V of
    // block 0, P V of block 1.  Block 0's softmax runs under phase 2, block
    // 1's under phase 3; each block's last eight probability pairs spill
    // into the next phase, ahead of the ops that read them.  Scores are read
    // no sooner than eight ops after the op that wrote them.
    float mxq[2] = {-INFINITY, -INFINITY};
    float rsum[2] = {0.f, 0.f};
    bool move[2] = {false, false};
    float alpha[2] = {1.f, 1.f};
    // Keys a query cannot see become -inf: keys at or past t_end, and
    // (causal) keys after the query's global position.  The block's first
    // query sits rel_block(..) - t0 positions past the tile start (clamped
    // to [-kN, kN]), the lane's query lq further.
    auto mask_rows = [&](int qb, int kb, int r0) {
      // Rows r0..r0+3 of key block kb: mask, then fold into the row max.
      const int rel = p.causal ? max(min(rel_block(wave_q0 + 32 * qb) - t0, kN), -kN) : kN;
      const int lim = min(rel + (p.causal ? lq : 0), last) - 4 * hh - 32 * kb;
#pragma unroll
      for (int r = r0; r < r0 + 4; ++r) {
        const int koff = 8 * (r >> 2) + (r & 3);
        s[kb][qb][r] = koff <= lim ? s[kb][qb][r] : -INFINITY;
      }
      mxq[qb] = vmax(vmax(mxq[qb], s[kb][qb][r0]), s[kb][qb][r0 + 1]);
      mxq[qb] = vmax(vmax(mxq[qb], s[kb][qb][r0 + 2]), s[kb][qb][r0 + 3]);
    };
    auto ref_update = [&](int qb) {
      const float m_tile = lane_swap32_max(mxq[qb]) * c;
      // The reference moves under the same rule as in the main walk (a
      // row's first visible keys always move it: -inf + slack = -inf).
      move[qb] = m_tile > m_ref[qb] + kRescaleSlack;
      const float m_new = move[qb] ? m_tile : m_ref[qb];
      alpha[qb] = move[qb] ? exp2_fast(m_ref[qb] - m_new) : 1.f;
      m_ref[qb] = m_new;
      m_use[qb] = m_new == -INFINITY ? 0.f : m_new;
      l_run[qb] *= alpha[qb];
    };
    auto exp_job = [&](int qb, int i) {  // probability pair i (0..15) of block qb
      exp_pair(s[i >> 3][qb], 2 * (i & 7), c, m_use[qb], pb[qb][i >> 2], (2 * i) & 7, rsum[qb]);
    };
    // Softmax slice of block qb under step st of a phase hosting it.
    auto softmax_slice = [&](int qb, int st) {
      if (st < 4) mask_rows(qb, 0, 4 * st);
      else if (st >= 8 && st < 12) mask_rows(qb, 1, 4 * (st - 8));
      if (st == 12) ref_update(qb);
      if (st >= 12) {
        exp_job(qb, 2 * (st - 12));
        exp_job(qb, 2 * (st - 12) + 1);
      }
    };
    // The rest of block qb's pairs (8..15) under steps 0..3 of the next phase.
    auto exp_tail = [&](int qb, int st) {
      if (st < 4) {
        exp_job(qb, 8 + 2 * st);
        exp_job(qb, 9 + 2 * st);
      }
      if (st == 3) l_run[qb] += rsum[qb];
    };
    auto rescale_o = [&](int qb) {
      if (__builtin_amdgcn_ballot_w64(move[qb]) != 0) {
        matrix_settle();
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          __builtin_amdgcn_sched_barrier(0);
          agpr_set(o[qb][db], agpr_get(o[qb][db]) * alpha[qb]);
        }
        scale_lr(lr[qb], alpha[qb]);
      }
    };
    auto qk_phase = [&](int qb, auto&& extra) {
      bf16x8 ka[3];  // K operands two steps ahead
      ka[0] = read_k(ktile, koff, 0, 0);
      ka[1] = read_k(ktile, koff, 0, 1);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        const int kb = t >> 3, kk = t & 7;
        if (t + 2 < 16) ka[(t + 2) % 3] = read_k(ktile, koff, (t + 2) >> 3, (t + 2) & 7);
        if (kk == 0) qk_mfma0(s[kb][qb], ka[t % 3], qv[qb][kk]);
        else qk_mfma(s[kb][qb], ka[t % 3], qv[qb][kk]);
        extra(t);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto pv_phase = [&](int qb, auto&& extra) {
      bf16x8 va[3];  // V operands two steps ahead
      va[0] = read_v(vrel, voff, 0, 0);
      va[1] = read_v(vrel, voff, 0, 1);
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        __builtin_amdgcn_sched_barrier(0);
        if (st + 2 < 16) va[(st + 2) % 3] = read_v(vrel, voff, (st + 2) >> 2, (st + 2) & 3);
        pv_mfma(o[qb][st & 3], va[st % 3], pb[qb][st >> 2]);
        if ((st & 3) == 3) psum_mfma(lr[qb], ones, pb[qb][st >> 2]);
        extra(st);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    qk_phase(0, [&](int) {});
    qk_phase(1, [&](int t) { softmax_slice(0, t); });
    rescale_o(0);
    pv_phase(0, [&](int st) {
      exp_tail(0, st);
      softmax_slice(1, st);
    });
    rescale_o(1);
    pv_phase(1, [&](int st) { exp_tail(1, st); });
    matrix_settle();
  }

  matrix_settle();
  // Finalise: O = acc / (sum of the rounded P it was built from), LSE =
  // (m_ref + log2 l) ln 2 with l the fp32 sum; l == 0 means no visible key
  // (O = 0, LSE = -inf).  NaN in l propagates.
  // bf16 output goes through LDS: each wave stages its 32-row blocks in its
  // own 16 KiB of the K ring (every wave is past its last tile once the
  // barrier below is passed), so that the stores write whole rows, 16 bytes
  // per lane, instead of 8 bytes into each of 32 rows per instruction.
  constexpr bool kStaged = sizeof(TOut) == 2;
  constexpr int kStageRow = 128 * 2 + 16;  // bytes per staged row (head_dim 128, padded: spreads banks)
  char* const stage = (char*)&lds_k[wave][0];
  if (kStaged) tile_barrier();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = lane_swap32_add(l_run[qb]);
    const float l_rnd = lr_total(lr[qb], lq);
    const bool empty = l_tot == 0.f;
    const float inv = empty ? 0.f : 1.f / l_rnd;
    const float lse = empty ? -INFINITY : (m_ref[qb] + __log2f(l_tot)) * 0.69314718055994530942f;
    const int64_t my_q = wave_q0 + 32 * qb + lq;
    if (kStaged) {
      // This lane's values of row lq: columns db*32 + 8*gq + 4*hh .. +3.
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const f32x16 ov = agpr_get(o[qb][db]);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const bf16x4 x = {(__bf16)(ov[4 * gq] * inv), (__bf16)(ov[4 * gq + 1] * inv),
                            (__bf16)(ov[4 * gq + 2] * inv), (__bf16)(ov[4 * gq + 3] * inv)};
          *(bf16x4*)(stage + lq * kStageRow + (db * 32 + 8 * gq + 4 * hh) * 2) = x;
        }
      }
      // Back by rows: row 4*i + lane/16, 16-byte chunk lane%16.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 4 * i + (lane >> 4), chunk = lane & 15;
        const u32x4 d = *(const u32x4*)(stage + row * kStageRow + chunk * 16);
        const int64_t q = wave_q0 + 32 * qb + row;
        if (q < p.seq_q)
          *(u32x4*)((char*)p.o + (b * p.o_sb + h * p.o_sh + q * p.o_ss) * 2 + chunk * 16) = d;
      }
      if (hh == 0 && my_q < p.seq_q) p.lse[((int64_t)b * p.heads_q + h) * p.seq_q + my_q] = lse;
    } else if (my_q < p.seq_q) {
      TOut* orow = (TOut*)p.o + b * p.o_sb + h * p.o_sh + my_q * p.o_ss;
      float* lrow = p.lse + ((int64_t)b * p.heads_q + h) * p.seq_q + my_q;
      // Accumulating (fp32 output only): merge into the running pair.
      const bool acc_mode = sizeof(TOut) == 4 && p.accumulate != 0;
      float wa = 0.f, wb = 1.f, lse_out = lse;
      if (acc_mode) merge_weights(*lrow, lse, wa, wb, lse_out);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const f32x16 ov = agpr_get(o[qb][db]);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4 v = {ov[4 * gq] * inv, ov[4 * gq + 1] * inv, ov[4 * gq + 2] * inv,
                     ov[4 * gq + 3] * inv};
          TOut* dst = orow + db * 32 + 8 * gq + 4 * hh;
          if (acc_mode) {
            const f32x4 old = *(const f32x4*)dst;
            v = old * wa + v * wb;
          }
          store4<TOut>(dst, v);
        }
      }
      if (hh == 0) *lrow = lse_out;
    }
  }
  }  // items
}

// Compute units of the current device (one resident block each).  The
// per-device cache is filled with relaxed atomic stores of the same value, so
// first calls racing from several host threads are well defined.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename TOut>
hipError_t launch_typed(const FwdParams& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.num_q_tiles * p.batch * p.heads_q / (p.quad_heads ? 4 : 1);
  if (items == 0) return hipSuccess;
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int64_t blocks = std::min<int64_t>(items, cus);
  FwdParams arg = p;
  void* args[] = {&arg};
  const void* fn = p.quad_heads ? (const void*)&attn_fwd_bf16_kernel<TOut, true>
                                : (const void*)&attn_fwd_bf16_kernel<TOut, false>;
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdParams& p, DType out, hipStream_t stream) {
  return out == DType::BF16 ? launch_typed<__bf16>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace shattn
