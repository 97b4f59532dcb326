// Fused shifted-chunk attention forward, bf16 inputs, for gfx950 (CDNA4).
//
// A workgroup owns 256 query rows of one (batch, query head): eight waves of
// 32 rows, two per SIMD.  It walks the KV chunks in the rank-shifted order
// c_j = (j + rank) % J (the `shift` primitive of CommIR, papers.lqhl.me
// summary "Mercury (SOSP 2025)", section 核心方法), 64 keys per tile, and
// carries the online-softmax state in registers across chunk boundaries.
// Rescaling that state when a chunk starts is exactly the log-sum-exp merge
// of the chunk's partial result, so one launch computes what attn_chunk_fwd
// followed by lse_merge computes chunk by chunk.  Chunk ranges that no query
// of the workgroup can see (causal) are skipped without touching memory.
//
// Matrix cores (v_mfma_f32_32x32x16_bf16), per wave and 64-key tile:
//   S^T[key][q] = sum_d K[key][d] Q[q][d]          2 key blocks x 8 steps
//     A = K rows from LDS (ds_read_b128), B = Q^T resident in VGPRs.
//   O^T[d][q] += sum_key V^T[d][key] P^T[key][q]   4 d blocks x 4 steps
//     A = V^T, read from row-major V in LDS with the transposing
//         ds_read_b64_tr_b16, B = P^T taken straight from the S^T accumulator.
// Each lane owns one query column of S^T, so the softmax row max/sum are
// in-lane reductions plus one v_permlane32_swap with the lane holding the
// other half of the keys.  Accumulator layout (lane l, register r):
//   column = l % 32, row = 8*(r/4) + 4*(l/32) + (r%4).
//
// Ping-pong: waves 0-3 (group A) and 4-7 (group B) share the SIMDs pairwise
// and run the same loop one phase apart (group B starts one barrier late):
//   MFMA phase j :  S = Q K[j]^T ;  O += P[j-1] V[j-1]
//   barrier
//   VALU phase j :  P[j] = softmax(S) ; A starts K[j+3], B starts V[j+3]
//   barrier
// so on every SIMD one wave feeds the matrix core while the other does the
// exponentials.  K and V tiles stream straight from global memory into a
// 4-deep LDS ring (global_load_lds_dwordx4, no registers involved), three
// tiles ahead; each wave waits only for its own copies of the tile the next
// barrier publishes.  A ring slot is refilled only after the phase that last
// read it has passed a barrier.  Tiles sit in LDS unpadded with XOR-swizzled
// 16-byte chunks (K: chunk ^ (row & 15); V: chunk ^ 4*(row & 3)) so that the
// K reads and the transposing V reads are free of bank conflicts.
//
// Lazy rescaling: exponentials use a reference max m_ref that only moves
// when a row's running max exceeds it by more than 8 (log2 units), so the
// output accumulator is rescaled only on those rare tiles.  O and l share
// the reference, so the result is unchanged; p <= 2^8 loses no relative
// precision in fp32 or bf16.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace shattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kBlockMBf16;  // 256 query rows per workgroup
constexpr int kN = 64;                // keys per tile
constexpr int kTile = kN * 128;       // elements of one K or V tile (16 KB, unpadded)
constexpr int kRing = 4;              // LDS ring depth per stream
constexpr float kRescaleSlack = 8.0f;  // log2 units
static_assert(kBlockM == kWaves * 32, "32 query rows per wave");

struct TileWalk {
  int j;       // step in visit order
  int64_t hi;  // end of the current chunk segment (global position)
  int64_t t0;  // tile start (global position)
};

__device__ __forceinline__ bool segment(const FwdParams& p, int j, int64_t limit, int64_t& lo,
                                        int64_t& hi) {
  int c = (j + p.rank) % p.num_chunks;
  lo = p.kv_pos0 + (int64_t)c * p.chunk_len;
  hi = lo + p.chunk_len;
  if (hi > limit) hi = limit;
  return hi > lo;
}

__device__ __forceinline__ bool walk_from(const FwdParams& p, int j0, int64_t limit, TileWalk& w) {
  for (int j = j0; j < p.num_chunks; ++j) {
    int64_t lo, hi;
    if (segment(p, j, limit, lo, hi)) {
      w.j = j;
      w.hi = hi;
      w.t0 = lo;
      return true;
    }
  }
  return false;
}

__device__ __forceinline__ bool walk_next(const FwdParams& p, int64_t limit, TileWalk& w) {
  if (w.t0 + kN < w.hi) {
    w.t0 += kN;
    return true;
  }
  return walk_from(p, w.j + 1, limit, w);
}

__device__ __forceinline__ int tile_rows(const TileWalk& w) { return (int)min((int64_t)kN, w.hi - w.t0); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Waits until at most n (0, 4 or 8) of this wave's global->LDS copies are
// still in flight.
__device__ __forceinline__ void wait_copies(int n) {
  if (n == 0)
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  else if (n == 4)
    __builtin_amdgcn_s_waitcnt(0xF74);  // vmcnt(4)
  else
    __builtin_amdgcn_s_waitcnt(0xF78);  // vmcnt(8)
}

// Workgroup barrier without the release fence __syncthreads() adds: that
// fence would wait for every global->LDS copy in flight, including the
// prefetches of later tiles.  Copies a barrier must publish are waited for
// explicitly with wait_copies(); LDS reads before a barrier have all returned
// (their data fed matrix-core ops of the phase).
__device__ __forceinline__ void phase_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Global -> LDS copy of one 64-row tile of K or V by the four waves of a wave
// group.  Wave wg copies rows 16*wg .. 16*wg+15 with four 1 KB instructions;
// lane i of instruction n writes LDS chunk i of rows 16*wg + 4*n + i/16,
// i.e. physical 16-byte chunk i%16 of that row, which holds logical chunk
// (i%16) ^ swz(row).  Rows past the tile end copy its last row instead (in
// bounds; their keys are masked and their P is 0).
struct CopyLane {
  int row[4];  // tile row of instruction n
  int col[4];  // element offset of the logical chunk within the row
};

__device__ __forceinline__ void copy_lane_init(CopyLane& cl, bool v_layout, int wg, int lane) {
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 16 * wg + 4 * n + (lane >> 4);
    const int pc = lane & 15;
    const int lc = v_layout ? (pc ^ (4 * (row & 3))) : (pc ^ (row & 15));
    cl.row[n] = row;
    cl.col[n] = lc * 8;
  }
}

// The copy is written as inline assembly on purpose: through the builtin,
// the compiler cannot tell which LDS bytes a copy writes and makes every
// later LDS read wait for all copies in flight, prefetches included.  Here
// every wait is explicit (wait_copies before the barrier that publishes a
// tile).  M0 holds the LDS destination; one wait state must separate its
// scalar write from the copy that reads it.
__device__ __forceinline__ void copy_tile(__bf16* lds_tile, const __bf16* gtile, int rows,
                                          int stride, const CopyLane& cl, int wg) {
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = min(cl.row[n], rows - 1);
    const __bf16* src = gtile + (r * stride + cl.col[n]);
    const uint32_t lds_addr =
        (uint32_t)(uintptr_t)(lds_void*)(lds_tile + (16 * wg + 4 * n) * 128);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds_addr), "v"(src)
        : "memory", "m0");
  }
}

// Step t of S (key block t/8, d step t%8): this lane's row is kb*32 + lq, its
// logical chunk 2*(t%8) + hh, physical chunk logical ^ (lq & 15).  koff[kk]
// is the byte offset for key block 0; key block 1 is 32 rows (8 KB) further.
__device__ __forceinline__ bf16x8 read_k(const __bf16* ktile, const int (&koff)[8], int t) {
  return *(const bf16x8*)((const char*)ktile + koff[t & 7] + (t >> 3) * 8192);
}

// Step t of P V (16-key step t/4, d block t%4): two transposing reads 8 rows
// apart.  voff[db] is this lane's byte address for 16-key step 0; step ks is
// 16 rows (4 KB) further.
__device__ __forceinline__ bf16x8 read_v(const __bf16* vtile, const int (&voff)[4], int t) {
  const char* src = (const char*)vtile + voff[t & 3] + (t >> 2) * 4096;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)src);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + 2048));
  bf16x8 a;
  a.lo = __builtin_bit_cast(bf16x4, lo);
  a.hi = __builtin_bit_cast(bf16x4, hi);
  return a;
}

// One MFMA phase of the wave:
//  * S^T (2 key blocks) of its 32 queries against K tile `ktile`;
//  * the second half of the previous tile's softmax: s_hi holds that tile's
//    scores for key block 1; p = exp2(s*c - m_use) goes to pb[2], pb[3] and
//    its sum is returned;
//  * O^T += V^T P^T for the previous tile (V tile `vtile`).
// The first 8 S steps are each paired with one P V step of key block 0 (its
// P is ready) and two exponentials; the P V steps of key block 1 follow the
// last 8 S steps.  Operand reads run 4 steps ahead.  The order is fixed with
// scheduling barriers so the compiler neither serialises reads and
// matrix-core ops nor hoists every read.
__device__ __forceinline__ float mfma_phase(const __bf16* ktile, const __bf16* vtile,
                                            const int (&koff)[8], const int (&voff)[4],
                                            const bf16x8 (&qv)[8], bf16x8 (&pb)[4],
                                            const f32x16& s_hi, float c, float m_use,
                                            f32x16 (&s)[2], f32x16 (&o)[4]) {
  constexpr int kAhead = 4;
  bf16x8 ka[kAhead], va[kAhead];
#pragma unroll
  for (int t = 0; t < kAhead; ++t) {
    ka[t] = read_k(ktile, koff, t);
    va[t] = read_v(vtile, voff, t);
  }
  s[0] = (f32x16){};
  s[1] = (f32x16){};
  float rs[2] = {0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    __builtin_amdgcn_sched_barrier(0);
    s[t >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % kAhead], qv[t & 7], s[t >> 3], 0,
                                                        0, 0);
    if (t < 8) {
      o[t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t % kAhead], pb[t >> 2], o[t & 3], 0,
                                                         0, 0);
      // Two exponentials of the previous tile's key block 1 per step, all
      // done before the new key block 1 (step 8 on) reuses those registers.
      const float e0 = exp2_fast(fmaf(s_hi[2 * t], c, -m_use));
      const float e1 = exp2_fast(fmaf(s_hi[2 * t + 1], c, -m_use));
      rs[0] += e0;
      rs[1] += e1;
      pb[2 + (t >> 2)][(2 * t) & 7] = (__bf16)e0;
      pb[2 + (t >> 2)][(2 * t + 1) & 7] = (__bf16)e1;
    }
    if (t + kAhead < 16) ka[t % kAhead] = read_k(ktile, koff, t + kAhead);
    if (t < 8 && t + kAhead < 16) va[t % kAhead] = read_v(vtile, voff, t + kAhead);
  }
#pragma unroll
  for (int u = 8; u < 16; ++u) {
    __builtin_amdgcn_sched_barrier(0);
    o[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[u % kAhead], pb[u >> 2], o[u & 3], 0, 0,
                                                       0);
    if (u + kAhead < 16) va[u % kAhead] = read_v(vtile, voff, u + kAhead);
  }
  __builtin_amdgcn_sched_barrier(0);
  return rs[0] + rs[1];
}

// The second half of a tile's softmax alone (after the loop).
__device__ __forceinline__ float softmax_hi(bf16x8 (&pb)[4], const f32x16& s_hi, float c,
                                            float m_use) {
  float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const float e = exp2_fast(fmaf(s_hi[t], c, -m_use));
    rs[t & 3] += e;
    pb[2 + (t >> 3)][t & 7] = (__bf16)e;
  }
  return (rs[0] + rs[1]) + (rs[2] + rs[3]);
}

// O^T += V^T P^T alone (the last tile, after the loop).
__device__ __forceinline__ void pv_tile(const __bf16* vtile, const int (&voff)[4],
                                        const bf16x8 (&pb)[4], f32x16 (&o)[4]) {
#pragma unroll
  for (int t = 0; t < 16; ++t)
    o[t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v(vtile, voff, t), pb[t >> 2], o[t & 3],
                                                       0, 0, 0);
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

// Keys of a tile that a query cannot see become -inf: keys at or past t_end,
// and (causal) keys after the query's global position.  rel0 = (global
// position of the wave's first query) - t0, a wave-uniform value; the lane's
// query is rel0 + lq positions past the tile start.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], bool causal, int64_t rel0, int64_t t0,
                                          int64_t t_end, int lq, int hh) {
  // Clamp the wave-uniform parts to small ints before adding the lane part.
  const int last = (int)(t_end - 1 - t0);  // in [0, kN)
  const int rel = causal ? (int)max(min(rel0, (int64_t)kN), (int64_t)-64) : kN;
  const int lim = min(rel + (causal ? lq : 0), last) - 4 * hh;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int koff = kb * 32 + 8 * (r >> 2) + (r & 3);
      s[kb][r] = koff <= lim ? s[kb][r] : -INFINITY;
    }
}

// Makes the compiler wait for outstanding loads into v before going on.
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

template <typename TOut>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) __bf16 lds_k[kRing][kTile];
  __shared__ __attribute__((aligned(16))) __bf16 lds_v[kRing][kTile];
  // All zeros: the V tile P V reads when P is known to be zero (a dead
  // tile), so that non-finite values in a V tile no query of the wave can
  // see never reach it through 0 * NaN.
  __shared__ __attribute__((aligned(16))) __bf16 lds_vzero[kTile];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in [0, 8)
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const bool group_b = wave >= 4;
  const int wg = wave & 3;  // wave index within its group

  // Block -> work item.  The hardware deals consecutive blocks round-robin to
  // the 8 XCDs; remap so that the work items sharing one KV head land on one
  // XCD (its L2 then serves their common K/V tiles), and within a head give
  // the heaviest (latest, for causal) query tiles out first.
  const int total = (int)gridDim.x;
  const int full = total - (total & 7);
  const int bid = (int)blockIdx.x;
  const int w = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
  const int qt = p.num_q_tiles - 1 - (w % p.num_q_tiles);
  int rest = w / p.num_q_tiles;
  const int g = rest % p.group;
  rest /= p.group;
  const int hk = rest % p.heads_kv;
  const int b = rest / p.heads_kv;
  const int h = hk * p.group + g;

  const int64_t q_start = (int64_t)qt * kBlockM;
  const int64_t q_rows_wg = min((int64_t)kBlockM, p.seq_q - q_start);
  const int64_t wave_q0 = q_start + wave * 32;
  const int64_t limit = p.causal ? p.q_pos0 + q_start + q_rows_wg : INT64_MAX;
  const int64_t wave_qpos_min = p.q_pos0 + wave_q0;
  // Last query position of the wave (below wave_qpos_min if it has no rows).
  const int64_t wave_qpos_max = p.q_pos0 + min(wave_q0 + 31, p.seq_q - 1);

  const __bf16* qbase = (const __bf16*)p.q + b * p.q_sb + h * p.q_sh;
  const __bf16* kbase = (const __bf16*)p.k + b * p.k_sb + hk * p.k_sh;
  const __bf16* vbase = (const __bf16*)p.v + b * p.v_sb + hk * p.v_sh;
  // Group A streams K tiles, group B streams V tiles.
  const __bf16* my_base = group_b ? vbase : kbase;
  const int my_stride = (int)(group_b ? p.v_ss : p.k_ss);
  __bf16* const my_ring = group_b ? &lds_v[0][0] : &lds_k[0][0];
  auto tile_ptr = [&](int64_t t0) { return my_base + (t0 - p.kv_pos0) * my_stride; };
  CopyLane cl;
  copy_lane_init(cl, group_b, wg, lane);

  // Q^T operand, resident for the whole kernel.
  bf16x8 qv[8];
  {
    const int64_t my_q = wave_q0 + lq;
    const bool row_ok = my_q < p.seq_q;
    const int64_t row = row_ok ? my_q : 0;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 x = *(const u32x4*)(qbase + row * p.q_ss + kk * 16 + hh * 8);
      u32x4 y;
      y[0] = row_ok ? x[0] : 0u;
      y[1] = row_ok ? x[1] : 0u;
      y[2] = row_ok ? x[2] : 0u;
      y[3] = row_ok ? x[3] : 0u;
      qv[kk] = __builtin_bit_cast(bf16x8, y);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) settle(qv[kk]);
  }

  // Per-lane LDS byte offsets of the matrix-core operands (see read_k, read_v).
  int koff[8], voff[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) koff[kk] = lq * 256 + (((2 * kk + hh) ^ (lq & 15)) * 16);
  {
    const int t = (lane >> 2) & 3, gq = (lane >> 4) & 1, u = lane & 3;
    const int row = 4 * hh + t;  // row & 3 == t
#pragma unroll
    for (int db = 0; db < 4; ++db)
      voff[db] = row * 256 + (((db * 4 + 2 * gq + (u >> 1)) ^ (4 * t)) * 16) + (u & 1) * 8;
  }

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
  float m_ref = -INFINITY;
  float l_run = 0.f;
  const float c = p.scale_log2;
  bf16x8 pb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int x = 0; x < 8; ++x) pb[ks][x] = (__bf16)0.f;

  // Tiles j (current) .. j+3 of the visit order.
  TileWalk t_cur, t_n1, t_n2, t_n3;
  bool have = walk_from(p, 0, limit, t_cur);
  t_n1 = t_cur;
  bool have1 = have && walk_next(p, limit, t_n1);
  t_n2 = t_n1;
  bool have2 = have1 && walk_next(p, limit, t_n2);

  // Prologue: the zero V tile, and tiles 0..2 of each group's stream.
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < kTile / 8; i += kThreads) *(u32x4*)(lds_vzero + 8 * i) = zero;
  }
  if (have) copy_tile(my_ring, tile_ptr(t_cur.t0), tile_rows(t_cur), my_stride, cl, wg);
  if (have1) copy_tile(my_ring + kTile, tile_ptr(t_n1.t0), tile_rows(t_n1), my_stride, cl, wg);
  if (have2) copy_tile(my_ring + 2 * kTile, tile_ptr(t_n2.t0), tile_rows(t_n2), my_stride, cl, wg);
  wait_copies(0);
  __syncthreads();
  if (group_b) phase_barrier();  // group B runs one phase behind group A

  int slot = 0;            // ring slot of tile j
  bool dead_prev = true;   // P[j-1] is all zeros (no tile before the first)
  // Second half of the previous tile's softmax, finished in the next MFMA
  // phase: its key-block-1 scores and the reference they are taken against.
  f32x16 s_hi;
#pragma unroll
  for (int r = 0; r < 16; ++r) s_hi[r] = -INFINITY;
  float m_use = 0.f;
  // The hot loop below modifies O only through the matrix-core ops: a tile
  // whose scores would move the reference max leaves it, and the outer loop
  // rescales O and finishes that tile.  (Rescaling inside the loop makes the
  // compiler keep two register copies of O and move all 64 values between
  // them twice per tile.)
  f32x16 s[2];
  int64_t t0 = 0, t_end = 0;
  bool dead = true, have3 = false;
  float m_tile = -INFINITY;

  // Second part of the VALU phase: exponentials of key block 0 (or P = 0
  // for a dead tile), the copy of tile j+3, the wait for tile j+1, the
  // barrier, and the rotation of the tile window.
  auto valu_rest = [&]() __attribute__((always_inline)) {
    if (dead) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int x = 0; x < 8; ++x) pb[ks][x] = (__bf16)0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) s_hi[r] = -INFINITY;
      m_use = 0.f;
    } else {
      m_use = m_ref == -INFINITY ? 0.f : m_ref;
      // First half (key block 0) now; key block 1 in the next MFMA phase.
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2_fast(fmaf(s[0][r], c, -m_use));
        rs[r & 3] += e;
        pb[r >> 3][r & 7] = (__bf16)e;
      }
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      s_hi = s[1];
    }
    dead_prev = dead;

    // Stream: start tile j+3 of this group's stream into the slot that held
    // tile j-1 (last read before the previous barrier), then wait until tile
    // j+1 of the stream has fully landed: only copies of tiles j+2 and j+3
    // (issued after it) may still be in flight.
    if (have3)
      copy_tile(my_ring + ((slot + 3) & (kRing - 1)) * kTile, tile_ptr(t_n3.t0), tile_rows(t_n3),
                my_stride, cl, wg);
    wait_copies(4 * ((int)have2 + (int)have3));
    // Finish this phase's softmax work before the barrier: without this the
    // compiler sinks the exponentials into the next matrix-core phase.
    asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(s_hi), "v"(l_run) : "memory");
    phase_barrier();

    t_cur = t_n1;
    have = have1;
    t_n1 = t_n2;
    have1 = have2;
    t_n2 = t_n3;
    have2 = have3;
    slot = (slot + 1) & (kRing - 1);
  };

  while (have) {
    bool move_ref = false;
    do {
      t0 = t_cur.t0;
      t_end = min(t0 + kN, t_cur.hi);
      t_n3 = t_n2;
      have3 = have2 && walk_next(p, limit, t_n3);
      // A tile is dead for this wave when every key of it lies after every
      // query of the wave (causal) or the wave holds no query rows: its
      // softmax is skipped, P = 0, and its P V reads the zero tile.  (The
      // matrix-core ops still run: a branch around them costs more in
      // register copies than it saves.)
      dead = (p.causal && t0 > wave_qpos_max) || wave_q0 >= p.seq_q;

      // ---- MFMA phase ------------------------------------------------------
      __builtin_amdgcn_s_setprio(1);
      const __bf16* ktile = &lds_k[slot][0];
      const __bf16* vtile = dead_prev ? lds_vzero : &lds_v[(slot + kRing - 1) & (kRing - 1)][0];
      l_run += mfma_phase(ktile, vtile, koff, voff, qv, pb, s_hi, c, m_use, s, o);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();

      // ---- VALU phase ------------------------------------------------------
      if (!dead) {
        if ((t_end - t0 < kN) || (p.causal && t_end - 1 > wave_qpos_min))
          mask_tile(s, p.causal != 0, wave_qpos_min - t0, t0, t_end, lq, hh);
        float mx0 = s[0][0], mx1 = s[1][0];
#pragma unroll
        for (int r = 1; r < 15; r += 2) {
          mx0 = vmax(vmax(mx0, s[0][r]), s[0][r + 1]);
          mx1 = vmax(vmax(mx1, s[1][r]), s[1][r + 1]);
        }
        const float mx = vmax(vmax(mx0, s[0][15]), vmax(mx1, s[1][15]));
        m_tile = lane_swap32_max(mx) * c;
        // Wave-uniform decision to move the reference max.
        move_ref = __builtin_amdgcn_ballot_w64(m_tile > m_ref + kRescaleSlack) != 0;
        if (move_ref) break;
      }
      valu_rest();
    } while (have);
    if (!move_ref) break;
    // Rare: move the reference max of this tile's rows and rescale O and l.
    {
      const float m_new = fmaxf(m_ref, m_tile);
      const float alpha = exp2_fast(m_new == m_ref ? 0.f : m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
    }
    valu_rest();
  }
  if (!group_b) phase_barrier();  // match group B's extra barrier

  // The last tile: second half of its softmax, then its P V (V[T-1] sits in
  // the slot before `slot`).
  l_run += softmax_hi(pb, s_hi, c, m_use);
  pv_tile(dead_prev ? lds_vzero : &lds_v[(slot + kRing - 1) & (kRing - 1)][0], voff, pb, o);

  // Finalise: O = acc / l, LSE = (m_ref + log2 l) ln 2; l == 0 means no
  // visible key (O = 0, LSE = -inf).  NaN in l propagates.
  const float l_tot = lane_swap32_add(l_run);
  const bool empty = l_tot == 0.f;
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float lse = empty ? -INFINITY : (m_ref + __log2f(l_tot)) * 0.69314718055994530942f;
  const int64_t my_q = wave_q0 + lq;
  if (my_q < p.seq_q) {
    TOut* orow = (TOut*)p.o + b * p.o_sb + h * p.o_sh + my_q * p.o_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 v = {o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv, o[db][4 * gq + 2] * inv,
                   o[db][4 * gq + 3] * inv};
        store4<TOut>(orow + db * 32 + 8 * gq + 4 * hh, v);
      }
    if (hh == 0) p.lse[((int64_t)b * p.heads_q + h) * p.seq_q + my_q] = lse;
  }
}

template <typename TOut>
hipError_t launch_typed(const FwdParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.num_q_tiles * p.batch * p.heads_q;
  if (blocks == 0) return hipSuccess;
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)&attn_fwd_bf16_kernel<TOut>, dim3((unsigned)blocks),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdParams& p, DType out, hipStream_t stream) {
  return out == DType::BF16 ? launch_typed<__bf16>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace shattn
