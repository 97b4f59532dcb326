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
//   VALU phase j :  P[j] = softmax(S) ; A stores K[j+1], loads K[j+2];
//                                        B stores V[j+1], loads V[j+2]
//   barrier
// so on every SIMD one wave feeds the matrix core while the other does the
// exponentials.  K and V are double-buffered in LDS; every buffer is written
// only after the phase that last read it has passed a barrier.
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

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kBlockMBf16;  // 256 query rows per workgroup
constexpr int kN = 64;                // keys per tile
constexpr int kKStride = 136;         // K row stride in LDS, elements (272 B)
constexpr int kVStride = 144;         // V row stride in LDS, elements (288 B)
constexpr int kKTile = kN * kKStride;
constexpr int kVTile = kN * kVStride;
constexpr int kChunks = kN * 16 / 256;  // 16-byte pieces per thread of a wave group
constexpr float kRescaleSlack = 8.0f;   // log2 units
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

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A 64-row x 256 B tile of K or V is 1024 sixteen-byte pieces; the 256
// threads of a wave group move kChunks each, piece id = gtid + 256*i (row
// id/16, column piece id%16).  Rows at or past the tile end are read from the
// tile's first row instead (always in bounds) and zeroed when stored, so
// neither loads nor stores branch, and nothing waits for the loads until the
// store two phases later.
struct Stage {
  u32x4 x[kChunks];
  uint32_t ok;  // bit i: piece i lies inside the tile
};

struct TileLoader {
  int64_t off[kChunks];  // element offset of each piece from the tile's first row
  int64_t off0[kChunks]; // the same piece column in the tile's first row
  int row[kChunks];
};

__device__ __forceinline__ void loader_init(TileLoader& ld, int64_t row_stride, int gtid) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int id = gtid + 256 * i;
    ld.row[i] = id >> 4;
    ld.off0[i] = (id & 15) * 8;
    ld.off[i] = (int64_t)ld.row[i] * row_stride + ld.off0[i];
  }
}

__device__ __forceinline__ void gload_tile(const __bf16* tile, int rows, const TileLoader& ld,
                                           Stage& st) {
  uint32_t ok = 0;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const bool in = ld.row[i] < rows;
    ok |= (uint32_t)in << i;
    st.x[i] = *(const u32x4*)(tile + (in ? ld.off[i] : ld.off0[i]));
  }
  st.ok = ok;
}

template <int kStride>
__device__ __forceinline__ void lstore_tile(__bf16* dst, int gtid, const Stage& st) {
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int id = gtid + 256 * i;
    const bool in = (st.ok >> i) & 1u;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = in ? st.x[i][e] : 0u;
    *(u32x4*)(dst + (id >> 4) * kStride + (id & 15) * 8) = v;
  }
}

__device__ __forceinline__ bf16x8 read_k(const __bf16* krow, int t) {
  // Step t of S: key block t/8, d step t%8.
  return *(const bf16x8*)(krow + (t >> 3) * 32 * kKStride + (t & 7) * 16);
}

__device__ __forceinline__ bf16x8 read_v(const __bf16* vs_lane, int t) {
  // Step t of P V: 16-key step t/4, d block t%4 (two transposing reads).
  const __bf16* src = vs_lane + (t >> 2) * 16 * kVStride + (t & 3) * 32;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)src);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + 8 * kVStride));
  bf16x8 a;
  a.lo = __builtin_bit_cast(bf16x4, lo);
  a.hi = __builtin_bit_cast(bf16x4, hi);
  return a;
}

// One MFMA phase: S^T (2 key blocks) of the wave's 32 queries against the K
// tile whose row lq, column 8*hh is krow, and O^T += V^T P^T for the V tile
// (vs_lane: this lane's source address for the transposing read, row
// 4*(lane/32) + (lane/4)%4 of a 16-key step, column 16*((lane/16)%2) +
// 4*(lane%4) of a 32-wide d block).  The 16 S steps and 16 P V steps
// alternate; operand reads run 4 steps ahead.  The order is fixed with
// scheduling barriers so the compiler neither serialises reads and
// matrix-core ops nor hoists every read (which would exhaust registers).
__device__ __forceinline__ void mfma_phase(const __bf16* krow, const __bf16* vs_lane,
                                           const bf16x8 (&qv)[8], const bf16x8 (&pb)[4],
                                           f32x16 (&s)[2], f32x16 (&o)[4]) {
  constexpr int kAhead = 4;
  bf16x8 ka[kAhead], va[kAhead];
#pragma unroll
  for (int t = 0; t < kAhead; ++t) {
    ka[t] = read_k(krow, t);
    va[t] = read_v(vs_lane, t);
  }
  s[0] = (f32x16){};
  s[1] = (f32x16){};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    __builtin_amdgcn_sched_barrier(0);
    s[t >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % kAhead], qv[t & 7], s[t >> 3], 0,
                                                        0, 0);
    o[t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t % kAhead], pb[t >> 2], o[t & 3], 0,
                                                       0, 0);
    if (t + kAhead < 16) {
      ka[t % kAhead] = read_k(krow, t + kAhead);
      va[t % kAhead] = read_v(vs_lane, t + kAhead);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// O^T += V^T P^T alone (the last tile, after the loop).
__device__ __forceinline__ void pv_tile(const __bf16* vs_lane, const bf16x8 (&pb)[4],
                                        f32x16 (&o)[4]) {
#pragma unroll
  for (int t = 0; t < 16; ++t)
    o[t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v(vs_lane, t), pb[t >> 2], o[t & 3], 0,
                                                       0, 0);
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
// and (causal) keys after the query's global position.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], const FwdParams& p, int64_t my_q,
                                          int64_t t0, int64_t t_end, int hh) {
  const int64_t lim64 = min(p.causal ? p.q_pos0 + my_q - t0 : (int64_t)kN, t_end - 1 - t0);
  const int lim = (int)max(min(lim64, (int64_t)kN), (int64_t)-1) - 4 * hh;
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
  __shared__ __attribute__((aligned(16))) __bf16 lds_k[2][kKTile];
  __shared__ __attribute__((aligned(16))) __bf16 lds_v[2][kVTile];
  // All zeros: the V tile P V reads when P is known to be zero (a dead
  // tile), so that non-finite values in a V tile no query of the wave can
  // see never reach it through 0 * NaN.
  __shared__ __attribute__((aligned(16))) __bf16 lds_vzero[kVTile];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in [0, 8)
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const bool group_b = wave >= 4;
  const int gtid = tid & 255;  // thread id within the wave group

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
  const int64_t my_q = wave_q0 + lq;
  const bool row_ok = my_q < p.seq_q;

  const __bf16* qbase = (const __bf16*)p.q + b * p.q_sb + h * p.q_sh;
  const __bf16* kbase = (const __bf16*)p.k + b * p.k_sb + hk * p.k_sh;
  const __bf16* vbase = (const __bf16*)p.v + b * p.v_sb + hk * p.v_sh;
  // Group A streams K tiles, group B streams V tiles.  group_b is derived
  // from the wave index read into a scalar register, so these selects stay
  // scalar.
  const __bf16* my_base_s = group_b ? vbase : kbase;
  const int64_t my_stride_s = group_b ? p.v_ss : p.k_ss;
  TileLoader ld;
  loader_init(ld, my_stride_s, gtid);
  auto tile_ptr = [&](int64_t t0) { return my_base_s + (t0 - p.kv_pos0) * my_stride_s; };

  // Q^T operand, resident for the whole kernel.
  bf16x8 qv[8];
  {
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

  const int v_row = 4 * (lane >> 5) + ((lane >> 2) & 3);
  const int v_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int v_lane_off = v_row * kVStride + v_col;
  const int k_lane_off = lq * kKStride + hh * 8;

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

  // Tiles j (current), j+1, j+2 of the visit order.
  TileWalk t_cur, t_n1, t_n2;
  bool have = walk_from(p, 0, limit, t_cur);
  t_n1 = t_cur;
  bool have1 = have && walk_next(p, limit, t_n1);
  Stage stage;

  // Prologue: K[0] and V[0] into buffer 0, the zero V tile, and tile 1 of
  // this group's stream into registers.
  if (have) {
    gload_tile(tile_ptr(t_cur.t0), (int)(min(t_cur.t0 + kN, t_cur.hi) - t_cur.t0), ld, stage);
    if (group_b)
      lstore_tile<kVStride>(lds_v[0], gtid, stage);
    else
      lstore_tile<kKStride>(lds_k[0], gtid, stage);
    Stage zero;
    zero.ok = 0u;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) zero.x[i] = (u32x4){0u, 0u, 0u, 0u};
    if (!group_b) lstore_tile<kVStride>(lds_vzero, gtid, zero);
    if (have1)
      gload_tile(tile_ptr(t_n1.t0), (int)(min(t_n1.t0 + kN, t_n1.hi) - t_n1.t0), ld, stage);
  }
  __syncthreads();
  if (group_b) __syncthreads();  // group B runs one phase behind group A

  int jb = 0;              // parity of tile j
  bool dead_prev = true;   // P[j-1] is all zeros (no tile before the first)
  while (have) {
    const int64_t t0 = t_cur.t0;
    const int64_t t_end = min(t0 + kN, t_cur.hi);
    t_n2 = t_n1;
    const bool have2 = have1 && walk_next(p, limit, t_n2);
    // A tile is dead for this wave when every key of it lies after every
    // query of the wave (causal) or the wave holds no query rows: its
    // softmax is skipped, P = 0, and its P V reads the zero tile.  (The
    // matrix-core ops still run: a branch around them costs more in register
    // copies than it saves.)
    const bool dead = (p.causal && t0 > wave_qpos_max) || wave_q0 >= p.seq_q;

    // ---- MFMA phase --------------------------------------------------------
    __builtin_amdgcn_s_setprio(1);
    f32x16 s[2];
    const __bf16* krow = lds_k[jb] + k_lane_off;
    const __bf16* vs_lane = (dead_prev ? lds_vzero : lds_v[jb ^ 1]) + v_lane_off;
    mfma_phase(krow, vs_lane, qv, pb, s, o);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();

    // ---- VALU phase --------------------------------------------------------
    if (dead) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int x = 0; x < 8; ++x) pb[ks][x] = (__bf16)0.f;
    } else {
      if ((t_end - t0 < kN) || (p.causal && t_end - 1 > wave_qpos_min))
        mask_tile(s, p, my_q, t0, t_end, hh);
      float mx0 = s[0][0], mx1 = s[1][0];
#pragma unroll
      for (int r = 1; r < 15; r += 2) {
        mx0 = vmax(vmax(mx0, s[0][r]), s[0][r + 1]);
        mx1 = vmax(vmax(mx1, s[1][r]), s[1][r + 1]);
      }
      const float mx = vmax(vmax(mx0, s[0][15]), vmax(mx1, s[1][15]));
      const float m_tile = lane_swap32_max(mx) * c;
      // Wave-uniform decision to move the reference max.
      const bool rescale = __builtin_amdgcn_ballot_w64(m_tile > m_ref + kRescaleSlack) != 0;
      if (rescale) {
        const float m_new = fmaxf(m_ref, m_tile);
        const float alpha = exp2_fast(m_new == m_ref ? 0.f : m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float rs[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: no serial add chain
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2_fast(fmaf(s[kb][r], c, -m_use));
          s[kb][r] = e;
          rs[r & 3] += e;
        }
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int x = 0; x < 8; ++x) pb[ks][x] = (__bf16)s[ks >> 1][(ks & 1) * 8 + x];
    }
    dead_prev = dead;

    // Stream the next tiles: group A stores K[j+1] (read from the next phase
    // on), group B stores V[j+1] (read two phases later); both then fetch
    // tile j+2 of their stream.
    if (have1) {
      if (group_b)
        lstore_tile<kVStride>(lds_v[jb ^ 1], gtid, stage);
      else
        lstore_tile<kKStride>(lds_k[jb ^ 1], gtid, stage);
    }
    if (have2)
      gload_tile(tile_ptr(t_n2.t0), (int)(min(t_n2.t0 + kN, t_n2.hi) - t_n2.t0), ld, stage);
    // Finish the softmax inside this phase: without this the compiler sinks
    // the exponentials past the barrier into the next matrix-core phase.
    asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3]), "v"(l_run) : "memory");
    __syncthreads();

    t_cur = t_n1;
    have = have1;
    t_n1 = t_n2;
    have1 = have2;
    jb ^= 1;
  }
  if (!group_b) __syncthreads();  // match group B's extra barrier

  // The last tile's P V: V[T-1] sits in buffer jb ^ 1.
  pv_tile((dead_prev ? lds_vzero : lds_v[jb ^ 1]) + v_lane_off, pb, o);

  // Finalise: O = acc / l, LSE = (m_ref + log2 l) ln 2; l == 0 means no
  // visible key (O = 0, LSE = -inf).  NaN in l propagates.
  const float l_tot = lane_swap32_add(l_run);
  const bool empty = l_tot == 0.f;
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float lse = empty ? -INFINITY : (m_ref + __log2f(l_tot)) * 0.69314718055994530942f;
  if (row_ok) {
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
