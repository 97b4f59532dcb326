// Fused shifted-chunk attention forward for gfx950 (CDNA4), fp32 inputs.
//
// One workgroup owns kBlockM = 128 query rows of one (batch, query head):
// four waves of 32 rows each.  It walks the KV chunks in the rank-shifted
// order c_j = (j + rank) % J (the `shift` primitive of CommIR, papers.lqhl.me
// summary "Mercury (SOSP 2025)", section 核心方法), streaming each chunk's
// key/value tiles (32 keys) through a double-buffered LDS stage, and carries
// the online-softmax state (running max m, running sum l, unnormalised
// output) in registers across chunk boundaries.  Rescaling the state at a
// chunk boundary is exactly the log-sum-exp merge of that chunk's partial
// result, so the fused loop computes what attn_chunk_fwd + lse_merge compute,
// in one launch.  Chunk ranges that are causally invisible to the whole
// workgroup are skipped without touching memory.
//
// Every product and sum stays in fp32 (v_mfma_f32_32x32x2_f32); this path
// exists for fp32 callers and small problems, not for throughput.
//
// Matrix-core mapping (per wave, 32 queries):
//   S^T[key][q] = sum_d K[key][d] Q[q][d]
//     A = K tile rows from LDS, B = Q^T held in VGPRs for the whole kernel.
//   O^T[d][q]  += sum_key V^T[d][key] P^T[key][q]
//     A = V from LDS (row-major, read per key), B = P^T straight from the S^T
//     accumulator registers (no cross-lane traffic).
// With S^T in the accumulator each lane owns one query column, so the row
// max / row sum are in-lane reductions plus one exchange with the partner
// lane (lane ^ 32) that holds the other half of the keys.
//
// Accumulator layout of a 32x32 MFMA (lane l, register r):
//   column = l % 32, row = 8*(r/4) + 4*(l/32) + (r%4).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace shattn {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kBlockMF32;
static_assert(kBlockM == kWaves * 32, "one wave per 32 query rows");

// Tile geometry: 32 keys per tile; K and V row-major in LDS.
constexpr int kN = 32;
constexpr int kKStride = 130;  // 2 floats pad: lanes (row, d parity) hit distinct banks
constexpr int kVStride = 136;
constexpr int kKElems = kN * kKStride;
constexpr int kVElems = kN * kVStride;

// Visit-order walker over KV tiles: chunk c_j = (j + rank) % J, clipped to the
// keys the workgroup can see (limit = one past its largest query position
// when causal).
struct TileWalk {
  int j;
  int64_t hi;  // end of the current chunk segment
  int64_t t0;  // start of the current tile
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

template <int N>
__device__ __forceinline__ bool walk_next(const FwdParams& p, int64_t limit, TileWalk& w) {
  if (w.t0 + N < w.hi) {
    w.t0 += N;
    return true;
  }
  return walk_from(p, w.j + 1, limit, w);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------------------------
// Global -> register staging and register -> LDS stores.
// ----------------------------------------------------------------------------

// fp32: K and V tiles are 32 rows x 512 B = 1024 16-byte pieces each, 4 per
// thread; both stay row-major in LDS.
struct StageF32 {
  f32x4 k[4];
  f32x4 v[4];
};

__device__ __forceinline__ void gload_f32(const FwdParams& p, const float* kb, const float* vb,
                                          int64_t t0, int64_t t_end, int tid, StageF32& s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int id = tid + kThreads * i;
    int row = id >> 5, ch = id & 31;
    int64_t key = t0 + row;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (key < t_end) {
      x = *(const f32x4*)(kb + (key - p.kv_pos0) * p.k_ss + ch * 4);
      y = *(const f32x4*)(vb + (key - p.kv_pos0) * p.v_ss + ch * 4);
    }
    s.k[i] = x;
    s.v[i] = y;
  }
}

__device__ __forceinline__ void lstore_f32(float* ks, float* vs, int tid, const StageF32& s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int id = tid + kThreads * i;
    int row = id >> 5, ch = id & 31;
    f32x2 lo = {s.k[i][0], s.k[i][1]};
    f32x2 hi = {s.k[i][2], s.k[i][3]};
    *(f32x2*)(ks + row * kKStride + ch * 4) = lo;
    *(f32x2*)(ks + row * kKStride + ch * 4 + 2) = hi;
    *(f32x4*)(vs + row * kVStride + ch * 4) = s.v[i];
  }
}

template <typename TOut>
__device__ __forceinline__ void store_row4(TOut* dst, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store_row4<float>(float* dst, float a, float b, float c, float d) {
  f32x4 x = {a, b, c, d};
  *(f32x4*)dst = x;
}

template <>
__device__ __forceinline__ void store_row4<__bf16>(__bf16* dst, float a, float b, float c,
                                                   float d) {
  bf16x4 x = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  *(bf16x4*)dst = x;
}

// ----------------------------------------------------------------------------
// The kernel.
// ----------------------------------------------------------------------------
template <typename TOut>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(FwdParams p) {

  __shared__ __attribute__((aligned(16))) float lds_k[2][kKElems];
  __shared__ __attribute__((aligned(16))) float lds_v[2][kVElems];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;  // query column owned by this lane
  const int hh = lane >> 5;  // which half of the keys / contraction slots

  // Workgroup -> (batch, head, query tile).
  const int bid = blockIdx.x;
  const int qt = bid % p.num_q_tiles;
  const int bh = bid / p.num_q_tiles;
  const int h = bh % p.heads_q;
  const int b = bh / p.heads_q;
  const int hk = h / p.group;

  const int64_t q_start = (int64_t)qt * kBlockM;
  const int64_t q_rows_wg = min((int64_t)kBlockM, p.seq_q - q_start);
  const int64_t wave_q0 = q_start + wave * 32;
  const int64_t my_q = wave_q0 + lq;
  const bool row_ok = my_q < p.seq_q;
  const int64_t qpos = p.q_pos0 + my_q;
  const int64_t wave_last_q = min(wave_q0 + 31, p.seq_q - 1);
  const bool wave_live = wave_q0 < p.seq_q;
  const int64_t wave_qpos_min = p.q_pos0 + wave_q0;
  const int64_t wave_qpos_max = p.q_pos0 + wave_last_q;
  const int64_t limit = p.causal ? p.q_pos0 + q_start + q_rows_wg : INT64_MAX;

  const float* qb = (const float*)p.q + b * p.q_sb + h * p.q_sh;
  const float* kbase = (const float*)p.k + b * p.k_sb + hk * p.k_sh;
  const float* vbase = (const float*)p.v + b * p.v_sb + hk * p.v_sh;

  // Q^T B-operands, resident for the whole kernel.
  // Lane half hh holds the odd (hh = 1) or even d of each pair of the
  // 2-deep fp32 contraction.
  float qv[64];
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (row_ok) x = *(const f32x4*)(qb + my_q * p.q_ss + c * 4);
    qv[2 * c] = hh ? x[1] : x[0];
    qv[2 * c + 1] = hh ? x[3] : x[2];
  }

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (f32x16){};
  float m_run = -INFINITY;  // running max in log2 units (score * scale * log2 e)
  float l_run = 0.f;        // this lane's half of the running sum
  const float sl2 = p.scale_log2;

  StageF32 st;

  TileWalk cur;
  bool have = walk_from(p, 0, limit, cur);
  if (have) {
    int64_t t_end = min(cur.t0 + kN, cur.hi);
    gload_f32(p, kbase, vbase, cur.t0, t_end, tid, st);
    lstore_f32(lds_k[0], lds_v[0], tid, st);
  }
  __syncthreads();

  int buf = 0;
  while (have) {
    const int64_t t0 = cur.t0;
    const int64_t t_end = min(t0 + kN, cur.hi);
    TileWalk nxt = cur;
    const bool have_next = walk_next<kN>(p, limit, nxt);
    if (have_next) {
      int64_t n_end = min(nxt.t0 + kN, nxt.hi);
      gload_f32(p, kbase, vbase, nxt.t0, n_end, tid, st);
    }

    // Skip waves whose every query precedes the whole tile (causal) or that
    // hold no query rows at all.
    const bool wave_work = wave_live && (!p.causal || t0 <= wave_qpos_max);
    if (wave_work) {
      const float* ks = lds_k[buf];
      const float* vs = lds_v[buf];
      f32x16 s = {};
#pragma unroll
      for (int kk = 0; kk < 64; ++kk) {
        float a = ks[lq * kKStride + 2 * kk + hh];
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qv[kk], s, 0, 0, 0);
      }

      // Mask: keys past the tile end, and (causal) keys after the query.
      const bool need_mask = (t_end - t0 < kN) || (p.causal && t_end - 1 > wave_qpos_min);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int64_t key = t0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool ok = key < t_end && (!p.causal || key <= qpos);
          s[r] = ok ? s[r] : -INFINITY;
        }
      }

      // Online softmax in log2 units.
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = fast_exp2(fmaf(s[r], sl2, -m_use));
        s[r] = e;
        rs += e;
      }
      l_run = fmaf(l_run, alpha, rs);
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= alpha;

      // O^T += V^T P^T.
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int key = 8 * (r >> 2) + 4 * hh + (r & 3);
          float a = vs[key * kVStride + db * 32 + lq];
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[r], acc[db], 0, 0, 0);
        }
    }

    if (have_next) lstore_f32(lds_k[buf ^ 1], lds_v[buf ^ 1], tid, st);
    __syncthreads();
    buf ^= 1;
    cur = nxt;
    have = have_next;
  }

  // Finalise: O = acc / l, LSE = (m + log2 l) * ln 2.  l == 0 means no key was
  // visible: O = 0, LSE = -inf.  NaN in l propagates to both.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool empty = (l_tot == 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float lse = empty ? -INFINITY : (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  if (row_ok) {
    TOut* orow = (TOut*)p.o + b * p.o_sb + h * p.o_sh + my_q * p.o_ss;
    float* lrow = p.lse + ((int64_t)b * p.heads_q + h) * p.seq_q + my_q;
    // Accumulating (fp32 output only): merge into the running pair.
    const bool acc_mode = sizeof(TOut) == 4 && p.accumulate != 0;
    float wa = 0.f, wb = 1.f, lse_out = lse;
    if (acc_mode) merge_weights(*lrow, lse, wa, wb, lse_out);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int d0 = db * 32 + 8 * g + 4 * hh;
        float x0 = acc[db][4 * g] * inv, x1 = acc[db][4 * g + 1] * inv;
        float x2 = acc[db][4 * g + 2] * inv, x3 = acc[db][4 * g + 3] * inv;
        if (acc_mode) {
          const float* old = (const float*)(orow + d0);
          x0 = old[0] * wa + x0 * wb;
          x1 = old[1] * wa + x1 * wb;
          x2 = old[2] * wa + x2 * wb;
          x3 = old[3] * wa + x3 * wb;
        }
        store_row4<TOut>(orow + d0, x0, x1, x2, x3);
      }
    if (hh == 0) *lrow = lse_out;
  }
}

template <typename TOut>
hipError_t launch_typed(const FwdParams& p, hipStream_t stream) {
  int64_t blocks = (int64_t)p.num_q_tiles * p.batch * p.heads_q;
  if (blocks == 0) return hipSuccess;
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)&attn_fwd_f32_kernel<TOut>, dim3((unsigned)blocks),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_attn_fwd_f32(const FwdParams& p, DType out, hipStream_t stream) {
  return out == DType::BF16 ? launch_typed<__bf16>(p, stream)
                            : launch_typed<float>(p, stream);
}

hipError_t launch_attn_fwd(const FwdParams& p, DType in, DType out, hipStream_t stream) {
  return in == DType::BF16 ? launch_attn_fwd_bf16(p, out, stream)
                           : launch_attn_fwd_f32(p, out, stream);
}

}  // namespace shattn
