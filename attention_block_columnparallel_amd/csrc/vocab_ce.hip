// Vocab-parallel cross entropy: each rank holds the logits of its vocab columns [rank*v, (rank+1)*v) for every
// token row; only per-row scalars cross ranks ("Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" §5, the
// vocab-parallel CE row: all-reduce(max), then all-reduce(sum), backward local; Megatron-LM visual reading, the
// remark that the column-parallel logits feed the loss directly).
//
//   local pass (per rank):  m_r = max_j x[i, j],  s_r = sum_j exp(x[i, j] - m_r),  tl_r = x[i, target - rank*v]
//                           when the target is in this rank's columns, else 0
//   combine (the two all-reduces, over the t ranks' per-row records):
//                           m = max_r m_r,  S = sum_r s_r exp(m_r - m),  lse = m + log S,  loss = lse - sum_r tl_r
//   backward (per rank):    dx[i, j] = (exp(x[i, j] - lse[i]) - [j is the target]) * dloss[i]
//
// A negative target marks an ignored row: loss 0 and a zero gradient row.  A target in no rank's columns gives NaN
// loss and lse (and so NaN gradients); a row whose logits are all -inf gives lse = -inf and a NaN loss.
//
// The local pass reads the logits once: each thread keeps a running (max, sum) over its chunks, rescaling the sum
// when the max rises, and the workgroup merges the (max, sum) pairs.  The max all-reduce then rescales each rank's
// sum by exp(m_r - m) instead of re-reading the logits with the global max; the value is the same up to rounding.
// All three kernels are HBM-bound: the local pass reads 2 bytes per bf16 logit, the backward reads 2 and writes 2.
#include "tp_common.h"

namespace tp {

namespace {

constexpr int CE_THREADS = 256;
constexpr float LOG2E = 1.44269504088896341f;
constexpr float LN2 = 0.69314718055994531f;

template <typename T>
struct Chunk8;

template <>
struct Chunk8<uint16_t> {  // 8 bf16 = one 16-byte access
  uint4 w;
  __device__ __forceinline__ void load(const void* base, int64_t e) {
    w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
  }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = bf16_to_f32(w.x & 0xFFFFu);
    v[1] = bf16_to_f32(w.x >> 16);
    v[2] = bf16_to_f32(w.y & 0xFFFFu);
    v[3] = bf16_to_f32(w.y >> 16);
    v[4] = bf16_to_f32(w.z & 0xFFFFu);
    v[5] = bf16_to_f32(w.z >> 16);
    v[6] = bf16_to_f32(w.w & 0xFFFFu);
    v[7] = bf16_to_f32(w.w >> 16);
  }
  static __device__ __forceinline__ void store(void* base, int64_t e, const float* v) {
    uint4 o;
    o.x = pack_bf16x2_hw(v[0], v[1]);
    o.y = pack_bf16x2_hw(v[2], v[3]);
    o.z = pack_bf16x2_hw(v[4], v[5]);
    o.w = pack_bf16x2_hw(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + e) = o;
  }
  static __device__ __forceinline__ float one(const void* base, int64_t e) {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[e]);
  }
};

template <>
struct Chunk8<float> {  // 8 fp32 = two 16-byte accesses
  float4 a, b;
  __device__ __forceinline__ void load(const void* base, int64_t e) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + e);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = a.x;
    v[1] = a.y;
    v[2] = a.z;
    v[3] = a.w;
    v[4] = b.x;
    v[5] = b.y;
    v[6] = b.z;
    v[7] = b.w;
  }
  static __device__ __forceinline__ void store(void* base, int64_t e, const float* v) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + e);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ float one(const void* base, int64_t e) {
    return static_cast<const float*>(base)[e];
  }
};

// (m, s) <- the pair for the union of two value sets, each given as (max, sum of exp(x - max)).  An empty set is
// (-inf, 0) and leaves the other unchanged.
__device__ __forceinline__ void merge(float& m, float& s, float om, float os) {
  if (om > m) {
    s = s * __builtin_amdgcn_exp2f((m - om) * LOG2E) + os;
    m = om;
  } else if (om != -INFINITY) {
    s += os * __builtin_amdgcn_exp2f((om - m) * LOG2E);
  }
}

// One workgroup per token row.  Chunks c = tid, tid + 256, ... of 8 columns; four chunks are loaded before any is
// folded into the running pair, so each thread keeps four 16-byte loads (bf16) in flight.
template <typename T>
__global__ __launch_bounds__(CE_THREADS) void ce_local_kernel(const void* __restrict__ logits,
                                                              const int32_t* __restrict__ targets, int v, int rank,
                                                              float4* __restrict__ stats) {
  __shared__ float red[2][CE_THREADS / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = v >> 3;
  const int64_t base = row * v;
  float m = -INFINITY, s = 0.0f;
  for (int c0 = tid; c0 < nch; c0 += 4 * CE_THREADS) {
    Chunk8<T> ch[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + k * CE_THREADS;
      if (c < nch) ch[k].load(logits, base + 8 * c);
    }
    // the four chunks' max first, then their exponentials against it and one merge into the running pair
    float x[4][8];
    float cm = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + k * CE_THREADS;
      if (c < nch) {
        ch[k].get(x[k]);
#pragma unroll
        for (int i = 0; i < 8; ++i) cm = fmaxf(cm, x[k][i]);
      }
    }
    const float nb = -cm * LOG2E;
    float cs = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + k * CE_THREADS;
      if (c < nch) {
#pragma unroll
        for (int i = 0; i < 8; ++i) cs += __builtin_amdgcn_exp2f(fmaf(x[k][i], LOG2E, nb));
      }
    }
    if (cm > -INFINITY) merge(m, s, cm, cs);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float om = __shfl_xor(m, off, 64);
    const float os = __shfl_xor(s, off, 64);
    merge(m, s, om, os);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = m;
    red[1][tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float M = red[0][0], S = red[1][0];
#pragma unroll
    for (int w = 1; w < CE_THREADS / 64; ++w) merge(M, S, red[0][w], red[1][w]);
    const int64_t local = (int64_t)targets[row] - (int64_t)rank * v;
    const bool mine = targets[row] >= 0 && local >= 0 && local < v;
    const float tl = mine ? Chunk8<T>::one(logits, base + local) : 0.0f;
    stats[row] = make_float4(M, S, tl, mine ? 1.0f : 0.0f);
  }
}

// One thread per row: the max all-reduce, the rescaled sum all-reduce (rank order 0..t-1), the target logit's sum.
__global__ __launch_bounds__(CE_THREADS) void ce_combine_kernel(const float4* __restrict__ stats, int t, int64_t rows,
                                                                const int32_t* __restrict__ targets,
                                                                float* __restrict__ loss, float* __restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * CE_THREADS + threadIdx.x;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int r = 0; r < t; ++r) m = fmaxf(m, stats[(int64_t)r * rows + row].x);
  float S = 0.0f, tl = 0.0f, owners = 0.0f;
  for (int r = 0; r < t; ++r) {
    const float4 st = stats[(int64_t)r * rows + row];
    if (m > -INFINITY) S += st.y * __builtin_amdgcn_exp2f((st.x - m) * LOG2E);
    tl += st.z;
    owners += st.w;
  }
  const int tg = targets[row];
  // a row of -inf logits has lse = -inf (its loss, -inf - (-inf), is NaN); a target in no rank's columns (at or past
  // t * v) is flagged with NaN in lse and loss, so the backward's exp(x - lse) turns NaN as well
  float l = m > -INFINITY ? m + __builtin_amdgcn_logf(S) * LN2 : -INFINITY;
  if (tg >= 0 && owners == 0.0f) l = __builtin_nanf("");
  if (lse != nullptr) lse[row] = l;
  loss[row] = tg >= 0 ? l - tl : 0.0f;
}

// One thread per 8-column chunk of the rank's [rows, v] logits.
template <typename T>
__global__ __launch_bounds__(CE_THREADS) void ce_bwd_kernel(const void* __restrict__ logits,
                                                            const int32_t* __restrict__ targets,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ dloss, int64_t rows, int v,
                                                            int rank, void* __restrict__ dlogits) {
  // one workgroup per row: the row's target, lse and dloss are read once, and each thread keeps four 16-byte
  // chunks of logits in flight
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = v >> 3;
  const int64_t base = row * v;
  const int tg = targets[row];
  const float l = lse[row], dl = dloss[row];
  const int64_t tloc = (int64_t)tg - (int64_t)rank * v;  // the target's column in this shard (if it is one)
  for (int c0 = tid; c0 < nch; c0 += 4 * CE_THREADS) {
    Chunk8<T> ch[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + k * CE_THREADS;
      if (c < nch && tg >= 0) ch[k].load(logits, base + 8 * c);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + k * CE_THREADS;
      if (c < nch) {
        float g[8];
        if (tg < 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) g[i] = 0.0f;
        } else {
          float x[8];
          ch[k].get(x);
          const int64_t local = tloc - 8 * c;  // the target's position within this chunk
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f((x[i] - l) * LOG2E);
            g[i] = (local == i ? p - 1.0f : p) * dl;
          }
        }
        Chunk8<T>::store(dlogits, base + 8 * c, g);
      }
    }
  }
}

}  // namespace

hipError_t vocab_ce_local(tp_dtype dt, const void* logits, const int32_t* targets, int64_t rows, int v, int rank,
                          float* stats, hipStream_t st) {
  float4* s4 = reinterpret_cast<float4*>(stats);
  if (dt == TP_BF16)
    return TP_LAUNCH("vocab_ce_local", ce_local_kernel<uint16_t>, dim3((unsigned)rows), dim3(CE_THREADS), 0, st,
                     logits, targets, v, rank, s4);
  return TP_LAUNCH("vocab_ce_local", ce_local_kernel<float>, dim3((unsigned)rows), dim3(CE_THREADS), 0, st, logits,
                   targets, v, rank, s4);
}

hipError_t vocab_ce_combine(const float* stats, int t, int64_t rows, const int32_t* targets, float* loss, float* lse,
                            hipStream_t st) {
  const unsigned blocks = (unsigned)((rows + CE_THREADS - 1) / CE_THREADS);
  return TP_LAUNCH("vocab_ce_combine", ce_combine_kernel, dim3(blocks), dim3(CE_THREADS), 0, st,
                   reinterpret_cast<const float4*>(stats), t, rows, targets, loss, lse);
}

hipError_t vocab_ce_bwd(tp_dtype dt, const void* logits, const int32_t* targets, const float* lse,
                        const float* dloss, int64_t rows, int v, int rank, void* dlogits, hipStream_t st) {
  const unsigned blocks = (unsigned)rows;  // one workgroup per row
  if (dt == TP_BF16)
    return TP_LAUNCH("vocab_ce_bwd", ce_bwd_kernel<uint16_t>, dim3(blocks), dim3(CE_THREADS), 0, st, logits,
                     targets, lse, dloss, rows, v, rank, dlogits);
  return TP_LAUNCH("vocab_ce_bwd", ce_bwd_kernel<float>, dim3(blocks), dim3(CE_THREADS), 0, st, logits, targets,
                   lse, dloss, rows, v, rank, dlogits);
}

}  // namespace tp
