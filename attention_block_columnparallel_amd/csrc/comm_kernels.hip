// Bandwidth-bound kernels: the g / f reduction over t partial buffers (all-reduce form and dim-0 reduce-scatter
// form), the dim-0 gather copy, the shard packer and the bias-gradient column sum.
//
// The reduction follows the g operator of "Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" (§2, the f/g
// table; §5 the SP variants): the block output is the element-wise sum of the ranks' partials.  On one GPU the t
// partial buffers sit side by side ([t][n]); each output element is read from every buffer once and written once,
// so the kernel is HBM-bound: 16-byte loads and stores, fp32 accumulation in rank order 0..t-1, the row bias
// last, one rounding.  Every thread keeps VPT * t independent 16-byte loads in flight.
#include "tp_common.h"

namespace tp {

namespace {

constexpr int RED_THREADS = 256;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte accesses: every partial is read exactly once and every output written once.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(uint4* p, const uint4& v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ void acc_add8(float* acc, const uint4& v) {
  acc[0] += bf16_to_f32(v.x & 0xFFFFu);
  acc[1] += bf16_to_f32(v.x >> 16);
  acc[2] += bf16_to_f32(v.y & 0xFFFFu);
  acc[3] += bf16_to_f32(v.y >> 16);
  acc[4] += bf16_to_f32(v.z & 0xFFFFu);
  acc[5] += bf16_to_f32(v.z >> 16);
  acc[6] += bf16_to_f32(v.w & 0xFFFFu);
  acc[7] += bf16_to_f32(v.w >> 16);
}
__device__ __forceinline__ void acc_set8(float* acc, const uint4& v) {
  acc[0] = bf16_to_f32(v.x & 0xFFFFu);
  acc[1] = bf16_to_f32(v.x >> 16);
  acc[2] = bf16_to_f32(v.y & 0xFFFFu);
  acc[3] = bf16_to_f32(v.y >> 16);
  acc[4] = bf16_to_f32(v.z & 0xFFFFu);
  acc[5] = bf16_to_f32(v.z >> 16);
  acc[6] = bf16_to_f32(v.w & 0xFFFFu);
  acc[7] = bf16_to_f32(v.w >> 16);
}
__device__ __forceinline__ uint4 pack8(const float* acc) {
  uint4 o;
  o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  return o;
}

// bf16, compile-time t: vector index v covers elements [8v, 8v+8) of the slice that starts at in_off.
template <int T, int VPT>
__global__ __launch_bounds__(RED_THREADS) void reduce_bf16_t(const uint16_t* __restrict__ P, int64_t stride,
                                                             int64_t in_off, int64_t nvec,
                                                             const uint16_t* __restrict__ bias, int64_t h,
                                                             uint16_t* __restrict__ out) {
  const int64_t v0 = (int64_t)blockIdx.x * (RED_THREADS * VPT) + threadIdx.x;
  uint4 r[VPT][T];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int64_t v = v0 + (int64_t)u * RED_THREADS;
    if (v < nvec) {
      const uint4* src = reinterpret_cast<const uint4*>(P + in_off) + v;
#pragma unroll
      for (int i = 0; i < T; ++i) r[u][i] = ld_stream(src + (stride >> 3) * i);
    }
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int64_t v = v0 + (int64_t)u * RED_THREADS;
    if (v < nvec) {
      float acc[8];
      acc_set8(acc, r[u][0]);
#pragma unroll
      for (int i = 1; i < T; ++i) acc_add8(acc, r[u][i]);
      if (bias != nullptr) {
        const int64_t col = (in_off + v * 8) % h;
        acc_add8(acc, *reinterpret_cast<const uint4*>(bias + col));
      }
      st_stream(reinterpret_cast<uint4*>(out) + v, pack8(acc));
    }
  }
}

// bf16, runtime t, one vector per thread.
__global__ __launch_bounds__(RED_THREADS) void reduce_bf16_any(const uint16_t* __restrict__ P, int t, int64_t stride,
                                                               int64_t in_off, int64_t nvec,
                                                               const uint16_t* __restrict__ bias, int64_t h,
                                                               uint16_t* __restrict__ out) {
  const int64_t v = (int64_t)blockIdx.x * RED_THREADS + threadIdx.x;
  if (v >= nvec) return;
  const uint4* src = reinterpret_cast<const uint4*>(P + in_off) + v;
  float acc[8];
  acc_set8(acc, src[0]);
  for (int i = 1; i < t; ++i) acc_add8(acc, src[(stride >> 3) * i]);
  if (bias != nullptr) acc_add8(acc, *reinterpret_cast<const uint4*>(bias + (in_off + v * 8) % h));
  reinterpret_cast<uint4*>(out)[v] = pack8(acc);
}

// Element-wise fallback (any alignment / tail), bf16 or fp32.
template <bool BF16>
__global__ __launch_bounds__(RED_THREADS) void reduce_scalar(const void* __restrict__ P, int t, int64_t stride,
                                                             int64_t in_off, int64_t e0, int64_t count,
                                                             const void* __restrict__ bias, int64_t h,
                                                             void* __restrict__ out) {
  const int64_t e = e0 + (int64_t)blockIdx.x * RED_THREADS + threadIdx.x;
  if (e >= count) return;
  const int64_t src = in_off + e;
  if (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(P);
    float acc = bf16_to_f32(p[src]);
    for (int i = 1; i < t; ++i) acc += bf16_to_f32(p[src + stride * i]);
    if (bias != nullptr) acc += bf16_to_f32(static_cast<const uint16_t*>(bias)[src % h]);
    static_cast<uint16_t*>(out)[e] = (uint16_t)f32_to_bf16_rne(acc);
  } else {
    const float* p = static_cast<const float*>(P);
    float acc = p[src];
    for (int i = 1; i < t; ++i) acc += p[src + stride * i];
    if (bias != nullptr) acc += static_cast<const float*>(bias)[src % h];
    static_cast<float*>(out)[e] = acc;
  }
}

// fp32, runtime t, 4 floats per vector.
__global__ __launch_bounds__(RED_THREADS) void reduce_f32_vec(const float* __restrict__ P, int t, int64_t stride,
                                                              int64_t in_off, int64_t nvec,
                                                              const float* __restrict__ bias, int64_t h,
                                                              float* __restrict__ out) {
  const int64_t v = (int64_t)blockIdx.x * RED_THREADS + threadIdx.x;
  if (v >= nvec) return;
  const float4* src = reinterpret_cast<const float4*>(P + in_off) + v;
  float4 acc = src[0];
  for (int i = 1; i < t; ++i) {
    float4 x = src[(stride >> 2) * i];
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  if (bias != nullptr) {
    float4 x = *reinterpret_cast<const float4*>(bias + (in_off + v * 4) % h);
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  reinterpret_cast<float4*>(out)[v] = acc;
}

template <int T>
hipError_t launch_reduce_bf16_t(const uint16_t* P, int64_t stride, int64_t in_off, int64_t nvec, const uint16_t* bias,
                                int64_t h, uint16_t* out, hipStream_t st) {
  constexpr int VPT = (T <= 2) ? 4 : 2;
  const int64_t per_block = (int64_t)RED_THREADS * VPT;
  const int64_t blocks = (nvec + per_block - 1) / per_block;
  return TP_LAUNCH(T == 8 ? "reduce_bf16_t8" : T == 4 ? "reduce_bf16_t4" : T == 2 ? "reduce_bf16_t2" : "reduce_bf16_t1",
                   (reduce_bf16_t<T, VPT>), dim3((unsigned)blocks), dim3(RED_THREADS), 0, st, P, stride, in_off, nvec,
                   bias, h, out);
}

// ------------------------------------------------------------------------------------------------------------------
// Copy (dim-0 gather of contiguous slices) and packer.
// ------------------------------------------------------------------------------------------------------------------
// Each thread moves COPY_VPT 16-byte vectors, all loads in flight before the first store; consecutive threads
// take consecutive vectors, so every wave-wide access is 1 KB contiguous.
constexpr int COPY_VPT = 8;
__global__ __launch_bounds__(256) void copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t nvec) {
  const int64_t v0 = (int64_t)blockIdx.x * (256 * COPY_VPT) + threadIdx.x;
  uint4 r[COPY_VPT];
#pragma unroll
  for (int u = 0; u < COPY_VPT; ++u) {
    const int64_t v = v0 + (int64_t)u * 256;
    if (v < nvec) r[u] = ld_stream(src + v);
  }
#pragma unroll
  for (int u = 0; u < COPY_VPT; ++u) {
    const int64_t v = v0 + (int64_t)u * 256;
    if (v < nvec) st_stream(dst + v, r[u]);
  }
}
__global__ __launch_bounds__(256) void copy1(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// Full-matrix column of shard column c ("Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" §2-3 and the
// Megatron-LM visual reading: fc1 split by output column, SwiGLU keeps gate and up columns of the same range,
// QKV split by head with each local head's q, k, v columns kept together).
__device__ __forceinline__ int64_t shard_src_col(int kind, int64_t c, int64_t f_l, int64_t ffn, int64_t rank,
                                                 int64_t hl, int64_t d, int64_t ad, int64_t G, int64_t gd) {
  switch (kind) {
    case TP_W_FC1:
    case TP_B_FC1:
      return rank * f_l + c;
    case TP_W_FC1_GATE_UP:
    case TP_B_FC1_GATE_UP:
      return c < f_l ? rank * f_l + c : ffn + rank * f_l + (c - f_l);
    default: {  // TP_W_QKV, TP_B_QKV: per local KV group [its G query heads | k | v]; full [Wq | Wk | Wv]
      const int64_t gw = (G + 2) * d;
      const int64_t jg = c / gw, rem = c % gw;
      const int64_t slot = rem / d, e = rem % d;
      const int64_t grp = rank * (hl / G) + jg;
      if (slot < G) return (grp * G + slot) * d + e;
      return ad + (slot == G ? 0 : gd) + grp * d + e;
    }
  }
}

// One thread per (row, VEC-element group); a group never straddles a segment because every segment width is a
// multiple of VEC (checked by the launcher).
template <typename V, int VEC, int ESZ>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ full, int64_t rows, int64_t full_cols,
                                                   uint8_t* __restrict__ shard, int64_t shard_cols, int kind,
                                                   int64_t f_l, int64_t ffn, int64_t rank, int64_t hl, int64_t d,
                                                   int64_t ad, int64_t G, int64_t gd) {
  const int64_t groups = shard_cols / VEC;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= rows * groups) return;
  const int64_t row = g / groups, c = (g % groups) * VEC;
  const int64_t sc = shard_src_col(kind, c, f_l, ffn, rank, hl, d, ad, G, gd);
  const V* src = reinterpret_cast<const V*>(full + (row * full_cols + sc) * ESZ);
  V* dst = reinterpret_cast<V*>(shard + (row * shard_cols + c) * ESZ);
  *dst = *src;
}

// Bias gradient: out[n] = sum over rows of x[row][n], fp32 accumulation, one rounding.
template <bool BF16>
__global__ __launch_bounds__(256) void colsum_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                     void* __restrict__ out) {
  __shared__ float part[4][64];
  const int lane_c = threadIdx.x & 63, lane_r = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane_c;
  float acc = 0.0f;
  if (c < cols) {
    for (int64_t r = lane_r; r < rows; r += 4) {
      acc += BF16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[r * cols + c]) : static_cast<const float*>(x)[r * cols + c];
    }
  }
  part[lane_r][lane_c] = acc;
  __syncthreads();
  if (lane_r == 0 && c < cols) {
    const float s = ((part[0][lane_c] + part[1][lane_c]) + part[2][lane_c]) + part[3][lane_c];
    if (BF16)
      static_cast<uint16_t*>(out)[c] = (uint16_t)f32_to_bf16_rne(s);
    else
      static_cast<float*>(out)[c] = s;
  }
}

}  // namespace

hipError_t reduce_partials(tp_dtype dt, const void* partials, int t, int64_t stride, int64_t in_off, int64_t count,
                           const void* bias, int64_t h, void* out, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const bool bf16 = (dt == TP_BF16);
  const int vec = bf16 ? 8 : 4;
  const bool aligned = (stride % vec == 0) && (in_off % vec == 0) && (bias == nullptr || h % vec == 0) &&
                       ((uintptr_t)partials % 16 == 0) && ((uintptr_t)out % 16 == 0) &&
                       (bias == nullptr || (uintptr_t)bias % 16 == 0);
  int64_t done = 0;
  if (aligned) {
    const int64_t nvec = count / vec;
    if (nvec > 0) {
      hipError_t e = hipSuccess;
      if (bf16) {
        const uint16_t* P = static_cast<const uint16_t*>(partials);
        const uint16_t* B = static_cast<const uint16_t*>(bias);
        uint16_t* O = static_cast<uint16_t*>(out);
        switch (t) {
          case 1: e = launch_reduce_bf16_t<1>(P, stride, in_off, nvec, B, h, O, st); break;
          case 2: e = launch_reduce_bf16_t<2>(P, stride, in_off, nvec, B, h, O, st); break;
          case 4: e = launch_reduce_bf16_t<4>(P, stride, in_off, nvec, B, h, O, st); break;
          case 8: e = launch_reduce_bf16_t<8>(P, stride, in_off, nvec, B, h, O, st); break;
          default: {
            const int64_t blocks = (nvec + RED_THREADS - 1) / RED_THREADS;
            e = TP_LAUNCH("reduce_bf16_any", reduce_bf16_any, dim3((unsigned)blocks), dim3(RED_THREADS), 0, st, P, t,
                          stride, in_off, nvec, B, h, O);
          }
        }
      } else {
        const int64_t blocks = (nvec + RED_THREADS - 1) / RED_THREADS;
        e = TP_LAUNCH("reduce_f32_vec", reduce_f32_vec, dim3((unsigned)blocks), dim3(RED_THREADS), 0, st,
                      static_cast<const float*>(partials), t, stride, in_off, nvec, static_cast<const float*>(bias), h,
                      static_cast<float*>(out));
      }
      if (e != hipSuccess) return e;
    }
    done = (count / vec) * vec;
  }
  if (done < count) {
    const int64_t rest = count - done;
    const int64_t blocks = (rest + RED_THREADS - 1) / RED_THREADS;
    if (bf16)
      return TP_LAUNCH("reduce_scalar_bf16", reduce_scalar<true>, dim3((unsigned)blocks), dim3(RED_THREADS), 0, st,
                       partials, t, stride, in_off, done, count, bias, h, out);
    return TP_LAUNCH("reduce_scalar_f32", reduce_scalar<false>, dim3((unsigned)blocks), dim3(RED_THREADS), 0, st,
                     partials, t, stride, in_off, done, count, bias, h, out);
  }
  return hipSuccess;
}

hipError_t copy_bytes(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  if (bytes <= 0) return hipSuccess;
  int64_t done = 0;
  if ((uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0) {
    const int64_t nvec = bytes / 16;
    if (nvec > 0) {
      const int64_t blocks = (nvec + 256 * COPY_VPT - 1) / (256 * COPY_VPT);
      hipError_t e = TP_LAUNCH("copy16", copy16, dim3((unsigned)blocks), dim3(256), 0, st,
                               static_cast<const uint4*>(src), static_cast<uint4*>(dst), nvec);
      if (e != hipSuccess) return e;
    }
    done = nvec * 16;
  }
  if (done < bytes) {
    const int64_t rest = bytes - done;
    return TP_LAUNCH("copy1", copy1, dim3((unsigned)((rest + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint8_t*>(src) + done, static_cast<uint8_t*>(dst) + done, rest);
  }
  return hipSuccess;
}

hipError_t pack_columns(tp_dtype dt, const void* full, int64_t rows, int64_t full_cols, void* shard,
                        int64_t shard_cols, int kind, int64_t f_l, int64_t ffn, int64_t rank, int64_t hl, int64_t d,
                        int64_t ad, int64_t G, int64_t gd, hipStream_t st) {
  const int esz = dt == TP_BF16 ? 2 : 4;
  // segment widths: f_l (FC kinds) or d (QKV kinds)
  const int64_t seg = (kind == TP_W_QKV || kind == TP_B_QKV) ? d : f_l;
  const bool vec_ok = ((seg * esz) % 16 == 0) && ((full_cols * esz) % 16 == 0) && ((shard_cols * esz) % 16 == 0) &&
                      ((uintptr_t)full % 16 == 0) && ((uintptr_t)shard % 16 == 0);
  const uint8_t* F = static_cast<const uint8_t*>(full);
  uint8_t* S = static_cast<uint8_t*>(shard);
  if (vec_ok) {
    const int vec = 16 / esz;
    const int64_t n = rows * (shard_cols / vec);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (esz == 2)
      return TP_LAUNCH("pack_vec_bf16", (pack_kernel<uint4, 8, 2>), dim3(blocks), dim3(256), 0, st, F, rows, full_cols,
                       S, shard_cols, kind, f_l, ffn, rank, hl, d, ad, G, gd);
    return TP_LAUNCH("pack_vec_f32", (pack_kernel<uint4, 4, 4>), dim3(blocks), dim3(256), 0, st, F, rows, full_cols, S,
                     shard_cols, kind, f_l, ffn, rank, hl, d, ad, G, gd);
  } else {
    const int64_t n = rows * shard_cols;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (esz == 2)
      return TP_LAUNCH("pack_elem_bf16", (pack_kernel<uint16_t, 1, 2>), dim3(blocks), dim3(256), 0, st, F, rows,
                       full_cols, S, shard_cols, kind, f_l, ffn, rank, hl, d, ad, G, gd);
    return TP_LAUNCH("pack_elem_f32", (pack_kernel<uint32_t, 1, 4>), dim3(blocks), dim3(256), 0, st, F, rows,
                     full_cols, S, shard_cols, kind, f_l, ffn, rank, hl, d, ad, G, gd);
  }
}

hipError_t colsum(tp_dtype dt, const void* x, int64_t rows, int64_t cols, void* out, hipStream_t st) {
  const unsigned blocks = (unsigned)((cols + 63) / 64);
  if (dt == TP_BF16)
    return TP_LAUNCH("colsum_bf16", colsum_kernel<true>, dim3(blocks), dim3(256), 0, st, x, rows, cols, out);
  return TP_LAUNCH("colsum_f32", colsum_kernel<false>, dim3(blocks), dim3(256), 0, st, x, rows, cols, out);
}

}  // namespace tp
