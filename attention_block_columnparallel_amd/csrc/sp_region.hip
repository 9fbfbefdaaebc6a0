// Sequence-parallel region kernels: dropout + residual add + LayerNorm on one rank's [s/t, b, h] slice, forward
// and backward.
//
// Under sequence parallelism the element-wise and per-token ops that sit between two tensor-parallel blocks
// (LayerNorm, dropout, the residual add) run on the rank's own 1/t of the sequence: the block output arrives by a
// reduce-scatter along s, and the LayerNorm output leaves by an all-gather along s into the next column GEMM
// ("Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" §5 SP rows and §6; "Sequence Parallel 与 Context
// Parallel", SP section; Megatron-LM visual reading, the sequence_parallel remark).  The pages name the ops but give
// no formulas; these kernels compute the standard definitions:
//
//   u    = residual + keep * z / (1 - p)       keep = (word >= floor(p * 2^32)), one 32-bit random word / element
//   y    = (u - mean(u)) * rstd * gamma + beta, rstd = 1 / sqrt(var(u) + eps), biased variance over the h columns
//   G    = dres_in + rstd * (g - mean(g) - xh * mean(g * xh)),   g = dy * gamma,  xh = (u - mean) * rstd
//   dz   = keep * G / (1 - p),  dres = G,  dgamma = sum_rows dy * xh,  dbeta = sum_rows dy
//
// Design.  Every kernel is HBM-bound (a handful of flops per element), so the layout serves the loads: one row is
// one workgroup (256 threads, 512 for h > 6144), each thread owning chunks of 8 consecutive columns (one 16-byte bf16 load per tensor and
// chunk; chunks c, c + 256, ... across the row so a wave's loads cover 1 KiB contiguous).  Row statistics are two
// block reductions (64-lane shuffles, then four per-wave partials through LDS in a fixed order, so results are
// deterministic); the two-pass variance uses the row held in registers.  The forward also packs the keep decisions
// into a bit mask (8 per byte, LSB first), 1/32 of the random words' bytes, so the backward never re-reads them.
// The LayerNorm reads the stored (rounded) u, so the forward and backward agree on its input.
//
// The backward cannot be one row per workgroup: dgamma / dbeta sum over rows.  A fixed grid of workgroups strides
// over the rows, keeps its column partial sums in registers, prefetches the next row while reducing the current
// one, and writes one fp32 partial row [dgamma | dbeta]; a second kernel sums the partials in a fixed order.
#include "tp_common.h"

#include <mutex>

// Scratch of the backward's entry point that allocates nothing: the partial [dgamma | dbeta] rows live here instead
// of in a caller workspace.  Each GPU holds its own copy until the process ends.  In host code this name is only a
// stand-in for the symbol; the device address comes from hipGetSymbolAddress (sp_noalloc_scratch).
static __device__ __align__(256) float scratch[tp::SP_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace tp {

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

// The address of `scratch` on the current device, looked up once per device (with that device current) and kept.
hipError_t sp_noalloc_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

constexpr int SP_THREADS = 256;

// 8 elements of a row <-> 8 floats.  bf16: one 16-byte access; fp32: two.
template <typename T>
struct Io;

template <>
struct Io<uint16_t> {
  static constexpr int W = 1;  // 16-byte words per 8 elements
  static __device__ __forceinline__ void unpack(const uint4* w, float* v) {
    v[0] = bf16_to_f32(w[0].x & 0xFFFFu);
    v[1] = bf16_to_f32(w[0].x >> 16);
    v[2] = bf16_to_f32(w[0].y & 0xFFFFu);
    v[3] = bf16_to_f32(w[0].y >> 16);
    v[4] = bf16_to_f32(w[0].z & 0xFFFFu);
    v[5] = bf16_to_f32(w[0].z >> 16);
    v[6] = bf16_to_f32(w[0].w & 0xFFFFu);
    v[7] = bf16_to_f32(w[0].w >> 16);
  }
  static __device__ __forceinline__ void load(const void* base, int64_t e, uint4* w) {
    w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
  }
  static __device__ __forceinline__ void store(void* base, int64_t e, const float* v) {
    uint4 o;
    o.x = pack_bf16x2_hw(v[0], v[1]);
    o.y = pack_bf16x2_hw(v[2], v[3]);
    o.z = pack_bf16x2_hw(v[4], v[5]);
    o.w = pack_bf16x2_hw(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + e) = o;
  }
  static __device__ __forceinline__ float round(float x) { return bf16_to_f32(f32_to_bf16_hw(x)); }
};

template <>
struct Io<float> {
  static constexpr int W = 2;
  static __device__ __forceinline__ void unpack(const uint4* w, float* v) {
    v[0] = __uint_as_float(w[0].x);
    v[1] = __uint_as_float(w[0].y);
    v[2] = __uint_as_float(w[0].z);
    v[3] = __uint_as_float(w[0].w);
    v[4] = __uint_as_float(w[1].x);
    v[5] = __uint_as_float(w[1].y);
    v[6] = __uint_as_float(w[1].z);
    v[7] = __uint_as_float(w[1].w);
  }
  static __device__ __forceinline__ void load(const void* base, int64_t e, uint4* w) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + e);
    w[0] = p[0];
    w[1] = p[1];
  }
  static __device__ __forceinline__ void store(void* base, int64_t e, const float* v) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + e);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ float round(float x) { return x; }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sums over the workgroup's NW waves: a 64-lane shuffle tree, then the per-wave partials through LDS added in wave
// order 0..NW-1 (deterministic).  `slot` is this reduction's LDS; the caller alternates slots so that one barrier per
// reduction suffices (a slot is rewritten only after every wave has passed a later barrier, hence has read it).
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* slot) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = slot[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += slot[w];
  return s;
}
template <int NW>
__device__ __forceinline__ float2 block_sum2(float a, float b, float* slot) {
  a = wave_sum(a);
  b = wave_sum(b);
  if ((threadIdx.x & 63) == 0) {
    slot[threadIdx.x >> 6] = a;
    slot[NW + (threadIdx.x >> 6)] = b;
  }
  __syncthreads();
  float sa = slot[0], sb = slot[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    sa += slot[w];
    sb += slot[NW + w];
  }
  return make_float2(sa, sb);
}

struct SpFwd {
  const void* z;
  const void* res;      // nullable
  const uint32_t* bits; // nullable when p == 0
  const void* gamma;
  const void* beta;
  void* out;            // nullable
  void* y;
  float* mean;          // nullable
  float* rstd;          // nullable
  uint8_t* mask;        // nullable
  int64_t rows;
  int h;
  uint32_t thr;         // keep iff word >= thr
  int drop;             // p > 0
  float scale;          // 1 / (1 - p)
  float eps;
};

template <typename T, int NV, int NT>
__global__ __launch_bounds__(NT) void sp_fwd_kernel(SpFwd p) {
  __shared__ float red[2][NT / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = p.h >> 3;
  const int64_t rbase = row * p.h;
  float u[NV][8];
  uint32_t kb[NV];
  uint4 wg[NV][Io<T>::W], wb[NV][Io<T>::W];  // gamma, beta: loaded with the row, used after the reductions
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = tid + j * NT;
    kb[j] = 0xFFu;
    if (c < nch) {
      Io<T>::load(p.gamma, 8 * c, wg[j]);
      Io<T>::load(p.beta, 8 * c, wb[j]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) u[j][i] = 0.0f;
    if (c < nch) {
      const int64_t e = rbase + 8 * c;
      uint4 wz[Io<T>::W], wr[Io<T>::W];
      Io<T>::load(p.z, e, wz);
      float z[8], r[8];
      Io<T>::unpack(wz, z);
      if (p.res != nullptr) {
        Io<T>::load(p.res, e, wr);
        Io<T>::unpack(wr, r);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = 0.0f;
      }
      if (p.drop) {
        const uint4* bp = reinterpret_cast<const uint4*>(p.bits + e);
        const uint4 b0 = bp[0], b1 = bp[1];
        const uint32_t w[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) m |= (w[i] >= p.thr ? 1u : 0u) << i;
        kb[j] = m;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float dz = ((kb[j] >> i) & 1u) ? z[i] * p.scale : 0.0f;
        u[j][i] = Io<T>::round(r[i] + dz);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) s += u[j][i];  // columns past h hold 0
  const float inv_h = 1.0f / (float)p.h;
  const float mean = block_sum<NT / 64>(s, red[0]) * inv_h;
  float q = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    if (tid + j * NT < nch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = u[j][i] - mean;
        q = fmaf(d, d, q);
      }
    }
  }
  const float var = block_sum<NT / 64>(q, red[1]) * inv_h;
  const float rstd = 1.0f / sqrtf(var + p.eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = tid + j * NT;
    if (c < nch) {
      const int64_t e = rbase + 8 * c;
      if (p.out != nullptr) Io<T>::store(p.out, e, u[j]);
      if (p.y != nullptr) {
        float g[8], b[8], y[8];
        Io<T>::unpack(wg[j], g);
        Io<T>::unpack(wb[j], b);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = fmaf((u[j][i] - mean) * rstd, g[i], b[i]);
        Io<T>::store(p.y, e, y);
      }
      if (p.mask != nullptr) p.mask[row * nch + c] = (uint8_t)kb[j];
    }
  }
  if (tid == 0) {
    if (p.mean != nullptr) p.mean[row] = mean;
    if (p.rstd != nullptr) p.rstd[row] = rstd;
  }
}

struct SpBwd {
  const void* u;
  const void* gamma;
  const float* mean;
  const float* rstd;
  const void* dy;
  const void* dres_in;  // nullable
  const uint8_t* mask;  // nullable when p == 0
  void* dres;           // nullable
  void* dz;             // nullable
  float* ws;            // [gridDim.x][2h] partial [dgamma | dbeta]
  int64_t rows;
  int h;
  int drop;
  float scale;
};

// One row's raw loads, held until the row is processed (the next row's are issued before this one is reduced).
template <typename T, int NV>
struct RowIn {
  uint4 u[NV][Io<T>::W];
  uint4 dy[NV][Io<T>::W];
  uint4 dr[NV][Io<T>::W];
  uint32_t m[NV];
  float mean, rstd;
};

template <typename T, int NV, int NT>
__device__ __forceinline__ void load_row(const SpBwd& p, int64_t row, int tid, int nch, RowIn<T, NV>& r) {
  const int64_t rbase = row * p.h;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = tid + j * NT;
    if (c < nch) {
      const int64_t e = rbase + 8 * c;
      Io<T>::load(p.u, e, r.u[j]);
      Io<T>::load(p.dy, e, r.dy[j]);
      if (p.dres_in != nullptr) Io<T>::load(p.dres_in, e, r.dr[j]);
      r.m[j] = p.drop ? (uint32_t)p.mask[row * nch + c] : 0xFFu;
    }
  }
  r.mean = p.mean[row];
  r.rstd = p.rstd[row];
}

template <typename T, int NV, int NT>
__global__ __launch_bounds__(NT) void sp_bwd_kernel(SpBwd p) {
  __shared__ float red[2][2 * (NT / 64)];
  const int tid = threadIdx.x;
  const int nch = p.h >> 3;
  const float inv_h = 1.0f / (float)p.h;
  // gamma stays packed; xh, g and dy are unpacked again after the row reduction rather than held across it
  uint4 gam[NV][Io<T>::W];
  float ag[NV][8], ab[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = tid + j * NT;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ag[j][i] = 0.0f;
      ab[j][i] = 0.0f;
    }
    if (c < nch) Io<T>::load(p.gamma, 8 * c, gam[j]);
  }
  int64_t row = blockIdx.x;
  RowIn<T, NV> cur;
  load_row<T, NV, NT>(p, row, tid, nch, cur);
  for (int it = 0; row < p.rows; ++it, row += gridDim.x) {
    RowIn<T, NV> nxt;
    const int64_t nrow = row + gridDim.x;
    if (nrow < p.rows) load_row<T, NV, NT>(p, nrow, tid, nch, nxt);
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (tid + j * NT < nch) {
        float u[8], dy[8], g[8];
        Io<T>::unpack(cur.u[j], u);
        Io<T>::unpack(cur.dy[j], dy);
        Io<T>::unpack(gam[j], g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xh = (u[i] - cur.mean) * cur.rstd;
          const float gg = dy[i] * g[i];
          s1 += gg;
          s2 = fmaf(gg, xh, s2);
        }
      }
    }
    const float2 s = block_sum2<NT / 64>(s1, s2, red[it & 1]);
    const float m1 = s.x * inv_h, m2 = s.y * inv_h;
    const int64_t rbase = row * p.h;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c = tid + j * NT;
      if (c < nch) {
        float u[8], dy[8], g[8], dr[8];
        Io<T>::unpack(cur.u[j], u);
        Io<T>::unpack(cur.dy[j], dy);
        Io<T>::unpack(gam[j], g);
        if (p.dres_in != nullptr) {
          Io<T>::unpack(cur.dr[j], dr);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) dr[i] = 0.0f;
        }
        float G[8], dz[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xh = (u[i] - cur.mean) * cur.rstd;
          G[i] = fmaf(cur.rstd, dy[i] * g[i] - m1 - xh * m2, dr[i]);
          dz[i] = ((cur.m[j] >> i) & 1u) ? G[i] * p.scale : 0.0f;
          ag[j][i] = fmaf(dy[i], xh, ag[j][i]);
          ab[j][i] += dy[i];
        }
        const int64_t e = rbase + 8 * c;
        if (p.dres != nullptr) Io<T>::store(p.dres, e, G);
        if (p.dz != nullptr) Io<T>::store(p.dz, e, dz);
      }
    }
    if (nrow < p.rows) cur = nxt;
  }
  float* wrow = p.ws + (int64_t)blockIdx.x * 2 * p.h;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = tid + j * NT;
    if (c < nch) {
      Io<float>::store(wrow, 8 * c, ag[j]);
      Io<float>::store(wrow + p.h, 8 * c, ab[j]);
    }
  }
}

// out[col] = sum over k = 0..nblk-1 of ws[k][col], col < n2 (n2 = 2h: dgamma then dbeta), summed in a fixed order:
// 16 row groups each add rows g, g + 16, ... in increasing k; the groups are then added in order 0..15.  Every
// thread issues all of its (at most SP_BWD_MAX_BLOCKS / 16) loads before the first add.
constexpr int CS_COLS = 64;  // columns per workgroup (16 threads x float4)
constexpr int CS_GROUPS = 16;
constexpr int CS_MAXK = (int)(SP_BWD_MAX_BLOCKS / CS_GROUPS);
__global__ __launch_bounds__(SP_THREADS) void sp_partial_colsum_kernel(const float* __restrict__ ws, int nblk,
                                                                       int n2, int h, float* __restrict__ dgamma,
                                                                       float* __restrict__ dbeta) {
  __shared__ float4 part[CS_GROUPS][CS_COLS / 4];
  const int tid = threadIdx.x;
  const int cq = tid & 15, grp = tid >> 4;
  const int col = blockIdx.x * CS_COLS + 4 * cq;
  float4 v[CS_MAXK];
#pragma unroll
  for (int i = 0; i < CS_MAXK; ++i) {
    const int k = grp + i * CS_GROUPS;
    v[i] = (col < n2 && k < nblk) ? *reinterpret_cast<const float4*>(ws + (int64_t)k * n2 + col)
                                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  float4 acc = v[0];
#pragma unroll
  for (int i = 1; i < CS_MAXK; ++i) {
    acc.x += v[i].x;
    acc.y += v[i].y;
    acc.z += v[i].z;
    acc.w += v[i].w;
  }
  part[grp][cq] = acc;
  __syncthreads();
  if (tid < 16 && col < n2) {
    float4 s = part[0][tid];
    for (int g = 1; g < CS_GROUPS; ++g) {
      const float4 w = part[g][tid];
      s.x += w.x;
      s.y += w.y;
      s.z += w.z;
      s.w += w.w;
    }
    // h is a multiple of 8, so a float4 never straddles the dgamma / dbeta boundary
    float* dst = col < h ? dgamma + col : dbeta + (col - h);
    *reinterpret_cast<float4*>(dst) = s;
  }
}

// Workgroup shape for a row of h columns: NV chunks of 8 columns per thread, NT threads.  At most 3 chunks per
// thread keeps the backward's row buffers (current + prefetched) and column sums in registers without spills.
template <typename T, template <typename, int, int> class L, typename... A>
hipError_t by_shape(int h, A... args) {
  const int nch = h / 8;
  if (nch <= 256) return L<T, 1, 256>::run(args...);
  if (nch <= 512) return L<T, 2, 256>::run(args...);
  if (nch <= 768) return L<T, 3, 256>::run(args...);
  if (nch <= 1024) return L<T, 2, 512>::run(args...);
  return L<T, 3, 512>::run(args...);  // h <= SP_MAX_H = 12288
}

template <typename T, int NV, int NT>
struct FwdLaunch {
  static hipError_t run(const SpFwd& p, hipStream_t st) {
    return TP_LAUNCH("sp_dropout_add_ln_fwd", (sp_fwd_kernel<T, NV, NT>), dim3((unsigned)p.rows), dim3(NT), 0, st,
                     p);
  }
};

template <typename T, int NV, int NT>
struct BwdLaunch {
  static hipError_t run(const SpBwd& p, int nblk, float* dgamma, float* dbeta, hipStream_t st) {
    hipError_t e = TP_LAUNCH("sp_dropout_add_ln_bwd", (sp_bwd_kernel<T, NV, NT>), dim3((unsigned)nblk), dim3(NT), 0,
                             st, p);
    if (e != hipSuccess) return e;
    const int n2 = 2 * p.h;
    return TP_LAUNCH("sp_ln_param_grad_sum", sp_partial_colsum_kernel,
                     dim3((unsigned)((n2 + CS_COLS - 1) / CS_COLS)), dim3(SP_THREADS), 0, st, (const float*)p.ws, nblk,
                     n2, p.h, dgamma, dbeta);
  }
};

}  // namespace

int64_t sp_bwd_blocks(int64_t rows) { return rows < SP_BWD_MAX_BLOCKS ? rows : SP_BWD_MAX_BLOCKS; }

hipError_t sp_dropout_add_ln_fwd(tp_dtype dt, const SpFwdArgs& a, hipStream_t st) {
  SpFwd p;
  p.z = a.z;
  p.res = a.residual;
  p.bits = a.bits;
  p.gamma = a.gamma;
  p.beta = a.beta;
  p.out = a.out;
  p.y = a.y;
  p.mean = a.mean;
  p.rstd = a.rstd;
  p.mask = a.mask;
  p.rows = a.rows;
  p.h = (int)a.h;
  p.drop = a.p > 0.0;
  p.thr = p.drop ? (uint32_t)floor(a.p * 4294967296.0) : 0u;
  p.scale = p.drop ? (float)(1.0 / (1.0 - a.p)) : 1.0f;
  p.eps = (float)a.eps;
  return dt == TP_BF16 ? by_shape<uint16_t, FwdLaunch>(p.h, p, st) : by_shape<float, FwdLaunch>(p.h, p, st);
}

hipError_t sp_dropout_add_ln_bwd(tp_dtype dt, const SpBwdArgs& a, hipStream_t st) {
  SpBwd p;
  p.u = a.u;
  p.gamma = a.gamma;
  p.mean = a.mean;
  p.rstd = a.rstd;
  p.dy = a.dy;
  p.dres_in = a.dres_in;
  p.mask = a.mask;
  p.dres = a.dres;
  p.dz = a.dz;
  p.ws = a.ws;
  p.rows = a.rows;
  p.h = (int)a.h;
  p.drop = a.p > 0.0;
  p.scale = p.drop ? (float)(1.0 / (1.0 - a.p)) : 1.0f;
  const int nblk = (int)sp_bwd_blocks(a.rows);
  return dt == TP_BF16 ? by_shape<uint16_t, BwdLaunch>(p.h, p, nblk, a.dgamma, a.dbeta, st)
                       : by_shape<float, BwdLaunch>(p.h, p, nblk, a.dgamma, a.dbeta, st);
}

}  // namespace tp
