// Internal declarations shared by the HIP sources of libtpshard (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpshard.h"

namespace tp {

// ------------------------------------------------------------------------------------------------------------------
// bfloat16 <-> float.  A bf16 value is the fp32 value whose top 16 bits are its pattern.
// ------------------------------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round to nearest, ties to even, with NaN mapped to a quiet NaN of the same sign.  Written out so that the
// reduction's output bits are fixed by this rule alone (used where outputs are compared bit for bit).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Hardware conversion (v_cvt_pk_bf16_f32, nearest-even) for GEMM epilogues.
__device__ __forceinline__ uint32_t f32_to_bf16_hw(float f) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f);
}
// Two floats -> a packed bf16 pair (lo in bits 0..15), nearest-even, as one v_cvt_pk_bf16_f32 (the two single
// conversions plus shift and or took four instructions).
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  typedef float f32x2_pk_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_pk_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_pk_t){lo, hi}, bf16x2_pk_t));
}

// ------------------------------------------------------------------------------------------------------------------
// Element-wise activations.
//
// GeLU (erf form) x * Phi(x) and its derivative Phi(x) + x * phi(x) take Phi from the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26: for z >= 0,
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2) + eps(z),  t = 1 / (1 + p z),  |eps| <= 1.5e-7,
// evaluated at z = |x| / sqrt(2), so exp(-z^2) = exp(-x^2 / 2) is also the Gaussian density's exponential.  One
// hardware reciprocal, one hardware exp2 and five FMAs replace the device library's erff (whose cost dominated the
// fused GeLU epilogues); the 1.5e-7 absolute error is far below bf16 output resolution.
// ------------------------------------------------------------------------------------------------------------------
struct NormalParts {
  float cdf;  // Phi(x)
  float pdf;  // phi(x) = exp(-x^2/2) / sqrt(2 pi)
};
__device__ __forceinline__ NormalParts normal_parts(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  const float e = __builtin_amdgcn_exp2f(-z * z * 1.44269504088896341f);  // exp(-z^2)
  float q = fmaf(1.061405429f, t, -1.453152027f);
  q = fmaf(q, t, 1.421413741f);
  q = fmaf(q, t, -0.284496736f);
  q = fmaf(q, t, 0.254829592f);
  q = q * t * e;  // erfc(z)
  NormalParts r;
  r.cdf = x >= 0.0f ? fmaf(-0.5f, q, 1.0f) : 0.5f * q;
  r.pdf = 0.39894228040143268f * e;  // a NaN x fails x >= 0 and reaches cdf through q
  return r;
}
__device__ __forceinline__ float act_gelu(float x) { return x * normal_parts(x).cdf; }
__device__ __forceinline__ float act_gelu_grad(float x) {
  const NormalParts n = normal_parts(x);
  return fmaf(x, n.pdf, n.cdf);
}
__device__ __forceinline__ float act_gelu_tanh(float x) {
  float u = 0.79788456080286536f * (x + 0.044715f * x * x * x);
  return 0.5f * x * (1.0f + tanhf(u));
}
__device__ __forceinline__ float act_gelu_tanh_grad(float x) {
  float u = 0.79788456080286536f * (x + 0.044715f * x * x * x);
  float th = tanhf(u);
  float du = 0.79788456080286536f * (1.0f + 3.0f * 0.044715f * x * x);
  return 0.5f * (1.0f + th) + 0.5f * x * (1.0f - th * th) * du;
}
// logistic sigmoid with the hardware exp2 and reciprocal (relative error a few ulp for |x| < 80; exact limits 0, 1)
__device__ __forceinline__ float act_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.44269504088896341f));
}

__device__ __forceinline__ float act_apply(int act, float x) {
  switch (act) {
    case TP_ACT_GELU: return act_gelu(x);
    case TP_ACT_GELU_TANH: return act_gelu_tanh(x);
    case TP_ACT_RELU: return x > 0.0f ? x : 0.0f;
    default: return x;
  }
}
__device__ __forceinline__ float act_grad(int act, float x) {
  switch (act) {
    case TP_ACT_GELU: return act_gelu_grad(x);
    case TP_ACT_GELU_TANH: return act_gelu_tanh_grad(x);
    case TP_ACT_RELU: return x > 0.0f ? 1.0f : 0.0f;
    default: return 1.0f;
  }
}

// ------------------------------------------------------------------------------------------------------------------
// Launch timing: when the calling thread is armed (tp_timing_begin), a LaunchTimer records the caller's start event
// before a launch and its stop event after it, on the launch stream, and logs the kernel name.
// ------------------------------------------------------------------------------------------------------------------
void timing_start(hipStream_t st, const char* name);
void timing_stop(hipStream_t st, const char* name);
struct LaunchTimer {
  hipStream_t st;
  const char* name;
  LaunchTimer(hipStream_t s, const char* n) : st(s), name(n) { timing_start(st, name); }
  ~LaunchTimer() { timing_stop(st, name); }
};

// Launch `kernel` on `stream` and evaluate to the launch status (hipGetLastError taken before the stop event).
#define TP_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                 \
  ([&]() -> hipError_t {                                                         \
    ::tp::LaunchTimer tp_launch_timer_((stream), (name));                        \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);         \
    return hipGetLastError();                                                    \
  }())

// ------------------------------------------------------------------------------------------------------------------
// GEMM description: C[m][n] = sum_k Aop(m, k) * Bop(n, k), then an epilogue.
// An operand is "K-major" when k is its contiguous index (row-major [rows][K]) and "MN-major" when m (or n) is
// ([K][rows]).  The forward column GEMM X A_i has K-major X and MN-major A_i; the dgrad GEMMs (x W^T) are K-major
// on both sides; the wgrad GEMMs (x^T y) are MN-major on both sides.
// ------------------------------------------------------------------------------------------------------------------
enum Epi {
  EPI_STORE = 0,       // C = acc
  EPI_BIAS = 1,        // C = acc + bias[n]
  EPI_BIAS_ACT = 2,    // C = u = acc + bias[n] (bias nullable); C2 = act(u)
  EPI_SWIGLU_FWD = 3,  // column pair (j, fhalf + j): C = [g | u] (+bias), C2[:, j] = silu(g) * u
  EPI_ACT_BWD = 4,     // C = acc * act'(aux[m][n])
  EPI_SWIGLU_BWD = 5,  // acc = dY[m][j]; aux = [g | u]: C[:, j] = dY*u*silu'(g), C[:, fhalf+j] = dY*silu(g)
  // LayerNorm folded into the column GEMM: A holds the LayerNorm input u and B the weight with gamma folded in
  // (diag(gamma) W); acc -> ln_rstd[m] * (acc - ln_mean[m] * ln_c[n]) + ln_b[n] (fp32 vectors), which is
  // LayerNorm(u) W + bias, then as EPI_BIAS_ACT / EPI_SWIGLU_FWD (p.bias unused).  Large-tile kernel only.
  EPI_LN_ACT = 6,
  EPI_LN_SWIGLU = 7
};
__host__ __device__ constexpr bool epi_swiglu_fwd(int e) { return e == EPI_SWIGLU_FWD || e == EPI_LN_SWIGLU; }
__host__ __device__ constexpr bool epi_ln(int e) { return e == EPI_LN_ACT || e == EPI_LN_SWIGLU; }

struct GemmParams {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int M, N, K;  // SwiGLU forward: N = 2 * fhalf (both halves)
  void* C;
  int64_t ldc;
  void* C2;
  int64_t ldc2;
  const void* bias;
  const void* aux;
  int64_t ldaux;
  int fhalf;
  int act;
  // EPI_LN_*: per-row mean and 1/std of the LayerNorm input [M], per-column sum of the folded weight's columns
  // and folded bias [N] (all fp32)
  const float* ln_mean;
  const float* ln_rstd;
  const float* ln_c;
  const float* ln_b;
};

// Launchers (return hipGetLastError after the launch).
hipError_t gemm_bf16(const GemmParams& p, bool a_kmajor, bool b_kmajor, int epi, hipStream_t st);
hipError_t gemm_bf16_wgrad_pair(const GemmParams& p0, const GemmParams& p1, hipStream_t st);
// gemm_bf16 given fp32 scratch (part_floats elements): a GEMM with too few output tiles to fill the GPU (store or
// bias epilogue, A K-major) splits K over several workgroups, writes fp32 partial tiles there and sums them in a
// fixed order with the epilogue; any other GEMM runs as gemm_bf16 and leaves the scratch alone.
hipError_t gemm_bf16_splitk(const GemmParams& p, bool a_kmajor, bool b_kmajor, int epi, float* part,
                            int64_t part_floats, hipStream_t st);
// gemm_bf16_wgrad_pair given fp32 scratch: when the pair's tiles overrun whole rounds of one tile per CU by a
// short tail, the tail tiles split K over several workgroups (fp32 partial blocks of 256 x 256 in the scratch,
// then a fixed-order sum); otherwise as gemm_bf16_wgrad_pair.
hipError_t gemm_bf16_wgrad_pair_splitk(const GemmParams& p0, const GemmParams& p1, float* part, int64_t part_floats,
                                       hipStream_t st);
hipError_t gemm_f32(const GemmParams& p, bool a_kmajor, bool b_kmajor, int epi, hipStream_t st);
// The LayerNorm-folded column GEMM (EPI_LN_ACT or EPI_LN_SWIGLU; A K-major, B MN-major) on the large-tile kernel;
// hipErrorInvalidValue when that kernel does not take the shape (K % 64 != 0 or K < 128).
hipError_t gemm_bf16_ln(const GemmParams& p, int epi, hipStream_t st);
// The fold: A_ln[k][j] = bf16(gamma[k] * A[k][j]), c[j] = sum_k A_ln[k][j], b[j] = sum_k beta[k] * A[k][j] + a[j]
// (a nullable), fp32 sums in a fixed order.  A [h, n] bf16 row-major, n % 2 == 0.
hipError_t ln_fold_weights(const void* gamma, const void* beta, const void* A, const void* a, int64_t h, int64_t n,
                           void* A_ln, float* c, float* b, hipStream_t st);
hipError_t colsum(tp_dtype dt, const void* x, int64_t rows, int64_t cols, void* out, hipStream_t st);

hipError_t reduce_partials(tp_dtype dt, const void* partials, int t, int64_t stride, int64_t in_off, int64_t count,
                           const void* bias, int64_t h, void* out, hipStream_t st);
hipError_t copy_bytes(const void* src, void* dst, int64_t bytes, hipStream_t st);
// QKV kinds: G query heads per KV head, gd = (KV heads) * d; other kinds ignore both.
hipError_t pack_columns(tp_dtype dt, const void* full, int64_t rows, int64_t full_cols, void* shard,
                        int64_t shard_cols, int kind, int64_t f_l, int64_t ffn, int64_t rank, int64_t hl, int64_t d,
                        int64_t ad, int64_t G, int64_t gd, hipStream_t st);

struct AttnParams {
  const void* qkv;  // [s, b, (hl + 2 hl/G) d]: per local KV group, its G query heads, then its K and V
  void* o;          // [s, b, hl*d]
  float* lse;       // [b, hl, s] or null
  int s, b, hl, d;
  int G;            // query heads per KV head (1: multi-head)
  int causal;
  float scale;      // 1/sqrt(d)
  int fold;         // set by the launcher: tile order for a grid resident all at once (see work_rank)
};
hipError_t attention_bf16(const AttnParams& p, hipStream_t st);
hipError_t attention_f32(const AttnParams& p, hipStream_t st);

// Attention backward core.  rec: per (batch, head, 64-query block) one 256-float record [lse(64) | D(64) | 0(128)]
// with D[q] = sum_e dO[q, e] O[q, e]; written by attention_bwd_prep, read by the dK/dV and dQ kernels.
struct AttnBwdParams {
  const void* qkv;   // [s, b, (hl + 2 hl/G) d], grouped as in AttnParams
  const void* o;     // [s, b, hl*d]
  const void* dout;  // [s, b, hl*d]
  const float* lse;  // [b, hl, s]
  float* rec;        // [b, hl, ceil(s/64), 256]
  void* dqkv;        // grouped like qkv; a KV head's dK / dV sum over its G query heads
  float* kvpart;     // G > 1, bf16: fp32 [G][s*b][hl/G][2d] per-head partial dK | dV (null: one workgroup per group)
  int s, b, hl, d;
  int G;             // query heads per KV head (1: multi-head)
  int causal;
  float scale;       // 1/sqrt(d)
  int fold;          // set by the launcher, as in AttnParams
};
hipError_t attention_bwd(tp_dtype dt, const AttnBwdParams& p, hipStream_t st);

// Sequence-parallel region: dropout + residual add + LayerNorm on one rank's [rows = s/t * b, h] slice.
struct SpFwdArgs {
  const void* z;
  const void* residual;  // nullable
  const uint32_t* bits;  // [rows, h], read only when p > 0
  const void* gamma;
  const void* beta;
  void* out;             // nullable
  void* y;
  float* mean;           // nullable
  float* rstd;           // nullable
  uint8_t* mask;         // nullable, [rows, h/8]
  int64_t rows, h;
  double p, eps;
};
struct SpBwdArgs {
  const void* u;
  const void* gamma;
  const float* mean;
  const float* rstd;
  const void* dy;
  const void* dres_in;   // nullable
  const uint8_t* mask;   // read only when p > 0
  void* dres;            // nullable
  void* dz;              // nullable
  float* dgamma;
  float* dbeta;
  float* ws;             // sp_bwd_blocks(rows) * 2h floats
  int64_t rows, h;
  double p;
};
constexpr int64_t SP_MAX_H = 12288;
constexpr int64_t SP_BWD_MAX_BLOCKS = 256;
int64_t sp_bwd_blocks(int64_t rows);
// The fixed device buffer that stands in for ws in the entry point that allocates nothing: 16 MiB, the partial
// rows of 256 workgroups at h = 8192.  sp_noalloc_scratch gives its address on the current device.
constexpr int64_t SP_NOALLOC_SCRATCH_BYTES = (int64_t)16 << 20;
hipError_t sp_noalloc_scratch(float** out);
hipError_t sp_dropout_add_ln_fwd(tp_dtype dt, const SpFwdArgs& a, hipStream_t st);
hipError_t sp_dropout_add_ln_bwd(tp_dtype dt, const SpBwdArgs& a, hipStream_t st);

// Vocab-parallel cross entropy.  stats: per row {max, sum of exp(x - max), target logit or 0, 0} as float4.
hipError_t vocab_ce_local(tp_dtype dt, const void* logits, const int32_t* targets, int64_t rows, int v, int rank,
                          float* stats, hipStream_t st);
hipError_t vocab_ce_combine(const float* stats, int t, int64_t rows, const int32_t* targets, float* loss, float* lse,
                            hipStream_t st);
hipError_t vocab_ce_bwd(tp_dtype dt, const void* logits, const int32_t* targets, const float* lse,
                        const float* dloss, int64_t rows, int v, int rank, void* dlogits, hipStream_t st);

}  // namespace tp
