// fp32 path: true fp32 products (FMA, no reduced-precision matrix format) for the fp32 workloads, with the same
// operand layouts and epilogues as the bf16 MFMA path.  64x64 output tile per workgroup, 16 k per LDS stage,
// each of the 256 threads owning a 4x4 set of outputs strided by 16 so LDS reads broadcast without conflicts.
#include <string>

#include "tp_common.h"

namespace tp {

namespace {

template <bool AK, bool BKM, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  constexpr bool SWIG = (EPI == EPI_SWIGLU_FWD);
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const float* __restrict__ A = static_cast<const float*>(p.A);
  const float* __restrict__ B = static_cast<const float*>(p.B);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64;
  const int tile_n = blockIdx.x;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      int r, k;
      if (AK) { r = e >> 4; k = e & 15; } else { k = e >> 6; r = e & 63; }
      const int m = m0 + r, kk = k0 + k;
      float v = 0.f;
      if (m < p.M && kk < p.K) v = AK ? A[(int64_t)m * p.lda + kk] : A[(int64_t)kk * p.lda + m];
      As[k][r] = v;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u;
      int c, k;
      if (BKM) { c = e >> 4; k = e & 15; } else { k = e >> 6; c = e & 63; }
      int col;
      bool valid;
      if (SWIG) {
        const int j = tile_n * 32 + (c & 31);
        valid = j < p.fhalf;
        col = (c >> 5) * p.fhalf + j;
      } else {
        col = tile_n * 64 + c;
        valid = col < p.N;
      }
      const int kk = k0 + k;
      float v = 0.f;
      if (valid && kk < p.K) v = BKM ? B[(int64_t)col * p.ldb + kk] : B[(int64_t)kk * p.ldb + col];
      Bs[k][c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = static_cast<float*>(p.C);
  float* C2 = static_cast<float*>(p.C2);
  const float* bias = static_cast<const float*>(p.bias);
  const float* aux = static_cast<const float*>(p.aux);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= p.M) continue;
    if constexpr (SWIG) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = tile_n * 32 + tx + 16 * j;
        if (col >= p.fhalf) continue;
        const float g = acc[i][j] + (bias ? bias[col] : 0.f);
        const float u = acc[i][j + 2] + (bias ? bias[p.fhalf + col] : 0.f);
        C[(int64_t)m * p.ldc + col] = g;
        C[(int64_t)m * p.ldc + p.fhalf + col] = u;
        C2[(int64_t)m * p.ldc2 + col] = g * act_sigmoid(g) * u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = tile_n * 64 + tx + 16 * j;
        if (col >= p.N) continue;
        const float v = acc[i][j];
        if constexpr (EPI == EPI_STORE) {
          C[(int64_t)m * p.ldc + col] = v;
        } else if constexpr (EPI == EPI_BIAS) {
          C[(int64_t)m * p.ldc + col] = v + (bias ? bias[col] : 0.f);
        } else if constexpr (EPI == EPI_BIAS_ACT) {
          const float u = v + (bias ? bias[col] : 0.f);
          C[(int64_t)m * p.ldc + col] = u;
          C2[(int64_t)m * p.ldc2 + col] = act_apply(p.act, u);
        } else if constexpr (EPI == EPI_ACT_BWD) {
          C[(int64_t)m * p.ldc + col] = v * act_grad(p.act, aux[(int64_t)m * p.ldaux + col]);
        } else if constexpr (EPI == EPI_SWIGLU_BWD) {
          const float g = aux[(int64_t)m * p.ldaux + col];
          const float u = aux[(int64_t)m * p.ldaux + p.fhalf + col];
          const float sg = act_sigmoid(g);
          C[(int64_t)m * p.ldc + col] = v * u * sg * (1.f + g * (1.f - sg));
          C[(int64_t)m * p.ldc + p.fhalf + col] = v * g * sg;
        }
      }
    }
  }
}

template <bool AK, bool BKM, int EPI>
hipError_t launch(const GemmParams& p, hipStream_t st) {
  const int nbn = (EPI == EPI_SWIGLU_FWD) ? (p.fhalf + 31) / 32 : (p.N + 63) / 64;
  const int nbm = (p.M + 63) / 64;
  static const std::string name = std::string("gemm_f32_") + (AK ? "K" : "M") + (BKM ? "K" : "M") + "_epi" +
                                  std::to_string(EPI);
  return TP_LAUNCH(name.c_str(), (gemm_f32_kernel<AK, BKM, EPI>), dim3((unsigned)nbn, (unsigned)nbm), dim3(256), 0, st,
                   p);
}

}  // namespace

hipError_t gemm_f32(const GemmParams& p, bool a_kmajor, bool b_kmajor, int epi, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (a_kmajor && !b_kmajor) {
    switch (epi) {
      case EPI_STORE: return launch<true, false, EPI_STORE>(p, st);
      case EPI_BIAS: return launch<true, false, EPI_BIAS>(p, st);
      case EPI_BIAS_ACT: return launch<true, false, EPI_BIAS_ACT>(p, st);
      case EPI_SWIGLU_FWD: return launch<true, false, EPI_SWIGLU_FWD>(p, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (a_kmajor && b_kmajor) {
    switch (epi) {
      case EPI_STORE: return launch<true, true, EPI_STORE>(p, st);
      case EPI_ACT_BWD: return launch<true, true, EPI_ACT_BWD>(p, st);
      case EPI_SWIGLU_BWD: return launch<true, true, EPI_SWIGLU_BWD>(p, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (!a_kmajor && !b_kmajor && epi == EPI_STORE) return launch<false, false, EPI_STORE>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace tp
