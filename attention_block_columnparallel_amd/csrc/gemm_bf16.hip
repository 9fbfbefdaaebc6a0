// bf16 GEMMs on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation) for every GEMM of the
// column->row block: the column GEMM X A_i with its fused bias + GeLU / SwiGLU epilogue, the row GEMM Y_i B_i,
// the dgrad GEMMs dZ B_i^T (fused with act') and dU_i A_i^T, and the wgrad GEMMs Y_i^T dZ and X^T dU_i
// ("Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" §2; the backward section of the 111qqz
// "tensor-parallelism-matrix-split" post).
//
// Design (one workgroup = one BM x BN output tile, NWM x NWN waves of 64 lanes, K stepped by 64):
//   * Operand tiles are staged through LDS as [row][k] with 64 k per row (8 chunks of 16 bytes).  A K-major
//     operand is copied chunk for chunk; an MN-major operand (the weight in X A_i, both operands of a wgrad) is
//     read as 8(k) x 4(mn) blocks and transposed in registers before the LDS store, so every MFMA fragment is one
//     16-byte LDS read no matter how the operand sits in HBM.
//   * Chunk c of row r is stored at chunk c ^ ((r ^ (r >> 2)) & 7): eight consecutive rows read at one logical
//     chunk hit eight distinct 16-byte bank groups, and so do the transposed stores of eight consecutive blocks.
//   * Two LDS stages; the next K tile's global loads are issued into registers before the current tile's MFMAs
//     and written to the other stage after them, with one barrier per K tile.
//   * Tiles are ordered XCD-aware: the hardware deals workgroup i to XCD i % 8, so the launch index is remapped
//     to give each XCD a contiguous run of tiles, walked in groups of GROUP_M row tiles so the A rows and B
//     columns an XCD touches stay in its own L2.
#include <string>

#include "tp_common.h"

namespace tp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int GROUP_M = 8;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 2)) & 7; }

// Physical column of logical output column `c` of the tile that starts at logical column n0.  Plain GEMMs map
// one to one.  The SwiGLU forward tile holds, per wave, WN/2 gate columns followed by the same WN/2 up columns,
// so each lane ends up with the gate and up accumulators of one output column j.
template <bool SWIG, int WN>
__device__ __forceinline__ int phys_col(int tile_n, int BN, int c, int fhalf, int N, bool& valid) {
  if (!SWIG) {
    const int col = tile_n * BN + c;
    valid = col < N;
    return col;
  }
  const int wn = c / WN, cw = c % WN;
  const int half = cw / (WN / 2), jj = cw % (WN / 2);
  const int j = tile_n * (BN / 2) + wn * (WN / 2) + jj;
  valid = j < fhalf;
  return half * fhalf + j;
}

// K-major operand: R rows x 64 k, 16-byte chunks, thread q -> row q/8, chunk q%8.
template <int R, int NT>
struct LoadK {
  static constexpr int TOTAL = R * 8;
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  uint4 v[PER];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int row0, int rows, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * NT;
      const int r = q >> 3, c = q & 7;
      const int row = row0 + r, k = k0 + c * 8;
      if ((TOTAL % NT == 0 || q < TOTAL) && row < rows && k < K)
        v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + k);
      else
        v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * NT;
      if (TOTAL % NT == 0 || q < TOTAL) {
        const int r = q >> 3, c = q & 7;
        lds[r * 8 + (c ^ swz(r))] = v[i];
      }
    }
  }
};

// MN-major operand: 64 k rows x R columns (columns contiguous in HBM).  Thread q takes the block of 8 k rows x 4
// columns (kg = q / (R/4), g = q % (R/4)); consecutive threads read consecutive 8-byte column groups of one k row.
template <int R, int NT, bool SWIG, int WN>
struct LoadMN {
  static constexpr int GROUPS = R / 4;
  static constexpr int TOTAL = 8 * GROUPS;
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  uint2 v[PER][8];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int tile_n, int N, int fhalf,
                                       int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * NT;
      const int g = q % GROUPS, kg = q / GROUPS;
      bool valid = false;
      const int col = phys_col<SWIG, WN>(tile_n, R, g * 4, fhalf, N, valid);
      valid = valid && (TOTAL % NT == 0 || q < TOTAL);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = k0 + kg * 8 + j;
        if (valid && k < K)
          v[i][j] = *reinterpret_cast<const uint2*>(base + (int64_t)k * ld + col);
        else
          v[i][j] = make_uint2(0u, 0u);
      }
    }
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = tid + i * NT;
      if (TOTAL % NT == 0 || q < TOTAL) {
        const int g = q % GROUPS, kg = q / GROUPS;
        uint32_t w[4][4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t x0 = v[i][2 * p].x, x1 = v[i][2 * p + 1].x;
          const uint32_t y0 = v[i][2 * p].y, y1 = v[i][2 * p + 1].y;
          w[0][p] = (x0 & 0xFFFFu) | (x1 << 16);
          w[1][p] = (x0 >> 16) | (x1 & 0xFFFF0000u);
          w[2][p] = (y0 & 0xFFFFu) | (y1 << 16);
          w[3][p] = (y0 >> 16) | (y1 & 0xFFFF0000u);
        }
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
          const int r = g * 4 + jn;
          lds[r * 8 + (kg ^ swz(r))] = make_uint4(w[jn][0], w[jn][1], w[jn][2], w[jn][3]);
        }
      }
    }
  }
};

template <bool KMAJ, int R, int NT, bool SWIG, int WN>
struct Loader;
template <int R, int NT, bool SWIG, int WN>
struct Loader<true, R, NT, SWIG, WN> {
  LoadK<R, NT> l;
  __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int tile, int rows, int fhalf, int k0, int K,
                                       int tid) {
    l.load(base, ld, tile * R, rows, k0, K, tid);
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const { l.store(lds, tid); }
};
template <int R, int NT, bool SWIG, int WN>
struct Loader<false, R, NT, SWIG, WN> {
  LoadMN<R, NT, SWIG, WN> l;
  __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int tile, int rows, int fhalf, int k0, int K,
                                       int tid) {
    l.load(base, ld, tile, rows, fhalf, k0, K, tid);
  }
  __device__ __forceinline__ void store(uint4* lds, int tid) const { l.store(lds, tid); }
};

__device__ __forceinline__ uint16_t ldg_bf16(const void* p, int64_t i) {
  return static_cast<const uint16_t*>(p)[i];
}
__device__ __forceinline__ void stg_bf16(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_hw(v);
}

template <int BM, int BN, int NWM, int NWN, bool AK, bool BKM, int EPI>
__global__ __launch_bounds__(NWM* NWN * 64) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = NWM * NWN * 64;
  constexpr int WM = BM / NWM, WN = BN / NWN;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr bool SWIG = (EPI == EPI_SWIGLU_FWD);
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(!SWIG || (TN % 2 == 0), "SwiGLU needs an even number of 16-column subtiles per wave");

  __shared__ uint4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;

  // ---- tile index: XCD-aware remap, then grouped row-major walk
  const int nbm = (p.M + BM - 1) / BM;
  const int nbn = SWIG ? (p.fhalf + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  const int nb = nbm * nbn;
  int bid = blockIdx.x;
  {
    const int q = nb / 8, r = nb % 8;
    const int xcd = bid % 8, idx = bid / 8;
    bid = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  }
  const int group = bid / (GROUP_M * nbn);
  const int first_m = group * GROUP_M;
  const int gsz = min(nbm - first_m, GROUP_M);
  const int tile_m = first_m + (bid % (GROUP_M * nbn)) % gsz;
  const int tile_n = (bid % (GROUP_M * nbn)) / gsz;

  const uint16_t* __restrict__ Ag = static_cast<const uint16_t*>(p.A);
  const uint16_t* __restrict__ Bg = static_cast<const uint16_t*>(p.B);

  Loader<AK, BM, NT, false, WN> la;
  Loader<BKM, BN, NT, SWIG, WN> lb;

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (p.K + BK - 1) / BK;
  la.load(Ag, p.lda, tile_m, p.M, 0, 0, p.K, tid);
  lb.load(Bg, p.ldb, tile_n, p.N, p.fhalf, 0, p.K, tid);
  la.store(&lds[0][0], tid);
  lb.store(&lds[0][BM * 8], tid);
  __syncthreads();

  const int arow0 = wm * WM + (lane & 15);
  const int brow0 = wn * WN + (lane & 15);
  const int kq = lane >> 4;

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = (kt + 1) < nk;
    if (more) {
      la.load(Ag, p.lda, tile_m, p.M, 0, (kt + 1) * BK, p.K, tid);
      lb.load(Bg, p.ldb, tile_n, p.N, p.fhalf, (kt + 1) * BK, p.K, tid);
    }
    const uint4* As = &lds[cur][0];
    const uint4* Bs = &lds[cur][BM * 8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + kq;
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = arow0 + i * 16;
        af[i] = __builtin_bit_cast(bf16x8_t, As[r * 8 + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = brow0 + j * 16;
        bfr[j] = __builtin_bit_cast(bf16x8_t, Bs[r * 8 + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.store(&lds[cur ^ 1][0], tid);
      lb.store(&lds[cur ^ 1][BM * 8], tid);
    }
    __syncthreads();
  }

  // ---- epilogue.  Lane holds rows (lane>>4)*4 + e, column lane&15 of each 16x16 subtile.
  const int mbase = tile_m * BM + wm * WM + (lane >> 4) * 4;
  if constexpr (SWIG) {
    constexpr int HT = TN / 2;
    const int jbase = tile_n * (BN / 2) + wn * (WN / 2) + (lane & 15);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < HT; ++j) {
        const int col = jbase + j * 16;
        if (col >= p.fhalf) continue;
        const float bg = p.bias ? bf16_to_f32(ldg_bf16(p.bias, col)) : 0.f;
        const float bu = p.bias ? bf16_to_f32(ldg_bf16(p.bias, p.fhalf + col)) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mbase + i * 16 + e;
          if (m >= p.M) continue;
          const float g = acc[i][j][e] + bg;
          const float u = acc[i][j + HT][e] + bu;
          stg_bf16(p.C, (int64_t)m * p.ldc + col, g);
          stg_bf16(p.C, (int64_t)m * p.ldc + p.fhalf + col, u);
          stg_bf16(p.C2, (int64_t)m * p.ldc2 + col, g * act_sigmoid(g) * u);
        }
      }
  } else {
    const int nbase = tile_n * BN + wn * WN + (lane & 15);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = nbase + j * 16;
      if (col >= p.N) continue;
      float bcol = 0.f;
      if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_ACT) bcol = p.bias ? bf16_to_f32(ldg_bf16(p.bias, col)) : 0.f;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mbase + i * 16 + e;
          if (m >= p.M) continue;
          const float v = acc[i][j][e];
          if constexpr (EPI == EPI_STORE) {
            stg_bf16(p.C, (int64_t)m * p.ldc + col, v);
          } else if constexpr (EPI == EPI_BIAS) {
            stg_bf16(p.C, (int64_t)m * p.ldc + col, v + bcol);
          } else if constexpr (EPI == EPI_BIAS_ACT) {
            const float u = v + bcol;
            stg_bf16(p.C, (int64_t)m * p.ldc + col, u);
            stg_bf16(p.C2, (int64_t)m * p.ldc2 + col, act_apply(p.act, u));
          } else if constexpr (EPI == EPI_ACT_BWD) {
            const float u = bf16_to_f32(ldg_bf16(p.aux, (int64_t)m * p.ldaux + col));
            stg_bf16(p.C, (int64_t)m * p.ldc + col, v * act_grad(p.act, u));
          } else if constexpr (EPI == EPI_SWIGLU_BWD) {
            const float g = bf16_to_f32(ldg_bf16(p.aux, (int64_t)m * p.ldaux + col));
            const float u = bf16_to_f32(ldg_bf16(p.aux, (int64_t)m * p.ldaux + p.fhalf + col));
            const float sg = act_sigmoid(g);
            stg_bf16(p.C, (int64_t)m * p.ldc + col, v * u * sg * (1.f + g * (1.f - sg)));
            stg_bf16(p.C, (int64_t)m * p.ldc + p.fhalf + col, v * g * sg);
          }
        }
    }
  }
}

// ------------------------------------------------------------------------------------------------------------------
// Tile configurations and dispatch.
// ------------------------------------------------------------------------------------------------------------------
struct Cfg {
  int bm, bn, nwm, nwn;
  float eff;  // relative per-tile efficiency used to trade tile size against filling 256 CUs
};
constexpr Cfg kCfgs[] = {
    {256, 256, 2, 4, 1.00f},
    {256, 128, 2, 2, 0.92f},
    {128, 128, 2, 2, 0.78f},
    {64, 64, 2, 2, 0.40f},
};
constexpr int kNumCUs = 256;
const char* const kEpiNames[] = {"store", "bias", "bias_act", "swiglu_fwd", "act_bwd", "swiglu_bwd"};

int choose_cfg(int M, int ntiles_cols_of_bn256, int N, bool swig, int fhalf) {
  (void)ntiles_cols_of_bn256;
  int best = 0;
  float best_score = -1.f;
  for (int i = 0; i < (int)(sizeof(kCfgs) / sizeof(kCfgs[0])); ++i) {
    const Cfg& c = kCfgs[i];
    const long nbm = (M + c.bm - 1) / c.bm;
    const long nbn = swig ? (fhalf + c.bn / 2 - 1) / (c.bn / 2) : (N + c.bn - 1) / c.bn;
    const long tiles = nbm * nbn;
    const long waves = (tiles + kNumCUs - 1) / kNumCUs;
    // useful fraction of the computed tile area (ragged edges) times the fill of the last wave
    const double rows_used = (double)M / (double)(nbm * c.bm);
    const double cols_used = swig ? (double)fhalf / (double)(nbn * c.bn / 2) : (double)N / (double)(nbn * c.bn);
    const double fill = (double)tiles / (double)(waves * kNumCUs);
    const float score = (float)(fill * rows_used * cols_used * c.eff);
    if (score > best_score + 1e-6f) {
      best_score = score;
      best = i;
    }
  }
  return best;
}

template <int BM, int BN, int NWM, int NWN, bool AK, bool BKM, int EPI>
hipError_t launch_one(const GemmParams& p, hipStream_t st) {
  const int nbm = (p.M + BM - 1) / BM;
  const int nbn = (EPI == EPI_SWIGLU_FWD) ? (p.fhalf + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  static const std::string name = "gemm_bf16_" + std::to_string(BM) + "x" + std::to_string(BN) + "_" +
                                  (AK ? "K" : "M") + (BKM ? "K" : "M") + "_" + kEpiNames[EPI];
  return TP_LAUNCH(name.c_str(), (gemm_bf16_kernel<BM, BN, NWM, NWN, AK, BKM, EPI>), dim3((unsigned)(nbm * nbn)),
                   dim3(NWM * NWN * 64), 0, st, p);
}

template <bool AK, bool BKM, int EPI>
hipError_t launch_cfg(int ci, const GemmParams& p, hipStream_t st) {
  switch (ci) {
    case 0: return launch_one<256, 256, 2, 4, AK, BKM, EPI>(p, st);
    case 1: return launch_one<256, 128, 2, 2, AK, BKM, EPI>(p, st);
    case 2: return launch_one<128, 128, 2, 2, AK, BKM, EPI>(p, st);
    default: return launch_one<64, 64, 2, 2, AK, BKM, EPI>(p, st);
  }
}

}  // namespace

// Only the (layout, epilogue) pairs the block uses are instantiated.
hipError_t gemm_bf16(const GemmParams& p, bool a_kmajor, bool b_kmajor, int epi, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const bool swig = epi == EPI_SWIGLU_FWD;
  const int ci = choose_cfg(p.M, 0, p.N, swig, p.fhalf);
  if (a_kmajor && !b_kmajor) {  // X W: forward GEMMs
    switch (epi) {
      case EPI_STORE: return launch_cfg<true, false, EPI_STORE>(ci, p, st);
      case EPI_BIAS: return launch_cfg<true, false, EPI_BIAS>(ci, p, st);
      case EPI_BIAS_ACT: return launch_cfg<true, false, EPI_BIAS_ACT>(ci, p, st);
      case EPI_SWIGLU_FWD: return launch_cfg<true, false, EPI_SWIGLU_FWD>(ci, p, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (a_kmajor && b_kmajor) {  // x W^T: dgrad GEMMs
    switch (epi) {
      case EPI_STORE: return launch_cfg<true, true, EPI_STORE>(ci, p, st);
      case EPI_ACT_BWD: return launch_cfg<true, true, EPI_ACT_BWD>(ci, p, st);
      case EPI_SWIGLU_BWD: return launch_cfg<true, true, EPI_SWIGLU_BWD>(ci, p, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (!a_kmajor && !b_kmajor && epi == EPI_STORE) return launch_cfg<false, false, EPI_STORE>(ci, p, st);  // wgrad
  return hipErrorInvalidValue;
}

}  // namespace tp
