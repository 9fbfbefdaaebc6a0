// bf16 GEMMs on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation) for every GEMM of the
// column->row block: the column GEMM X A_i with its fused bias + GeLU / SwiGLU epilogue, the row GEMM Y_i B_i,
// the dgrad GEMMs dZ B_i^T (fused with act') and dU_i A_i^T, and the wgrad GEMMs Y_i^T dZ and X^T dU_i
// ("Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" §2; the backward section of the 111qqz
// "tensor-parallelism-matrix-split" post).
//
// Two kernels.  The large-tile kernel (gemm_bf16_big_kernel: 256 x 256 tiles, 4 waves of 128 x 128 or 8 of 64 x 128,
// a 4-stage LDS ring fed by direct global -> LDS copies, transposing LDS reads for MN-major operands) runs
// every GEMM whose K is a multiple of 64 and whose tile count fills the GPU; its design is described above it.
// The register-staged kernel (gemm_bf16_kernel) takes the rest:
//   * one workgroup = one BM x BN output tile, NWM x NWN waves of 64 lanes, K stepped by 64;
//   * operand tiles are staged through LDS as [row][k] with 64 k per row (8 chunks of 16 bytes).  A K-major
//     operand is copied chunk for chunk; an MN-major operand is read as 8(k) x 4(mn) blocks and transposed in
//     registers before the LDS store, so every MFMA fragment is one 16-byte LDS read;
//   * chunk c of row r is stored at chunk c ^ ((r ^ (r >> 2)) & 7): eight consecutive rows read at one logical
//     chunk hit eight distinct 16-byte bank groups, and so do the transposed stores of eight consecutive blocks;
//   * two LDS stages; the next K tile's global loads are issued into registers before the current tile's MFMAs
//     and written to the other stage after them, with one barrier per K tile.
// Both order tiles XCD-aware: the hardware deals workgroup i to XCD i % 8, so the launch index is remapped to give
// each XCD a contiguous run of tiles, walked in groups of a few row tiles so the A rows and B columns an XCD
// touches stay in its own L2.
#include <string>
#include <type_traits>

#include "tp_common.h"

#include <atomic>

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
// Large-tile kernel: 256 x 256 output tile, 8 waves (4 x 2) of 64 x 128 = 4 x 8 MFMA subtiles, 128 fp32
// accumulators per lane (two waves per SIMD, 256 registers each), so one wave's waits and epilogue run beside the
// other's MFMAs.  Needs K % 64 == 0 (whole pairs of 32-deep k-tiles).  Out-of-range rows of either operand are
// clamped to the last valid row: they only feed output rows or columns that are never stored, so no load needs a
// bounds branch.
//
// Each operand is kept in LDS in the orientation it has in HBM, a pair of k-tiles (64 k) per buffer:
//   * K-major ([rows][k]): 256 rows x 128 bytes; 16-byte chunk c of row r sits at chunk c ^ (r & 7).  An MFMA
//     fragment (16 rows x 8 consecutive k per lane) is one 16-byte read.
//   * MN-major ([k][cols]): 64 k rows x 512 bytes; chunk c of row k sits at chunk c ^ swz_mn(k).  A fragment is
//     built by two transposing reads (ds_read_b64_tr_b16): in each 16-lane group, lane k' points at row k0 + k'/4,
//     columns n0 + 4 (k' % 4) .. +3, and lane i receives column n0 + i of rows k0 .. k0 + 3.
// Both permutations make the lanes served together touch distinct banks.
//
// Pipeline: step j computes k-tile j from registers while reading k-tile j+1's fragments; odd steps wait for the
// copies of the pair k-tile j+1 opens, barrier, and copy the pair after it into the buffer just freed.
// Two GEMMs of the same layout can share one launch (the two weight gradients): workgroups [0, tiles0) take the
// first, the rest the second.
// ------------------------------------------------------------------------------------------------------------------
// Transposed 16x16 blocks: the B fragment goes first, so the accumulator holds (A B)^T block by block.
template <int T0, int T1, int TN, int TM>
__device__ __forceinline__ void mfma_rows_t(f32x4_t (&acc)[TM][TN], const bf16x8_t (&af)[TM],
                                            const bf16x8_t (&bfr)[TN]) {
#pragma unroll
  for (int i = T0; i < T1; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
}

struct GemmPair {
  GemmParams g[2];
  int tiles0, tiles1;
  // Split-K launches: the first nfull workgroups take whole tiles 0 .. nfull-1; each later run of ksplit workgroups
  // takes one of the remaining tiles, one K range each, and writes an fp32 partial tile to part: [ksplit][M][N]
  // (A K-major: a single GEMM with every tile split), or 256 x 256 blocks [tile - nfull][ksplit] (A M-major: the
  // tail tiles of a weight-gradient pair).
  int ksplit, nfull;
  float* part;
};

// XCD-aware order over nb workgroups: the hardware deals workgroup i to XCD i % 8; the result gives each XCD a
// contiguous run of indices (a bijection on 0 .. nb-1).
__device__ __forceinline__ int xcd_remap(int u, int nb) {
  const int q = nb / 8, r = nb % 8;
  const int xcd = u % 8, idx = u / 8;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int BK2 = 32;  // k-tile depth of the large-tile kernel

__device__ __forceinline__ int swz_mn(int k) { return (2 * (k & 3)) ^ (8 * ((k >> 3) & 1)); }  // MN-major tiles

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Direct global -> LDS copy of 16 bytes per lane from a wave-uniform base held in scalar registers plus a per-lane
// 32-bit byte offset: lane l's bytes land at LDS byte address m0 + 16 l, and the address arithmetic stays on the
// scalar unit.  Issued as inline assembly so that the compiler does not wait for these copies at every barrier; the
// kernel waits for them itself (s_waitcnt vmcnt) before the barrier that publishes a buffer.  (A vector instruction
// next to a matrix instruction runs in the matrix instruction's shadow only two or so at a time; longer runs of them
// hold the matrix core idle.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Pair buffers of the 8-wave kernel: an operand's pair of k-tiles is 32 KB (256 rows of 64 k, or 64 k rows of
// 256), buffer b at 32 KB * b (A) and 64 KB + 32 KB * b (B).  K-major rows are 128 bytes; chunk c of row r sits at
// c ^ (r & 7).  A 16-byte read is served 8 lanes (128 bytes) at a time, and with 128-byte rows those 8 lanes' rows
// all start on the same bank, so their 8 chunks must differ (the counter showed 2-way conflicts with a 2-bit
// permutation).  A copy is 8 rows.
constexpr int kPairOp = 32768;  // bytes of one operand's pair buffer
constexpr int kLdsB = 65536;    // the B buffers start 64 KB in

template <bool KMAJ, bool SWIG, int CPP, int TW = 256>
struct DmaP;

// (TW: the operand's rows per tile -- 256, or 192 for the narrower column tiles; an MN-major copy still moves 256
// columns, the ones past the tile clamped inside the matrix and never read)
template <bool SWIG, int CPP, int TW>
struct DmaP<true, SWIG, CPP, TW> {  // K-major: copy i holds rows 8 i .. 8 i + 7, 128 bytes each
  uint32_t voff[CPP];
  __device__ __forceinline__ void init(int64_t ld, int tile, int rows, int fhalf, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < CPP; ++q) {
      const int r = 8 * (CPP * wave + q) + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);  // the logical chunk this slot holds
      const int row = min(tile * TW + r, rows - 1);
      voff[q] = (uint32_t)(((int64_t)row * ld + c * 8) * 2);
    }
  }
  static __device__ __forceinline__ int64_t pstride(int64_t ld) { return 4 * BK2; }  // bytes per pair along a row
};

template <bool SWIG, int CPP, int TW>
struct DmaP<false, SWIG, CPP, TW> {  // MN-major: copy i holds k rows 2 i, 2 i + 1 (512 bytes each)
  uint32_t voff[CPP];
  __device__ __forceinline__ void init(int64_t ld, int tile, int rows, int fhalf, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < CPP; ++q) {
      const int k = 2 * (CPP * wave + q) + (lane >> 5);
      const int cl = 8 * ((lane & 31) ^ swz_mn(k));
      int col;
      if (SWIG) {
        const int wn = cl / 128, cw = cl % 128;
        const int half = cw / 64, jj = min(tile * 128 + wn * 64 + (cw % 64), fhalf - 8);
        col = half * fhalf + jj;
      } else {
        col = min(tile * TW + cl, rows - 8);
      }
      voff[q] = (uint32_t)((col + (int64_t)k * ld) * 2);
    }
  }
  static __device__ __forceinline__ int64_t pstride(int64_t ld) { return 4 * BK2 * ld; }  // 64 k rows
};

// Fragment addresses in buffer 0 (K-major: one per half of the pair); read<B, H> takes buffer B, half H (k-tile
// 2m + H of the pair) through immediate offsets.  K-major: fragment i one 16-byte read; MN-major: two transposing
// 8-byte reads 2048 apart.
template <bool KMAJ, int NFR, int OPB>
struct FragP {
  uint32_t a[KMAJ ? 2 : NFR];
  __device__ __forceinline__ void init(int rbase, int lane) {
    if constexpr (KMAJ) {
      const int r = rbase + (lane & 15);
#pragma unroll
      for (int h = 0; h < 2; ++h) a[h] = OPB + r * 128 + (((4 * h + (lane >> 4)) ^ (r & 7)) << 4);
    } else {
      const int g = lane >> 4, kq = lane & 15;
      const int k1 = 8 * g + (kq >> 2);
      const int cq = 4 * (kq & 3);
#pragma unroll
      for (int i = 0; i < NFR; ++i) {
        const int col = rbase + i * 16 + cq;
        const int ch = col >> 3, hf = (col >> 2) & 1;
        a[i] = OPB + k1 * 512 + ((ch ^ swz_mn(k1)) << 4) + (hf << 3);
      }
    }
  }
  template <int B, int H>
  __device__ __forceinline__ void read(const char* ldsc, int i, bf16x8_t& f) const {
    if constexpr (KMAJ) {
      f = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(ldsc + a[H] + (B * kPairOp + i * 2048)));
    } else {
      const char* b = ldsc + a[i] + (B * kPairOp + H * 16384);
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(b));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(b + 2048));
      typedef short v8i16_t __attribute__((ext_vector_type(8)));
      const v8i16_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      f = __builtin_bit_cast(bf16x8_t, w);
    }
  }
};

// Fragment reads of one k-tile, spread over the first 3/4 of a step's TM MFMA segments: fragments are taken in
// the order A0 B0 A1 B1 ... (then the B fragments past TM) and fragment f goes to segment f (3 TM / 4) / (TM + TN).
template <int TM, int TN>
constexpr int frag_seg(int f) { return f * (3 * TM / 4) / (TM + TN); }
template <int TM>
constexpr bool frag_is_a(int f) { return f < 2 * TM && f % 2 == 0; }
template <int TM>
constexpr int frag_idx(int f) { return f < 2 * TM ? f / 2 : f - TM; }
template <bool AK, bool BKM, int TM, int TN>
constexpr int seg_ds_count(int s) {
  int n = 0;
  for (int f = 0; f < TM + TN; ++f)
    if (frag_seg<TM, TN>(f) == s) n += frag_is_a<TM>(f) ? (AK ? 1 : 2) : (BKM ? 1 : 2);
  return n;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return pack_bf16x2_hw(lo, hi); }
__device__ __forceinline__ void stg_bf16x2(void* p, int64_t i, float lo, float hi) {
  *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + i) = pack_bf16x2(lo, hi);
}
__device__ __forceinline__ float2 ldg_bf16x2(const void* p, int64_t i) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
  return make_float2(bf16_to_f32(w & 0xFFFFu), bf16_to_f32(w >> 16));
}

// One wave's 16 x 128 chunk of fp32 results in LDS (pitch ep_pitch) -> fp32 partial block of 256 x 256 (blk; the
// tile's first row is m_tile).  Lane l owns columns 2l, 2l+1 of each row.
__device__ __forceinline__ void partial_chunk(const GemmParams& p, const float* ep, int ep_pitch, int m0, int m_tile,
                                              int tile_n, int wn, int lane, float* blk) {
  const int col = tile_n * 256 + wn * 128 + 2 * lane;
  if (col >= p.N) return;  // N % 8 == 0: a column pair is entirely in or out
  const int rows = min(16, p.M - m0);
  float* dst = blk + (int64_t)(m0 - m_tile) * 256 + wn * 128 + 2 * lane;
  for (int r = 0; r < rows; ++r)
    *reinterpret_cast<float2*>(dst + r * 256) = make_float2(ep[r * ep_pitch + 2 * lane], ep[r * ep_pitch + 2 * lane + 1]);
}

// One wave's 16 x 128 chunk of fp32 results in LDS (pitch ep_pitch) -> epilogue -> HBM.  Plain epilogues: lane l
// owns columns 2l, 2l+1 of each row.  SwiGLU forward: the wave's 128 columns are 64 gate then 64 up columns of the
// same 64 outputs j; lane l owns output j = l.
__device__ __forceinline__ float2 lds_bf16x2(const uint16_t* ax, int i) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(ax + i);
  return make_float2(bf16_to_f32(w & 0xFFFFu), bf16_to_f32(w >> 16));
}

// Eight fp32 values -> bf16, one 16-byte store (the column is a multiple of 8 and rows are 16-byte aligned).
__device__ __forceinline__ void stg_bf16x8(void* p, int64_t i, const float (&v)[8]) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) = w;
}
// Eight bf16 values of the staged auxiliary input (16-byte LDS read).
__device__ __forceinline__ void lds_bf16x8(const uint16_t* ax, int i, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(ax + i);
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = bf16_to_f32(q[k] & 0xFFFFu);
    v[2 * k + 1] = bf16_to_f32(q[k] >> 16);
  }
}

// The plain epilogues' rows of one chunk: lane l owns the 8 columns col .. col + 7 (cl .. cl + 7 of the wave's) of
// rows rr, rr + 4, rr + 8, rr + 12 (rr = l / 16), so a chunk row leaves as 16-byte stores of 16 lanes.  The
// activation is a template argument, picked once per chunk: with the choice made per element, each of the kernel's
// 8 unrolled chunks carried the code of every activation, and since a tile runs its epilogue once, that code ran
// mostly from instruction-cache misses (the GeLU epilogues took 25-30 us longer per launch at h=4096, ffn/t=2048).
// The row loop stays rolled for the same reason.
template <int EPI, int ACT>
__device__ __forceinline__ void chunk_rows(const GemmParams& p, const float* ep, int ep_pitch, int m0, int col, int cl,
                                           int rr, const uint16_t* ax, const float (&b)[8], const float (&c)[8],
                                           int rows) {
#pragma unroll 1
  for (int r = rr; r < rows; r += 4) {
    float v[8];
    {
      const float4 x0 = *reinterpret_cast<const float4*>(ep + r * ep_pitch + cl);
      const float4 x1 = *reinterpret_cast<const float4*>(ep + r * ep_pitch + cl + 4);
      v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
      v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
    }
    const int64_t m = m0 + r;
    if constexpr (EPI == EPI_LN_ACT) {
      // LayerNorm(u) W + bias = rstd (u W' - mean c) + b, with W' = diag(gamma) W and c its column sums
      const float mu = p.ln_mean[m], rs = p.ln_rstd[m];
      float u[8], y[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        u[k] = fmaf(rs, fmaf(-mu, c[k], v[k]), b[k]);
        y[k] = act_apply(ACT, u[k]);
      }
      stg_bf16x8(p.C, m * p.ldc + col, u);
      stg_bf16x8(p.C2, m * p.ldc2 + col, y);
    } else if constexpr (EPI == EPI_STORE) {
      stg_bf16x8(p.C, m * p.ldc + col, v);
    } else if constexpr (EPI == EPI_BIAS) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += b[k];
      stg_bf16x8(p.C, m * p.ldc + col, v);
    } else if constexpr (EPI == EPI_BIAS_ACT) {
      float y[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[k] += b[k];
        y[k] = act_apply(ACT, v[k]);
      }
      stg_bf16x8(p.C, m * p.ldc + col, v);
      stg_bf16x8(p.C2, m * p.ldc2 + col, y);
    } else if constexpr (EPI == EPI_ACT_BWD) {
      float u[8];
      lds_bf16x8(ax, r * 128 + cl, u);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] *= act_grad(ACT, u[k]);
      stg_bf16x8(p.C, m * p.ldc + col, v);
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
      float g[8], u[8], dg[8], du[8];
      lds_bf16x8(ax, r * 128 + cl, g);
      lds_bf16x8(ax, 2048 + r * 128 + cl, u);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float s = act_sigmoid(g[k]);
        dg[k] = v[k] * u[k] * s * (1.f + g[k] * (1.f - s));
        du[k] = v[k] * g[k] * s;
      }
      stg_bf16x8(p.C, m * p.ldc + col, dg);
      stg_bf16x8(p.C, m * p.ldc + p.fhalf + col, du);
    }
  }
}

// ax: this wave's 16 x 128 tile of the epilogue's auxiliary input (U for act', [gate | up] at +2048 for SwiGLU),
// staged in LDS.
template <int EPI, int WN = 128>
__device__ __forceinline__ void epilogue_chunk(const GemmParams& p, const float* ep, int ep_pitch, int m0, int tile_n,
                                               int wn, int lane, const uint16_t* ax) {
  if constexpr (epi_swiglu_fwd(EPI)) {
    const int j = tile_n * 128 + wn * 64 + lane;
    if (j >= p.fhalf) return;
    float bg, bu, cg = 0.f, cu = 0.f;
    if constexpr (epi_ln(EPI)) {
      bg = p.ln_b[j];
      bu = p.ln_b[p.fhalf + j];
      cg = p.ln_c[j];
      cu = p.ln_c[p.fhalf + j];
    } else {
      bg = p.bias ? bf16_to_f32(ldg_bf16(p.bias, j)) : 0.f;
      bu = p.bias ? bf16_to_f32(ldg_bf16(p.bias, p.fhalf + j)) : 0.f;
    }
    const int rows = min(16, p.M - m0);
    for (int r = 0; r < rows; ++r) {
      float g, u;
      if constexpr (epi_ln(EPI)) {
        const float mu = p.ln_mean[m0 + r], rs = p.ln_rstd[m0 + r];
        g = fmaf(rs, fmaf(-mu, cg, ep[r * ep_pitch + lane]), bg);
        u = fmaf(rs, fmaf(-mu, cu, ep[r * ep_pitch + 64 + lane]), bu);
      } else {
        g = ep[r * ep_pitch + lane] + bg;
        u = ep[r * ep_pitch + 64 + lane] + bu;
      }
      const int64_t m = m0 + r;
      stg_bf16(p.C, m * p.ldc + j, g);
      stg_bf16(p.C, m * p.ldc + p.fhalf + j, u);
      stg_bf16(p.C2, m * p.ldc2 + j, g * act_sigmoid(g) * u);
    }
  } else {
    const int cl = 8 * (lane & 15), rr = lane >> 4;
    if (cl >= WN) return;  // a 96-column wave: lanes with cl >= 96 have no columns
    const int col = tile_n * 2 * WN + wn * WN + cl;
    if (col >= p.N) return;  // N % 8 == 0: a group of 8 columns is entirely in or out
    float b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, c[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_ACT) {
      if (p.bias) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.bias) + col);
        const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          b[2 * k] = bf16_to_f32(q[k] & 0xFFFFu);
          b[2 * k + 1] = bf16_to_f32(q[k] >> 16);
        }
      }
    }
    if constexpr (EPI == EPI_LN_ACT) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        b[k] = p.ln_b[col + k];
        c[k] = p.ln_c[col + k];
      }
    }
    const int rows = min(16, p.M - m0);
    if constexpr (EPI == EPI_BIAS_ACT || EPI == EPI_ACT_BWD || EPI == EPI_LN_ACT) {  // the activation chosen once per chunk
      switch (p.act) {
        case TP_ACT_GELU: chunk_rows<EPI, TP_ACT_GELU>(p, ep, ep_pitch, m0, col, cl, rr, ax, b, c, rows); break;
        case TP_ACT_GELU_TANH:
          chunk_rows<EPI, TP_ACT_GELU_TANH>(p, ep, ep_pitch, m0, col, cl, rr, ax, b, c, rows);
          break;
        default: chunk_rows<EPI, TP_ACT_RELU>(p, ep, ep_pitch, m0, col, cl, rr, ax, b, c, rows); break;
      }
    } else {
      chunk_rows<EPI, TP_ACT_RELU>(p, ep, ep_pitch, m0, col, cl, rr, ax, b, c, rows);
    }
  }
}

// Row tiles per group of the large-tile kernel's walk over its tiles (each XCD walks its tiles a group of row tiles
// at a time, column by column): 8 for a two-GEMM (pair) launch, the act' epilogues and the activation epilogues of
// the column GEMM, 2 for the plain K-major A x MN-major B store (the row GEMM), 4 otherwise -- measured best for
// each at h = 4096, ffn/t = 2048 (column GEMM + GeLU 247 -> 240 us with 8 against 4).  The split-K tail sum decodes
// tiles with the same rule.
__host__ __device__ constexpr int big_row_group(bool pair, int epi, bool ak, bool bkm) {
  return pair ? 8
              : (epi == EPI_ACT_BWD || epi == EPI_SWIGLU_BWD) ? 8
              : (ak && !bkm) ? (epi == EPI_STORE ? 2 : epi == EPI_BIAS ? 4 : 8)
                             : 4;
}

// Large-tile kernel: one 256 x 256 output tile per workgroup, 8 waves of 64 x 128 (two per SIMD), K in pairs of
// 32-deep k-tiles through two LDS pair buffers fed by direct global -> LDS copies two steps ahead of their use.  The
// MFMAs take the B fragment first, so each 16 x 16 accumulator block is the transposed product: lane l holds row
// 16 i + (l & 15), columns 16 j + 4 (l >> 4) .. + 3 of the wave's sub-tile, which the epilogue stages through LDS
// with one 16-byte write per block.  (A persistent launch, one workgroup per CU walking its tiles so that a tile's
// stores drain under the next tile's first copies, measured no faster than one workgroup per tile.)
template <bool AK, bool BKM, int EPI, bool SPLIT = false, int NW = 8, int BNT = 256>
__global__ __launch_bounds__(NW * 64, 1) void gemm_bf16_big_kernel(GemmPair pp) {
  static_assert(NW == 8, "the pair-buffer loop is written for 8 waves of 64 x 128");
  // BNT: 256 columns per tile (waves of 64 x 128), or 192 (waves of 64 x 96) where 256-column tiles would leave
  // most of a round of CUs idle; not for the SwiGLU forward's interleaved halves or the pair's split tail blocks
  static_assert(BNT == 256 || (BNT == 192 && !epi_swiglu_fwd(EPI) && !(SPLIT && !AK)), "192-column tiles");
  constexpr int BM = 256, BN = BNT, WM = 512 / NW, WN = BN / 2, TM = WM / 16, TN = WN / 16;
  constexpr int RING_B = 2 * 2 * kPairOp;  // two pair buffers of A and B
  constexpr bool SWIG = epi_swiglu_fwd(EPI);
  constexpr int EP = 132;  // epilogue fp32 row pitch: 16-byte writes of 16 consecutive rows hit distinct banks
  constexpr int NAUX = EPI == EPI_SWIGLU_BWD ? 8 : EPI == EPI_ACT_BWD ? 4 : 0;  // 16-byte aux loads per lane
  constexpr int EPW = 16 * EP * 4 + NAUX * 1024;                                  // epilogue bytes per wave
  constexpr int LDS_U4 = (RING_B > NW * EPW ? RING_B : NW * EPW) / 16;
  __shared__ u32x4_t lds[LDS_U4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- problem and tile: XCD-aware remap over the whole launch (the hardware deals workgroup i to XCD i % 8;
  // each XCD gets a contiguous run of tiles), then split between the two problems of a pair
  int bid = blockIdx.x;
  int split = -1;  // -1: the whole K range
  if constexpr (SPLIT) {
    if (bid >= pp.nfull) {  // nfull is a multiple of 8, so each range starts on XCD 0
      const int v = xcd_remap(bid - pp.nfull, (int)gridDim.x - pp.nfull);
      split = v % pp.ksplit;
      bid = pp.nfull + v / pp.ksplit;
    } else {
      bid = xcd_remap(bid, pp.nfull);
    }
  } else {
    bid = xcd_remap(bid, (int)gridDim.x);
  }
  const int tile_id = bid;
  const int which = bid < pp.tiles0 ? 0 : 1;
  const GemmParams& p = pp.g[which];
  if (which) bid -= pp.tiles0;
  const int nbm = (p.M + BM - 1) / BM;
  const int nbn = SWIG ? (p.fhalf + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  // (the split K-major x K-major kernel on 192-column tiles, the attention backward's dO GEMM, walks groups of 2:
  // 54 -> 49 us per rank at the 22B shape against 4)
  const int gm = (SPLIT && BNT == 192 && AK && BKM) ? 2 : big_row_group(pp.tiles1 > 0, EPI, AK, BKM);
  const int group = bid / (gm * nbn);
  const int first_m = group * gm;
  const int gsz = min(nbm - first_m, gm);
  const int tile_m = first_m + (bid % (gm * nbn)) % gsz;
  const int tile_n = (bid % (gm * nbn)) / gsz;

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Pair buffers: k-tiles 2m and 2m+1 (64 k) of each operand sit in buffer m % 2, so a K-major row's 64 k (128
  // bytes, a whole cache line) comes in one piece; copying one k-tile (64 bytes of each line) reads every line
  // twice at half the rate of whole lines from L2.  Layout: A buffers at 0 and 32 KB, B buffers at 64 and 96 KB.
  constexpr int CPP = 32 / NW;  // copies per wave per operand and pair (A; and B at 256 columns)
  constexpr int CPPB = BKM ? BN / 64 : CPP;  // B's: a K-major copy is 8 rows; an MN-major one 2 k rows of 256
  constexpr int NCPY = CPP + CPPB;
  DmaP<AK, false, CPP> da;
  DmaP<BKM, SWIG, CPPB, BN> db;
  da.init(p.lda, tile_m, p.M, p.fhalf, wave, lane);
  db.init(p.ldb, tile_n, p.N, p.fhalf, wave, lane);
  int kp0 = 0, kp1 = p.K / (2 * BK2);  // pairs of k-tiles: all of K, or split `split` of pp.ksplit runs
  if (SPLIT && split >= 0) {
    const int np = kp1, base = np / pp.ksplit, rem = np % pp.ksplit;
    kp0 = split * base + min(split, rem);
    kp1 = kp0 + base + (split < rem ? 1 : 0);
  }
  const int64_t astr = DmaP<AK, false, CPP>::pstride(p.lda), bstr = DmaP<BKM, SWIG, CPPB, BN>::pstride(p.ldb);
  const char* const Ab = static_cast<const char*>(p.A) + kp0 * astr;  // uniform: pair 0 of the range
  const char* const Bb = static_cast<const char*>(p.B) + kp0 * bstr;
  const int npair = kp1 - kp0, nk = 2 * npair;
  const uint32_t lds0 = (uint32_t)(uintptr_t)&lds[0];
  const char* const ldsc = reinterpret_cast<const char*>(&lds[0]);
  FragP<AK, TM, 0> fra;
  FragP<BKM, TN, kLdsB> frb;
  fra.init(wm * WM, lane);
  frb.init(wn * WN, lane);
  // copy q of this wave's share of pair pr into buffer BUF (A copies q < CPP, B copies after)
  auto copy = [&](auto bufc, int q, int pr) {
    constexpr int BUF = decltype(bufc)::value;
    if (q < CPP)
      dma16s(Ab + pr * astr, da.voff[q], lds0 + BUF * kPairOp + (CPP * wave + q) * 1024);
    else
      dma16s(Bb + pr * bstr, db.voff[q - CPP], lds0 + kLdsB + BUF * kPairOp + (CPPB * wave + q - CPP) * 1024);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // prologue: pairs 0 and 1 into buffers 0 and 1; pair 0 landed (pair 1's copies may be in flight)
#pragma unroll
  for (int q = 0; q < NCPY; ++q) copy(I0{}, q, 0);
  if (npair > 1) {
#pragma unroll
    for (int q = 0; q < NCPY; ++q) copy(I1{}, q, 1);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NCPY) : "memory");
  } else {
    wait_vmcnt0();
  }
  __syncthreads();
  bf16x8_t fa[TM], fb[TN], ga[TM], gb[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) fra.template read<0, 0>(ldsc, i, fa[i]);
#pragma unroll
  for (int i = 0; i < TN; ++i) frb.template read<0, 0>(ldsc, i, fb[i]);

  // Step j (U = j % 4; k-tile j's fragments in FC): read k-tile j+1's fragments into FN, run k-tile j's MFMAs.
  // An odd step first waits for its own copies of pair (j+1)/2, the pair k-tile j+1 opens (issued two steps
  // earlier; nothing was issued since), and barriers, which publishes that pair and proves every wave done with
  // the buffer of pair (j-1)/2 (its last fragments were read in step j-1); then it copies pair (j+3)/2 into that
  // buffer (past the last pair: the last pair again, into a free buffer or over its own identical bytes, so the
  // step has no branch).  Even steps neither wait nor barrier: k-tile j+1 is in the pair of k-tile j.
  // TM segments: segment G holds its share of the copies, its share of the reads and the 8 MFMAs of fragment row
  // G, the copies and reads slotted between the MFMAs (a wave waits at each MFMA issue, so anything placed there
  // runs while the matrix core is busy).
  auto step = [&](auto uc, int j, bf16x8_t(&FCA)[TM], bf16x8_t(&FCB)[TN], bf16x8_t(&FNA)[TM], bf16x8_t(&FNB)[TN]) {
    constexpr int U = decltype(uc)::value;
    constexpr bool ODD = U & 1;
    constexpr int RB = ((U + 1) >> 1) & 1, RH = (U + 1) & 1;  // buffer and half of k-tile j+1
    constexpr int CB = ((U + 3) >> 1) & 1;                      // buffer of pair (j+3)/2
    using IC = std::integral_constant<int, CB>;
    const int pc = min((j + 3) >> 1, npair - 1);
    if constexpr (ODD) {
      // the wave waits at raised priority, so that once its copies land it passes the barrier and issues the next
      // pair's first copies ahead of the other wave's MFMA stream (priority back to normal after segment 0):
      // headline GEMMs 1-2% faster, side by side
      __builtin_amdgcn_s_setprio(2);
      wait_vmcnt0();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
    auto segment = [&](auto segc) {
      constexpr int G = decltype(segc)::value;
      if constexpr (ODD) {  // this step copies the pair's A and B shares, spread over the segments
#pragma unroll
        for (int q = 0; q < NCPY; ++q)
          if (q * TM / NCPY == G) copy(IC{}, q, pc);
      }
#pragma unroll
      for (int f = 0; f < TM + TN; ++f) {
        if (frag_seg<TM, TN>(f) == G) {
          if (frag_is_a<TM>(f)) fra.template read<RB, RH>(ldsc, frag_idx<TM>(f), FNA[frag_idx<TM>(f)]);
          else frb.template read<RB, RH>(ldsc, frag_idx<TM>(f), FNB[frag_idx<TM>(f)]);
        }
      }
      mfma_rows_t<G, G + 1, TN>(acc, FCA, FCB);
      constexpr int nds = seg_ds_count<AK, BKM, TM, TN>(G);
      static_assert(nds <= TN, "a segment's fragment reads pair with its MFMAs");
      if constexpr (nds > 0) {
#pragma unroll
        for (int r = 0; r < nds; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x008, TN - nds, 0);
    };
    segment(I0{});
    if constexpr (ODD) __builtin_amdgcn_s_setprio(0);
    segment(I1{});
    segment(I2{});
    segment(I3{});
  };
  for (int j = 0; j < nk; j += 4) {
    step(I0{}, j, fa, fb, ga, gb);
    step(I1{}, j + 1, ga, gb, fa, fb);
    if (j + 2 < nk) {
      step(I2{}, j + 2, fa, fb, ga, gb);
      step(I3{}, j + 3, ga, gb, fa, fb);
    }
  }
  wait_vmcnt0();

  // (a run-time test on purpose: with the LDS epilogue below still compiled in, the kernel keeps the plain kernel's
  // register allocation; as a compile-time branch the compiler spills around the partial-tile stores)
  if (SPLIT && AK && split >= 0) {
    // fp32 partial tile [split][M][N], straight from the accumulators: lane l holds row 16 tm + (l & 15) and the 4
    // columns 16 tn + 4 (l >> 4) .. + 3 of the wave's sub-tile (N % 8 == 0: a 4-column group is in or out)
    const int r0 = tile_m * BM + wm * WM + (lane & 15), c0 = tile_n * BN + wn * WN + 4 * (lane >> 4);
    const float* const part = pp.part + (int64_t)split * p.M * p.N;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int r = r0 + 16 * tm;
      if (r < p.M) {
        float* const row = const_cast<float*>(part) + (int64_t)r * p.N;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int c = c0 + 16 * tn;
          if (c < p.N) *reinterpret_cast<f32x4_t*>(row + c) = acc[tm][tn];
        }
      }
    }
    return;
  }

  // ---- epilogue, staged through LDS one 16-row chunk at a time: each wave writes the fp32 accumulators of its
  // rows 16 tm .. 16 tm + 15 (all 128 of its columns) to a padded buffer of its own, one 16-byte write per block,
  // then walks the chunk row by row with consecutive lanes on consecutive column pairs, so the math runs in a
  // compact loop and every row leaves as one contiguous 256-byte store.
  __syncthreads();
  float* ep = reinterpret_cast<float*>(reinterpret_cast<char*>(&lds[0]) + wave * EPW);
  uint16_t* ax = reinterpret_cast<uint16_t*>(ep + 16 * EP);
  const int row0 = tile_m * BM + wm * WM;
  // aux prefetch: lane covers rows lane/16 + 4q of the chunk, 8 columns at 8 (lane % 16); q >= 4: the up half
  u32x4_t xr[NAUX > 0 ? NAUX : 1];
  const int xcol = min(tile_n * BN + wn * WN + 8 * (lane & 15), p.N - 8);
#define TP_AUX_LOAD(TMC)                                                                                       \
  _Pragma("unroll") for (int q = 0; q < NAUX; ++q) {                                                           \
    const int xrow = min(row0 + (TMC) * 16 + (lane >> 4) + 4 * (q & 3), p.M - 1);                              \
    xr[q] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.aux) + (int64_t)xrow * p.ldaux +  \
                                             (q >> 2) * p.fhalf + xcol);                                       \
  }
  if constexpr (NAUX > 0) { TP_AUX_LOAD(0) }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      *reinterpret_cast<f32x4_t*>(ep + (lane & 15) * EP + tn * 16 + 4 * (lane >> 4)) = acc[tm][tn];
    if constexpr (NAUX > 0) {
#pragma unroll
      for (int q = 0; q < NAUX; ++q)
        *reinterpret_cast<u32x4_t*>(ax + (q >> 2) * 2048 + ((lane >> 4) + 4 * (q & 3)) * 128 + 8 * (lane & 15)) = xr[q];
      if (tm + 1 < TM) { TP_AUX_LOAD(tm + 1) }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (SPLIT && !AK && split >= 0) {
      // a weight-gradient pair's tail tile: the fp32 partial goes to its 256 x 256 block (the direct stores of the
      // K-major case above cost this layout some 90 registers)
      float* const blk = pp.part + ((int64_t)(tile_id - pp.nfull) * pp.ksplit + split) * (BM * BN);
      partial_chunk(p, ep, EP, row0 + tm * 16, tile_m * BM, tile_n, wn, lane, blk);
    } else {
      epilogue_chunk<EPI, WN>(p, ep, EP, row0 + tm * 16, tile_n, wn, lane, ax);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#undef TP_AUX_LOAD
}

// ------------------------------------------------------------------------------------------------------------------
// Tile configurations and dispatch.
// ------------------------------------------------------------------------------------------------------------------
struct Cfg {
  int bm, bn, nwm, nwn;
  float eff;  // relative per-tile efficiency used to trade tile size against filling the CUs
};
// eff: measured throughput of a full wave of tiles relative to the large-tile kernel (at K in the thousands)
constexpr Cfg kCfgs[] = {
    {256, 256, 2, 4, 1.00f},
    {256, 128, 2, 2, 0.50f},
    {128, 128, 2, 2, 0.50f},
    {64, 64, 2, 2, 0.25f},
};
// Compute units of the current device (256 on an MI355X), asked once per device.  The large-tile kernel holds one
// workgroup per CU, so this is also how many of its tiles run at once (one round).
int num_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0: not yet asked
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}
const char* const kEpiNames[] = {"store", "bias", "bias_act", "swiglu_fwd", "act_bwd", "swiglu_bwd", "ln_act",
                                 "ln_swiglu"};

int choose_cfg(int M, int ntiles_cols_of_bn256, int N, bool swig, int fhalf) {
  (void)ntiles_cols_of_bn256;
  const int ncu = num_cus();
  int best = 0;
  float best_score = -1.f;
  for (int i = 0; i < (int)(sizeof(kCfgs) / sizeof(kCfgs[0])); ++i) {
    const Cfg& c = kCfgs[i];
    const long nbm = (M + c.bm - 1) / c.bm;
    const long nbn = swig ? (fhalf + c.bn / 2 - 1) / (c.bn / 2) : (N + c.bn - 1) / c.bn;
    const long tiles = nbm * nbn;
    const long waves = (tiles + ncu - 1) / ncu;
    // useful fraction of the computed tile area (ragged edges) times the fill of the last wave
    const double rows_used = (double)M / (double)(nbm * c.bm);
    const double cols_used = swig ? (double)fhalf / (double)(nbn * c.bn / 2) : (double)N / (double)(nbn * c.bn);
    const double fill = (double)tiles / (double)(waves * ncu);
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

int big_tiles(const GemmParams& p, bool swig, int bn = 256) {
  const int nbm = (p.M + 255) / 256;
  const int nbn = swig ? (p.fhalf + 127) / 128 : (p.N + bn - 1) / bn;
  return nbm * nbn;
}

// Throughput per flop of the 192-column tiles relative to the 256-column ones (more copy bytes and fragment reads
// per MFMA): 0.82, measured where both widths take one round (the 22B attention block's QKV GEMM, 144 tiles of
// 256 or 192 of 192 columns: 120.5 -> 109 us).
constexpr double kEff192 = 0.82;

// Relative time of a large-tile launch of `tiles` workgroups of bn columns, ksplit K runs each: rounds of one tile
// per CU, each as long as a tile's share of the work.
double big_time(int tiles, int bn, int ksplit) {
  const int ncu = num_cus();
  const long wg = (long)tiles * ksplit;
  const long rounds = (wg + ncu - 1) / ncu;
  return (double)rounds * (bn / 256.0) / ksplit / (bn == 256 ? 1.0 : kEff192);
}

// 192-column tiles where they finish sooner: a GEMM whose 256-column tiles leave much of their last round of CUs
// idle (the attention block's per-rank GEMMs, the 8.3B-width MLP).  K-major A only, and not for the SwiGLU
// epilogues (their column halves are laid out for 256).
bool use_n192(const GemmParams& p, bool ak, int epi) {
  if (!ak || epi == EPI_SWIGLU_FWD || epi == EPI_SWIGLU_BWD || epi == EPI_LN_SWIGLU) return false;
  return big_time(big_tiles(p, false, 192), 192, 1) < big_time(big_tiles(p, false), 256, 1);
}

template <bool AK, bool BKM, int EPI, int BNT = 256>
hipError_t launch_big(const GemmParams& p0, const GemmParams* p1, hipStream_t st) {
  GemmPair pp;
  pp.g[0] = p0;
  pp.g[1] = p1 ? *p1 : p0;
  pp.tiles0 = big_tiles(p0, epi_swiglu_fwd(EPI), BNT);
  pp.tiles1 = p1 ? big_tiles(*p1, epi_swiglu_fwd(EPI), BNT) : 0;
  pp.ksplit = 1;
  pp.nfull = 0;
  pp.part = nullptr;
  const int total = pp.tiles0 + pp.tiles1;

  const std::string w = BNT == 256 ? "" : std::to_string(BNT);
  static const std::string name = std::string("gemm_bf16_big") + w + "_" + (AK ? "K" : "M") + (BKM ? "K" : "M") +
                                  "_" + kEpiNames[EPI];
  static const std::string name2 = std::string("gemm_bf16_big") + w + "_pair_" + (AK ? "K" : "M") +
                                   (BKM ? "K" : "M") + "_" + kEpiNames[EPI];
  // 8 waves (two per SIMD, the pair-buffer loop) for every layout
  constexpr int NW = 8;
  return TP_LAUNCH(p1 ? name2.c_str() : name.c_str(), (gemm_bf16_big_kernel<AK, BKM, EPI, false, NW, BNT>),
                   dim3((unsigned)total), dim3(NW * 64), 0, st, pp);
}

// Sum of the ksplit fp32 partial tiles in split order, then the epilogue (store, or bias + store), one rounding.
// One thread per 4 consecutive columns.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_sum_kernel(GemmParams p, const float* __restrict__ part, int ksplit) {
  const int64_t nq = (int64_t)p.M * (p.N / 4);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nq) return;
  const int64_t m = i / (p.N / 4);
  const int c = (int)(i - m * (p.N / 4)) * 4;
  const int64_t stride = (int64_t)p.M * p.N;
  const float* src = part + m * p.N + c;
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(src);
  for (int sp = 1; sp < ksplit; ++sp) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + sp * stride);
    acc[0] += v[0];
    acc[1] += v[1];
    acc[2] += v[2];
    acc[3] += v[3];
  }
  if constexpr (EPI == EPI_BIAS) {
    if (p.bias != nullptr) {
      const float2 b01 = ldg_bf16x2(p.bias, c), b23 = ldg_bf16x2(p.bias, c + 2);
      acc[0] += b01.x;
      acc[1] += b01.y;
      acc[2] += b23.x;
      acc[3] += b23.y;
    }
  }
  uint2 w;
  w.x = pack_bf16x2(acc[0], acc[1]);
  w.y = pack_bf16x2(acc[2], acc[3]);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.C) + m * p.ldc + c) = w;
}

// Split-K for a single GEMM whose 256 x 256 tiles fill few CUs: the number of K runs that brings tiles * runs
// closest to one full round (at most 8 runs, each at least two 64-deep pairs of k-tiles, the partials fitting the
// scratch); 1 when splitting does not pay.
int choose_ksplit(const GemmParams& p, int tiles, int64_t part_floats) {
  const int ncu = num_cus();
  if (tiles * 4 >= ncu * 3) return 1;
  const int pairs = p.K / (2 * BK2);
  int best = 1;
  for (int sp = 2; sp <= 8; ++sp) {
    if (tiles * sp > ncu) break;
    if (pairs / sp < 2) break;
    if ((int64_t)sp * p.M * p.N > part_floats) break;
    best = sp;
  }
  return best;
}

template <bool AK, bool BKM, int EPI, int BNT = 256>
hipError_t launch_big_split(const GemmParams& p, int ksplit, float* part, hipStream_t st) {
  GemmPair pp;
  pp.g[0] = p;
  pp.g[1] = p;
  pp.tiles0 = big_tiles(p, false, BNT);
  pp.tiles1 = 0;
  pp.ksplit = ksplit;
  pp.nfull = 0;
  pp.part = part;
  const std::string w = BNT == 256 ? "" : std::to_string(BNT);
  static const std::string name = std::string("gemm_bf16_big") + w + "_splitk_" + (AK ? "K" : "M") + (BKM ? "K" : "M");
  hipError_t e = TP_LAUNCH(name.c_str(), (gemm_bf16_big_kernel<AK, BKM, EPI_STORE, true, 8, BNT>),
                           dim3((unsigned)(pp.tiles0 * ksplit)), dim3(512), 0, st, pp);
  if (e != hipSuccess) return e;
  const int64_t nq = (int64_t)p.M * (p.N / 4);
  return TP_LAUNCH("gemm_bf16_splitk_sum", splitk_sum_kernel<EPI>, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0,
                   st, p, part, ksplit);
}

// Sum of the tail tiles' fp32 partial blocks (tile-block layout) in split order, stored as bf16 into the problem
// each tile belongs to.  One thread per 4 consecutive columns of a 256 x 256 block; the tile decode is the large-tile
// kernel's (big_row_group).
__global__ __launch_bounds__(256) void splitk_tail_sum_kernel(GemmPair pp, int ntail) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)ntail * (256 * 64)) return;
  const int j = (int)(i >> 14);  // tail tile
  const int e = (int)(i & 16383) * 4;
  const int rl = e >> 8, cl = e & 255;
  int u = pp.nfull + j;
  const int which = u < pp.tiles0 ? 0 : 1;
  const GemmParams& p = pp.g[which];
  if (which) u -= pp.tiles0;
  const int nbm = (p.M + 255) / 256, nbn = (p.N + 255) / 256;
  const int gm = big_row_group(pp.tiles1 > 0, EPI_STORE, false, false);  // the kernel's own walk (MN x MN, store)
  const int first_m = (u / (gm * nbn)) * gm;
  const int gsz = min(nbm - first_m, gm);
  const int tile_m = first_m + (u % (gm * nbn)) % gsz;
  const int tile_n = (u % (gm * nbn)) / gsz;
  const int r = tile_m * 256 + rl, c = tile_n * 256 + cl;
  if (r >= p.M || c >= p.N) return;
  const float* src = pp.part + (int64_t)j * pp.ksplit * 65536 + rl * 256 + cl;
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(src);
  for (int sp = 1; sp < pp.ksplit; ++sp) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src + (int64_t)sp * 65536);
    acc[0] += v[0];
    acc[1] += v[1];
    acc[2] += v[2];
    acc[3] += v[3];
  }
  uint2 w;
  w.x = pack_bf16x2(acc[0], acc[1]);
  w.y = pack_bf16x2(acc[2], acc[3]);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.C) + (int64_t)r * p.ldc + c) = w;
}

// The large-tile kernel needs an even number of 32-deep k-tiles, more than it keeps in flight (K >= 128), and
// every per-lane copy offset below 2^32 bytes: the whole operand for a K-major one, one k-tile's 32 rows for an
// MN-major one (whose k-tiles advance a 64-bit base).
bool big_fits(const GemmParams& p, bool a_kmajor, bool b_kmajor) {
  if (p.K % (2 * BK2) != 0 || p.K < 4 * BK2) return false;
  const int64_t lim = (int64_t)1 << 31;  // elements of 2 bytes
  const int64_t a_end = a_kmajor ? (int64_t)(p.M - 1) * p.lda + p.K : (int64_t)(BK2 - 1) * p.lda + p.M;
  const int64_t b_end = b_kmajor ? (int64_t)(p.N - 1) * p.ldb + p.K : (int64_t)(BK2 - 1) * p.ldb + p.N;
  return a_end < lim && b_end < lim;
}

template <bool AK, bool BKM, int EPI>
hipError_t launch_cfg(int ci, const GemmParams& p, hipStream_t st) {
  switch (ci) {
    case 0:
      if (big_fits(p, AK, BKM)) {
        if constexpr (AK && !epi_swiglu_fwd(EPI) && EPI != EPI_SWIGLU_BWD) {
          if (use_n192(p, AK, EPI)) return launch_big<AK, BKM, EPI, 192>(p, nullptr, st);
        }
        return launch_big<AK, BKM, EPI>(p, nullptr, st);
      }
      return launch_one<256, 256, 2, 4, AK, BKM, EPI>(p, st);
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

hipError_t gemm_bf16_ln(const GemmParams& p, int epi, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (!big_fits(p, true, false)) return hipErrorInvalidValue;
  if (epi == EPI_LN_ACT) return launch_big<true, false, EPI_LN_ACT>(p, nullptr, st);
  if (epi == EPI_LN_SWIGLU) return launch_big<true, false, EPI_LN_SWIGLU>(p, nullptr, st);
  return hipErrorInvalidValue;
}

// The LayerNorm fold: 16 waves per workgroup, 128 columns (2 per lane); wave w takes rows w, w + 16, ...; the 16
// partial sums of a column are added in wave order.
__global__ __launch_bounds__(1024) void ln_fold_kernel(const uint16_t* __restrict__ gamma,
                                                       const uint16_t* __restrict__ beta,
                                                       const uint16_t* __restrict__ A, const uint16_t* __restrict__ a,
                                                       int64_t h, int64_t n, uint16_t* __restrict__ A_ln,
                                                       float* __restrict__ c, float* __restrict__ b) {
  __shared__ float red[2][16][128];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 128 + 2 * lane;
  float c0 = 0.f, c1 = 0.f, b0 = 0.f, b1 = 0.f;
  if (j < n) {
#pragma unroll 4
    for (int64_t k = wave; k < h; k += 16) {
      const float g = bf16_to_f32(gamma[k]), be = bf16_to_f32(beta[k]);
      const uint32_t w = *reinterpret_cast<const uint32_t*>(A + k * n + j);
      const float a0 = bf16_to_f32(w & 0xFFFFu), a1 = bf16_to_f32(w >> 16);
      const uint32_t o = pack_bf16x2(g * a0, g * a1);  // the product of two bf16 values is exact in fp32
      *reinterpret_cast<uint32_t*>(A_ln + k * n + j) = o;
      c0 += bf16_to_f32(o & 0xFFFFu);
      c1 += bf16_to_f32(o >> 16);
      b0 = fmaf(be, a0, b0);
      b1 = fmaf(be, a1, b1);
    }
  }
  red[0][wave][2 * lane] = c0;
  red[0][wave][2 * lane + 1] = c1;
  red[1][wave][2 * lane] = b0;
  red[1][wave][2 * lane + 1] = b1;
  __syncthreads();
  if (wave == 0 && j < n) {
    float sc0 = 0.f, sc1 = 0.f, sb0 = 0.f, sb1 = 0.f;
    for (int w = 0; w < 16; ++w) {
      sc0 += red[0][w][2 * lane];
      sc1 += red[0][w][2 * lane + 1];
      sb0 += red[1][w][2 * lane];
      sb1 += red[1][w][2 * lane + 1];
    }
    if (a != nullptr) {
      sb0 += bf16_to_f32(a[j]);
      sb1 += bf16_to_f32(a[j + 1]);
    }
    c[j] = sc0;
    c[j + 1] = sc1;
    b[j] = sb0;
    b[j + 1] = sb1;
  }
}

hipError_t ln_fold_weights(const void* gamma, const void* beta, const void* A, const void* a, int64_t h, int64_t n,
                           void* A_ln, float* c, float* b, hipStream_t st) {
  return TP_LAUNCH("ln_fold_weights", ln_fold_kernel, dim3((unsigned)((n + 127) / 128)), dim3(1024), 0, st,
                   static_cast<const uint16_t*>(gamma), static_cast<const uint16_t*>(beta),
                   static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(a), h, n,
                   static_cast<uint16_t*>(A_ln), c, b);
}

// The two weight-gradient GEMMs of a backward (both MN-major x MN-major, same K = s*b): one launch over both tile
// sets when the large-tile kernel applies to both and together they fill the GPU better than each alone.
hipError_t gemm_bf16_wgrad_pair(const GemmParams& p0, const GemmParams& p1, hipStream_t st) {
  if (p0.M > 0 && p0.N > 0 && p1.M > 0 && p1.N > 0 && p0.K == p1.K && big_fits(p0, false, false) &&
      big_fits(p1, false, false)) {
    const int t = big_tiles(p0, false) + big_tiles(p1, false);
    const int c0 = choose_cfg(p0.M, 0, p0.N, false, 0), c1 = choose_cfg(p1.M, 0, p1.N, false, 0);
    if (t >= num_cus() * 3 / 4 || (c0 == 0 && c1 == 0)) return launch_big<false, false, EPI_STORE>(p0, &p1, st);
  }
  hipError_t e = gemm_bf16(p0, false, false, EPI_STORE, st);
  if (e == hipSuccess) e = gemm_bf16(p1, false, false, EPI_STORE, st);
  return e;
}

// The pair's tile count past its last full round of one tile per CU (the tail): when the tail fills under three
// quarters of the CUs and the scratch allows, the tail tiles split K over ksplit workgroups each.
hipError_t gemm_bf16_wgrad_pair_splitk(const GemmParams& p0, const GemmParams& p1, float* part, int64_t part_floats,
                                       hipStream_t st) {
  if (part != nullptr && p0.M > 0 && p0.N > 0 && p1.M > 0 && p1.N > 0 && p0.K == p1.K && big_fits(p0, false, false) &&
      big_fits(p1, false, false)) {
    const int t = big_tiles(p0, false) + big_tiles(p1, false);
    const int ncu = num_cus();
    const int ntail = t % ncu;
    if (t > ncu && ntail > 0 && ntail * 4 < ncu * 3) {
      const int pairs = p0.K / (2 * BK2);
      int ks = 1;
      for (int sp = 2; sp <= 8; ++sp) {
        if (ntail * sp > ncu || pairs / sp < 2 || (int64_t)ntail * sp * 65536 > part_floats) break;
        ks = sp;
      }
      if (ks > 1) {
        GemmPair pp;
        pp.g[0] = p0;
        pp.g[1] = p1;
        pp.tiles0 = big_tiles(p0, false);
        pp.tiles1 = big_tiles(p1, false);
        pp.ksplit = ks;
        pp.nfull = t - ntail;
        pp.part = part;
        hipError_t e = TP_LAUNCH("gemm_bf16_big_pair_splitk_MM", (gemm_bf16_big_kernel<false, false, EPI_STORE, true, 8>),
                                 dim3((unsigned)(pp.nfull + ntail * ks)), dim3(512), 0, st, pp);
        if (e != hipSuccess) return e;
        const int64_t nq = (int64_t)ntail * 16384;
        return TP_LAUNCH("gemm_bf16_splitk_tail_sum", splitk_tail_sum_kernel, dim3((unsigned)((nq + 255) / 256)),
                         dim3(256), 0, st, pp, ntail);
      }
    }
  }
  return gemm_bf16_wgrad_pair(p0, p1, st);
}

hipError_t gemm_bf16_splitk(const GemmParams& p, bool a_kmajor, bool b_kmajor, int epi, float* part,
                            int64_t part_floats, hipStream_t st) {
  if (part != nullptr && p.M > 0 && p.N > 0 && (epi == EPI_STORE || epi == EPI_BIAS) && a_kmajor &&
      big_fits(p, a_kmajor, b_kmajor)) {
    // the tile width and the split together: each width's best split, then the sooner of the two
    const int ks = choose_ksplit(p, big_tiles(p, false), part_floats);
    const int ks192 = choose_ksplit(p, big_tiles(p, false, 192), part_floats);
    const bool n192 = big_time(big_tiles(p, false, 192), 192, ks192) < big_time(big_tiles(p, false), 256, ks);
    if (n192 && ks192 > 1) {
      if (b_kmajor)
        return epi == EPI_STORE ? launch_big_split<true, true, EPI_STORE, 192>(p, ks192, part, st)
                                : launch_big_split<true, true, EPI_BIAS, 192>(p, ks192, part, st);
      return epi == EPI_STORE ? launch_big_split<true, false, EPI_STORE, 192>(p, ks192, part, st)
                              : launch_big_split<true, false, EPI_BIAS, 192>(p, ks192, part, st);
    }
    if (!n192 && ks > 1) {
      if (b_kmajor)
        return epi == EPI_STORE ? launch_big_split<true, true, EPI_STORE>(p, ks, part, st)
                                : launch_big_split<true, true, EPI_BIAS>(p, ks, part, st);
      return epi == EPI_STORE ? launch_big_split<true, false, EPI_STORE>(p, ks, part, st)
                              : launch_big_split<true, false, EPI_BIAS>(p, ks, part, st);
    }
  }
  return gemm_bf16(p, a_kmajor, b_kmajor, epi, st);
}

}  // namespace tp
