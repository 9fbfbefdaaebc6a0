// Per-rank attention forward for the a/t local heads: O_j = softmax(Q_j K_j^T / sqrt(d), causal) V_j, computed
// one key block at a time with the online-softmax merge of running (max, sum) statistics ("Tensor Parallelism
// (TP) 与 Sequence Parallelism (SP)" §3 and the Megatron-LM visual reading: heads are independent, each is local
// to its rank; "Sequence Parallel 与 Context Parallel", CP step 3: block statistics merged by online softmax).
//
// bf16 kernel, one workgroup = 64 queries of one (batch, head), 4 waves x 16 queries, key blocks of 64:
//   * S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16): K rows come from LDS, the wave's 16 queries sit
//     in registers for the whole kernel.  In the transposed product every lane owns one query (lane & 15), so the
//     row statistics need only a max over the 4 lane groups that share it.
//   * O^T = V^T P^T: the probabilities never leave registers.  A lane holds scores for keys 4g..4g+3 and
//     16+4g..16+4g+3 of each 32-key step (g = lane >> 4); the V^T fragment is read with the same key order, so the
//     pair of operands agree on k and the product is exact whatever order the 32 keys take.
//   * V is transposed on its way into LDS (8 keys x 4 dims per thread), K is copied as is; both are double
//     buffered with the next block's loads in flight during the current block's math.
//   * Query tiles are issued heaviest first (causal work grows with the tile index).
#include <math.h>

#include <string>

#include "tp_common.h"

namespace tp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int QT = 64;   // queries per workgroup
constexpr int KT = 64;   // keys per block
constexpr int VP = KT + 8;  // V^T row pitch in elements (odd number of 16-byte chunks)

template <int DP>
__global__ __launch_bounds__(256) void attn_fwd_bf16_kernel(AttnParams p) {
  constexpr int KP = DP + 8;       // K row pitch in elements (odd number of 16-byte chunks)
  constexpr int NDS = DP / 32;     // 32-wide d steps of S^T
  constexpr int NST = DP / 16;     // 16-row d subtiles of O^T
  constexpr int KCH = DP / 8;      // 16-byte chunks per K row
  constexpr int KLD = (KT * KCH + 255) / 256;  // K chunks per thread
  constexpr int VBLK = (KT / 8) * (DP / 4);     // 8x4 blocks in a V tile
  constexpr int VLD = (VBLK + 255) / 256;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][DP * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  const int nq = (p.s + QT - 1) / QT;
  const int qtile = nq - 1 - (int)blockIdx.x;
  const int bh = blockIdx.y;
  const int bidx = bh / p.hl, jj = bh % p.hl;
  const int d = p.d;
  const int64_t ldq = (int64_t)p.hl * 3 * d;  // elements per token row of QKV
  const int64_t tok_stride = ldq * p.b;        // consecutive sequence positions
  const uint16_t* __restrict__ qkv = static_cast<const uint16_t*>(p.qkv) + (int64_t)bidx * ldq + (int64_t)jj * 3 * d;
  const uint16_t* __restrict__ kbase = qkv + d;
  const uint16_t* __restrict__ vbase = qkv + 2 * d;

  // ---- this lane's query and its fragments (k = d: lane supplies d = 32u + 8g .. +8)
  const int q = qtile * QT + wave * 16 + (lane & 15);
  bf16x8_t qf[NDS];
#pragma unroll
  for (int u = 0; u < NDS; ++u) {
    const int dd = 32 * u + 8 * g;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (q < p.s && dd < d) v = *reinterpret_cast<const uint4*>(qkv + (int64_t)q * tok_stride + dd);
    qf[u] = __builtin_bit_cast(bf16x8_t, v);
  }

  uint4 kreg[KLD];
  uint2 vreg[VLD][8];
  auto load_tile = [&](int kt) {
    const int kv0 = kt * KT;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int c = tid + 256 * i;
      const int r = c / KCH, ch = c % KCH;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (c < KT * KCH && kv0 + r < p.s && ch * 8 < d)
        v = *reinterpret_cast<const uint4*>(kbase + (int64_t)(kv0 + r) * tok_stride + ch * 8);
      kreg[i] = v;
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int bq = tid + 256 * i;
      const int gd = bq % (DP / 4), kg = bq / (DP / 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kv = kv0 + kg * 8 + j;
        uint2 v = make_uint2(0u, 0u);
        if (bq < VBLK && kv < p.s && gd * 4 < d)
          v = *reinterpret_cast<const uint2*>(vbase + (int64_t)kv * tok_stride + gd * 4);
        vreg[i][j] = v;
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int c = tid + 256 * i;
      if (c < KT * KCH) {
        const int r = c / KCH, ch = c % KCH;
        *reinterpret_cast<uint4*>(&Ks[buf][r * KP + ch * 8]) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int bq = tid + 256 * i;
      if (bq < VBLK) {
        const int gd = bq % (DP / 4), kg = bq / (DP / 4);
        uint32_t w[4][4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint32_t x0 = vreg[i][2 * pp].x, x1 = vreg[i][2 * pp + 1].x;
          const uint32_t y0 = vreg[i][2 * pp].y, y1 = vreg[i][2 * pp + 1].y;
          w[0][pp] = (x0 & 0xFFFFu) | (x1 << 16);
          w[1][pp] = (x0 >> 16) | (x1 & 0xFFFF0000u);
          w[2][pp] = (y0 & 0xFFFFu) | (y1 << 16);
          w[3][pp] = (y0 >> 16) | (y1 & 0xFFFF0000u);
        }
#pragma unroll
        for (int jn = 0; jn < 4; ++jn)
          *reinterpret_cast<uint4*>(&Vt[buf][(gd * 4 + jn) * VP + kg * 8]) =
              make_uint4(w[jn][0], w[jn][1], w[jn][2], w[jn][3]);
      }
    }
  };

  const float sl2 = p.scale * 1.4426950408889634f;  // scores in log2 units
  float m_run = -INFINITY, l_part = 0.f;
  f32x4_t acc_o[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) acc_o[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nkt_all = (p.s + KT - 1) / KT;
  const int nkt = p.causal ? min(nkt_all, qtile + 1) : nkt_all;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) load_tile(kt + 1);
    const uint16_t* K_ = Ks[cur];
    const uint16_t* V_ = Vt[cur];
    const int kv0 = kt * KT;

    // S^T [64 keys x 16 queries] in 4 subtiles of 16 keys
    f32x4_t sc[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      sc[ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int kr = ks * 16 + (lane & 15);
#pragma unroll
      for (int u = 0; u < NDS; ++u) {
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&K_[kr * KP + 32 * u + 8 * g]));
        sc[ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[u], sc[ks], 0, 0, 0);
      }
    }
    // scale, mask, block max
    const bool need_mask = (p.causal && kt == qtile) || (kv0 + KT > p.s);
    float mx = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = sc[ks][e] * sl2;
        if (need_mask) {
          const int kv = kv0 + ks * 16 + 4 * g + e;
          if (kv >= p.s || (p.causal && kv > q)) x = -INFINITY;
        }
        sc[ks][e] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float corr = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
    uint32_t pk[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = (m_new == -INFINITY) ? 0.f : exp2f(sc[ks][e] - m_new);
        psum += pe[e];
      }
      pk[ks][0] = f32_to_bf16_hw(pe[0]) | (f32_to_bf16_hw(pe[1]) << 16);
      pk[ks][1] = f32_to_bf16_hw(pe[2]) | (f32_to_bf16_hw(pe[3]) << 16);
    }
    l_part = l_part * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int st = 0; st < NST; ++st) acc_o[st] *= corr;

    // O^T [d x 16 queries] += V^T P^T, two 32-key steps
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pk[2 * u][0], pk[2 * u][1], pk[2 * u + 1][0], pk[2 * u + 1][1]));
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int dr = st * 16 + (lane & 15);
        const uint2 lo = *reinterpret_cast<const uint2*>(&V_[dr * VP + 32 * u + 4 * g]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&V_[dr * VP + 32 * u + 16 + 4 * g]);
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc_o[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc_o[st], 0, 0, 0);
      }
    }
    if (more) store_tile(cur ^ 1);
    __syncthreads();
  }

  float l_tot = l_part;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (q < p.s) {
    const float inv = 1.f / l_tot;
    uint16_t* o = static_cast<uint16_t*>(p.o) + ((int64_t)q * p.b + bidx) * ((int64_t)p.hl * d) + (int64_t)jj * d;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int dd = st * 16 + 4 * g;
      if (dd < d) {
        uint2 w;
        w.x = f32_to_bf16_hw(acc_o[st][0] * inv) | (f32_to_bf16_hw(acc_o[st][1] * inv) << 16);
        w.y = f32_to_bf16_hw(acc_o[st][2] * inv) | (f32_to_bf16_hw(acc_o[st][3] * inv) << 16);
        *reinterpret_cast<uint2*>(o + dd) = w;
      }
    }
    if (p.lse != nullptr && g == 0)
      p.lse[((int64_t)bidx * p.hl + jj) * p.s + q] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  }
}

// fp32: one thread per query, keys visited one at a time with the same online merge.
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnParams p) {
  constexpr int DMAX = 128;
  const int q = blockIdx.x * 64 + threadIdx.x;
  const int bh = blockIdx.y;
  const int bidx = bh / p.hl, jj = bh % p.hl;
  if (q >= p.s) return;
  const int d = p.d;
  const int64_t ldq = (int64_t)p.hl * 3 * d;
  const int64_t tok = ldq * p.b;
  const float* qkv = static_cast<const float*>(p.qkv) + (int64_t)bidx * ldq + (int64_t)jj * 3 * d;
  const float* qv = qkv + (int64_t)q * tok;
  float o[DMAX];
  for (int e = 0; e < d; ++e) o[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int nk = p.causal ? q + 1 : p.s;
  for (int k = 0; k < nk; ++k) {
    const float* kv = qkv + (int64_t)k * tok;
    float sdot = 0.f;
    for (int e = 0; e < d; ++e) sdot = fmaf(qv[e], kv[d + e], sdot);
    const float x = sdot * p.scale;
    const float mn = fmaxf(m, x);
    const float corr = expf(m - mn);
    const float pe = expf(x - mn);
    l = l * corr + pe;
    for (int e = 0; e < d; ++e) o[e] = o[e] * corr + pe * kv[2 * d + e];
    m = mn;
  }
  float* out = static_cast<float*>(p.o) + ((int64_t)q * p.b + bidx) * ((int64_t)p.hl * d) + (int64_t)jj * d;
  for (int e = 0; e < d; ++e) out[e] = o[e] / l;
  if (p.lse != nullptr) p.lse[((int64_t)bidx * p.hl + jj) * p.s + q] = m + logf(l);
}

template <int DP>
hipError_t launch_bf16(const AttnParams& p, hipStream_t st) {
  const int nq = (p.s + QT - 1) / QT;
  static const std::string name = "attn_fwd_bf16_d" + std::to_string(DP);
  return TP_LAUNCH(name.c_str(), (attn_fwd_bf16_kernel<DP>), dim3((unsigned)nq, (unsigned)(p.b * p.hl)), dim3(256), 0,
                   st, p);
}

}  // namespace

hipError_t attention_bf16(const AttnParams& p, hipStream_t st) {
  if (p.s <= 0 || p.b <= 0 || p.hl <= 0) return hipSuccess;
  if (p.d <= 32) return launch_bf16<32>(p, st);
  if (p.d <= 64) return launch_bf16<64>(p, st);
  if (p.d <= 96) return launch_bf16<96>(p, st);
  return launch_bf16<128>(p, st);
}

hipError_t attention_f32(const AttnParams& p, hipStream_t st) {
  if (p.s <= 0 || p.b <= 0 || p.hl <= 0) return hipSuccess;
  return TP_LAUNCH("attn_fwd_f32", attn_fwd_f32_kernel, dim3((unsigned)((p.s + 63) / 64), (unsigned)(p.b * p.hl)),
                   dim3(64), 0, st, p);
}

}  // namespace tp
