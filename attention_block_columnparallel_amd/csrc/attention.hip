// Per-rank attention forward for the a/t local heads: O_j = softmax(Q_j K_j^T / sqrt(d), causal) V_j, computed
// one key block at a time with the online-softmax merge of running (max, sum) statistics ("Tensor Parallelism
// (TP) 与 Sequence Parallelism (SP)" §3 and the Megatron-LM visual reading: heads are independent, each is local
// to its rank; "Sequence Parallel 与 Context Parallel", CP step 3: block statistics merged by online softmax).
//
// bf16 kernel, one workgroup = 64 queries of one (batch, head), key blocks of 64, 8 waves: wave (kh, qw) takes 16
// queries (qw) and one 32-key half (kh) of every block, with statistics of its own, merged at the end:
//   * K and V tiles are copied as they sit in HBM (direct global -> LDS copies, 16 bytes per lane) into a ring of
//     LDS stages (3 at d <= 96, 2 at d = 128), so the copies of the next blocks are in flight while one block is
//     multiplied.  Within a row the 16-byte chunks are permuted by a per-row XOR pattern (tile_chunk), so both the
//     16-byte fragment reads and the transposing reads of a pass fall in distinct banks.
//   * S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16): K fragments are 16-byte LDS reads, the wave's
//     16 queries sit in registers for the whole kernel.  In the transposed product every lane owns one query
//     (lane & 15), so the row statistics need only a max over the 4 lane groups that share it.
//   * O^T = V^T P^T: the probabilities never leave registers.  A lane holds scores for keys 4g..4g+3 and
//     16+4g..16+4g+3 of its 32-key half (g = lane >> 4); the V^T fragment is gathered from the untransposed V tile
//     by two transposing LDS reads (ds_read_b64_tr_b16) whose row addresses follow the same key order, so the pair
//     of operands agree on k.
//   * Softmax in base 2 with the scale folded into one FMA per score (exp2(s c - m c), c = scale log2 e) and the
//     hardware exp2; row statistics combine the 4 lane groups with the gfx950 lane swaps; the running output is
//     rescaled only in blocks where some query's maximum rose; the causal mask is one select per score.
//   * Query tiles are issued heaviest first over all heads (causal work grows with the tile index).
#include <math.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <type_traits>

#include "tp_common.h"

namespace tp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int QT = 64;   // queries per workgroup
constexpr int KT = 64;   // keys per block
// LDS stages (forward and backward kernels); 2 stages with three workgroups per CU and 4 stages with one each
// measured slower for the forward kernel at d = 96
constexpr int NSTG_F = 3;
constexpr int NSTG = 3;
// Stages of the forward's and the dQ pass's K / V ring for head size DP.  At d = 128 three stages take 96 KB, one
// workgroup per CU; two stages (64 KB) let two share a CU, which hides more latency than the deeper ring did
// (grouped-query shape, per rank: forward 116 -> 94 us, dQ 184 -> 176 us).
template <int DP>
constexpr int kv_stages() { return DP >= 128 ? 2 : NSTG_F; }
// Stages of the dK / dV pass's Q / dO ring: likewise two at d = 128, where two workgroups then share a CU
// (grouped-query shape: 204 -> 180 us per rank).
template <int DP>
constexpr int dkv_stages() { return DP >= 128 ? 2 : NSTG; }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Columns of a rank's QKV rows (grouped-query attention, G query heads per KV head; G = 1 is multi-head): per
// local KV group, the d columns of each of its G query heads, then the group's d key and d value columns (the
// interleave of the fused QKV weight in the Megatron-LM visual reading).
struct QkvCols {
  int64_t ld;  // elements per token row
  int64_t q;   // first column of query head jj
  int64_t k;   // first key column of jj's group; its values follow at + d
};
__device__ __forceinline__ QkvCols qkv_cols(int hl, int G, int d, int jj) {
  const int64_t gw = (int64_t)(G + 2) * d;
  const int jg = jj / G;
  QkvCols c;
  c.ld = (int64_t)(hl / G) * gw;
  c.q = jg * gw + (int64_t)(jj - jg * G) * d;
  c.k = jg * gw + (int64_t)G * d;
  return c;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at LDS byte address m0 + 16 l.  Inline
// assembly, so that the compiler does not wait for these copies at every barrier; the kernel waits itself.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr) : "memory", "m0");
}
// The same from a wave-uniform base (scalar registers) plus a 32-bit per-lane byte offset: no per-lane address
// arithmetic when the base moves.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}
// max(a, b) of two finite-or-infinite values, one instruction: fmaxf on values fresh from a lane swap costs two
// more, which quiet signalling NaNs that cannot occur here.
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
#pragma clang diagnostic pop
// Max / sum over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48) with the gfx950 lane swaps: with
// both operands equal, permlane32_swap returns {v[l], v[l^32]} in some order in its two results, permlane16_swap
// {v[l], v[l^16]}.  Every lane of a column ends with the same value.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Physical 16-byte chunk of logical chunk c of row r in a K / V (forward, dQ) or Q / dO (dK / dV) tile of CH
// chunks per row: c XOR z(r mod 8).  The LDS serves a 16-byte fragment read 8 lanes (128 bytes, 32 banks) per pass
// and a transposing 8-byte read 32 lanes (256 bytes, 64 banks) per pass -- the widths under which the large-tile
// GEMM's reads, which the bank-conflict counter reports free, are conflict-free, and which account for the counts
// measured here.  The two reads of these tiles touch 8 consecutive rows at one chunk (16-byte reads) and 8
// consecutive rows at an even-odd chunk pair (transposing reads); z makes both hit distinct banks:
//   CH = 4, 12 (rows start 0 or 4 chunks into a 128-byte window): z = r / 2;
//   CH = 8: z = r;  CH = 16: z = 2 r + r / 4.
// Each z keeps c ^ z a chunk of the row.  A rotation by the row index doubled the passes of the transposing reads
// at every head size and of the 16-byte reads at d = 96.
template <int CH>
__device__ __forceinline__ int tile_chunk(int r, int c) {
  static_assert(CH == 4 || CH == 8 || CH == 12 || CH == 16, "chunks per row");
  const int b = r & 7;
  const int z = (CH == 8) ? b : (CH == 16) ? 2 * b + (b >> 2) : (b >> 1);
  return c ^ z;
}

// Complete a wave's register-resident fragments (ordinary global loads) before its key or query loop: left to the
// compiler, the wait for them lands at their first use inside the loop as vmcnt(0) -- the compiler does not count
// the direct copies -- and drains the copies of the next blocks once per unrolled iteration.
template <typename T, int N>
__device__ __forceinline__ void settle(const T (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(f[i]));
}

// Work rank (0 = the most work) of the causal tile a workgroup takes, from its launch-order index u over n tiles.
// Heaviest first, so that workgroups dealt out as CUs free up balance greedily -- unless the whole grid is resident
// at once (fold): then the first half of the launch takes ranks 0 .. h-1 and the second half ranks n-1 down to h,
// so the two workgroups a CU receives (one from each half, in launch order) carry about the same total work.
__device__ __forceinline__ int work_rank(int u, int n, int fold) {
  const int h = (n + 1) / 2;
  return (fold && u >= h) ? n - 1 - (u - h) : u;
}

// Four fp32 values -> bf16 hi pairs and bf16 lo pairs with x = hi + lo to about 2^-16 relative: hi = bf16(x), lo =
// bf16(x - hi), the hi value read back from its packed bits.
__device__ __forceinline__ void split_hi_lo(const float (&x)[4], uint32_t (&hi)[2], uint32_t (&lo)[2]) {
  hi[0] = pack_bf16x2_hw(x[0], x[1]);
  hi[1] = pack_bf16x2_hw(x[2], x[3]);
  lo[0] = pack_bf16x2_hw(x[0] - __uint_as_float(hi[0] << 16), x[1] - __uint_as_float(hi[0] & 0xFFFF0000u));
  lo[1] = pack_bf16x2_hw(x[2] - __uint_as_float(hi[1] << 16), x[3] - __uint_as_float(hi[1] & 0xFFFF0000u));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The forward kernel.  Wave (kh, qw) of the 8 takes queries 16 qw .. 16 qw + 15 of the tile and keys
// 32 kh .. 32 kh + 31 of every block, with running statistics of its own; the two halves of each query group merge
// through LDS at the end (m = max(m0, m1), l = l0 2^(m0-m) + l1 2^(m1-m), likewise O).  Splitting the keys rather
// than giving each wave all 64 keys of a block (4 waves of 16 queries; about 5% slower at d = 96 and 128) lets a
// SIMD hold four waves over the same K / V tiles instead of two.  Only the kh = 0 waves issue the copies (their
// waits count them); a key half that is entirely masked (the diagonal block's upper half for the tile's first 32
// queries, every block when s <= 32) keeps m = -inf, and its probabilities are taken as 0, not exp2(-inf + inf).
//
// Two workgroups share a CU (LDS), so four waves share a SIMD; the kernel asks the compiler for that register budget
// (128), which the d = 128 instance otherwise overran (136 registers, one workgroup per CU; grouped-query shape,
// per rank: 77 -> 63 us).  Measured slower at d = 96: computing the next block's scores ahead of this block's softmax
// (52 against 50 us), and splitting the key range of the heaviest causal tiles over two workgroups merged by a
// second kernel (49 us + 12 us of merge against 53 us).
template <int DP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void attn_fwd_bf16_ks_kernel(AttnParams p) {
  constexpr int CH = DP / 8;
  constexpr int TILE_B = KT * CH * 16;
  constexpr int STAGE_B = 2 * TILE_B;
  constexpr int CPW = CH / 4;   // copies per copying wave per tile and operand
  constexpr int NC = 2 * CPW;   // copies per copying wave per block
  constexpr int NDS = DP / 32;
  constexpr int NST = DP / 16;
  constexpr int NS = kv_stages<DP>();
  constexpr int MREC = NST * 4 + 2;  // merge record per lane: O (NST x 4), m, l
  static_assert(4 * 64 * MREC * 4 <= NS * STAGE_B, "merge records fit in the ring");
  __shared__ __attribute__((aligned(16))) char lds[NS * STAGE_B];
  constexpr int D = NS - 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4;
  const int l16 = lane & 15;
  const int qw = wave & 3, kh = wave >> 2;
  const int nq = (p.s + QT - 1) / QT;
  const int nbh = p.b * p.hl;
  const int qtile = nq - 1 - work_rank((int)blockIdx.x / nbh, nq, p.fold);
  const int bh = (int)blockIdx.x % nbh;
  const int bidx = bh / p.hl, jj = bh % p.hl;
  const int d = p.d;
  const QkvCols cols = qkv_cols(p.hl, p.G, d, jj);
  const int64_t ldq = cols.ld;
  const int64_t tok_stride = ldq * p.b;
  const uint16_t* __restrict__ qkv = static_cast<const uint16_t*>(p.qkv) + (int64_t)bidx * ldq + cols.q;
  const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(p.qkv) + (int64_t)bidx * ldq + cols.k;

  const int q = qtile * QT + qw * 16 + l16;
  bf16x8_t qf[NDS];
#pragma unroll
  for (int u = 0; u < NDS; ++u) {
    const int dd = 32 * u + 8 * g;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (q < p.s && dd < d) v = *reinterpret_cast<const uint4*>(qkv + (int64_t)q * tok_stride + dd);
    qf[u] = __builtin_bit_cast(bf16x8_t, v);
  }
  settle(qf);

  const int nkt_all = (p.s + KT - 1) / KT;
  const int nkt = p.causal ? min(nkt_all, qtile + 1) : nkt_all;
  const int klim = p.causal ? min(q, p.s - 1) : p.s - 1;

  // copies (kh = 0 waves): copy c of a tile fills LDS chunks 64 c .. 64 c + 63; wave qw issues copies qw + 4 i
  int crow[CPW], ccol[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int P = (qw + 4 * i) * 64 + lane;
    const int r = P / CH, slot = P % CH;
    const int c = tile_chunk<CH>(r, slot);
    crow[i] = r;
    ccol[i] = (c * 8 < d) ? c * 8 : 0;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)&lds[0];
  // this lane's byte offset of copy i within a key tile (the keys; the values at 2 d bytes further), from the
  // tile's first key row; whole tiles move only the wave-uniform base
  uint32_t coff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) coff[i] = (uint32_t)(((int64_t)crow[i] * tok_stride + ccol[i]) * 2);
  const bool off32 = (int64_t)KT * tok_stride * 2 < (int64_t)1 << 32;
  const int64_t tile_elems = (int64_t)KT * tok_stride;
  auto issue_tile = [&](int kt, int st) {
    if (kh != 0) return;
    const int ktc = min(kt, nkt - 1);
    const int kv0 = ktc * KT;
    const uint32_t sb = lds0 + st * STAGE_B;
    if (kv0 + KT <= p.s && off32) {  // every row of the tile exists: no per-row clamp
      const uint16_t* tb = kbase + (int64_t)ktc * tile_elems;
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const uint32_t dst = sb + (qw + 4 * i) * 1024;
        dma16s(tb, coff[i], dst);
        dma16s(tb + d, coff[i], dst + TILE_B);
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int row = min(kv0 + crow[i], p.s - 1);
        const uint16_t* src = kbase + (int64_t)row * tok_stride + ccol[i];
        const uint32_t dst = sb + (qw + 4 * i) * 1024;
        dma16(src, __builtin_amdgcn_readfirstlane(dst));
        dma16(src + d, __builtin_amdgcn_readfirstlane(dst + TILE_B));
      }
    }
  };
  auto chunk_off = [&](int r, int c) { return r * CH * 16 + tile_chunk<CH>(r, c) * 16; };
  int koff[2][NDS];  // this wave's two 16-key subtiles 2 kh, 2 kh + 1
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int u = 0; u < NDS; ++u) koff[i][u] = chunk_off(16 * (2 * kh + i) + l16, 4 * u + g);
  int voff[NST][2];  // V^T fragments of this wave's 32-key step
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int R = 32 * kh + 16 * hh + 4 * g + (l16 >> 2);
      const int dc = 16 * st + 4 * (l16 & 3);
      voff[st][hh] = chunk_off(R, dc >> 3) + ((dc >> 2) & 1) * 8;
    }

  const float c2 = p.scale * 1.4426950408889634f;
  const float thr = 8.f / c2;  // a rise of 2^8 in the exp2 domain, in score units
  // m_thr = m_run + thr and nm = -m_run c2 (0 while m_run = -inf) change only with m_run
  float m_run = -INFINITY, l_part = 0.f, m_thr = -INFINITY, nm = 0.f;
  f32x4_t acc_o[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) acc_o[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < D; ++i) issue_tile(i, i);
  wait_vmcnt<(D - 1) * NC>();
  __syncthreads();

  auto block = [&](int kt, auto stage) {
    constexpr int st_cur = decltype(stage)::value;
    constexpr int st_new = (st_cur + D) % NS;
    issue_tile(kt + D, st_new);
    const char* Kt = &lds[st_cur * STAGE_B];
    const char* Vt = Kt + TILE_B;
    const int kv0 = kt * KT + 32 * kh;  // this wave's first key

    bf16x8_t kfr[2][NDS];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int u = 0; u < NDS; ++u) kfr[i][u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(Kt + koff[i][u]));
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t sc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NDS; ++u) sc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr[i][u], qf[u], sc[i], 0, 0, 0);
    }
    // the V fragments are read only once the K fragments are dead (their latency hides under the softmax)
    if constexpr (DP >= 128) __builtin_amdgcn_sched_barrier(0);
    bf16x8_t vfr[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(Vt + voff[st][0]));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(Vt + voff[st][1]));
      const v8i16_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      vfr[st] = __builtin_bit_cast(bf16x8_t, w);
    }
    __builtin_amdgcn_sched_barrier(0);
    if ((p.causal && kt == qtile) || (kt * KT + KT > p.s)) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[i][e] = (kv0 + i * 16 + 4 * g + e > klim) ? -INFINITY : sc[i][e];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[i][e]);
    mx = max_over_groups(mx);
    const float m_new = max2(m_run, mx);
    // lazy rescale: the running maximum moves (and the sums are rescaled) only when some row's maximum rose by more
    // than 2^8 in the exp2 domain; until then probabilities of up to 2^8 are taken against the kept maximum, which
    // the sum and the output share, so the result is the same up to rounding (and the first finite maximum always
    // moves it: -inf to finite is an infinite rise)
    if (__any(m_new > m_thr)) {
      const float corr = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      l_part *= corr;
#pragma unroll
      for (int st = 0; st < NST; ++st) acc_o[st] *= corr;
      m_run = m_new;
      m_thr = m_run + thr;
      nm = m_run == -INFINITY ? 0.f : -m_run * c2;  // a fully masked half: every p is exp2(-inf) = 0
    }
    float psum = 0.f;
    uint32_t pk[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = __builtin_amdgcn_exp2f(fmaf(sc[i][e], c2, nm));
        psum += pe[e];
      }
      pk[i][0] = pack_bf16x2_hw(pe[0], pe[1]);
      pk[i][1] = pack_bf16x2_hw(pe[2], pe[3]);
    }
    l_part += psum;
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]));
#pragma unroll
    for (int st = 0; st < NST; ++st) acc_o[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr[st], pf, acc_o[st], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // the wait and the barrier after the products are issued
    wait_vmcnt<(D - 1) * NC>();
    __syncthreads();
  };
  for (int kt = 0; kt < nkt; kt += NS) {
    block(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nkt) block(kt + 1, std::integral_constant<int, 1>{});
    if constexpr (NS > 2) {
      if (kt + 2 < nkt) block(kt + 2, std::integral_constant<int, 2 % NS>{});
    }
  }
  wait_vmcnt<0>();
  __syncthreads();  // every copy has landed and every read of the ring is done: it holds the merge records now

  float* rec = reinterpret_cast<float*>(lds) + (qw * 64 + lane) * MREC;
  if (kh == 1) {
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) rec[st * 4 + e] = acc_o[st][e];
    rec[NST * 4] = m_run;
    rec[NST * 4 + 1] = l_part;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m1 = rec[NST * 4], l1 = rec[NST * 4 + 1];
  const float m = fmaxf(m_run, m1);  // m_run is finite: key 0 is visible to every query in block 0
  const float f0 = __builtin_amdgcn_exp2f((m_run - m) * c2), f1 = __builtin_amdgcn_exp2f((m1 - m) * c2);
  const float l_tot = sum_over_groups(l_part * f0 + l1 * f1);
  if (q < p.s) {
    const float inv = 1.f / l_tot;
    uint16_t* o = static_cast<uint16_t*>(p.o) + ((int64_t)q * p.b + bidx) * ((int64_t)p.hl * d) + (int64_t)jj * d;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int dd = st * 16 + 4 * g;
      if (dd < d) {
        float ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (acc_o[st][e] * f0 + rec[st * 4 + e] * f1) * inv;
        uint2 w;
        w.x = pack_bf16x2_hw(ov[0], ov[1]);
        w.y = pack_bf16x2_hw(ov[2], ov[3]);
        *reinterpret_cast<uint2*>(o + dd) = w;
      }
    }
    if (p.lse != nullptr && g == 0)
      p.lse[((int64_t)bidx * p.hl + jj) * p.s + q] = (m * c2 + log2f(l_tot)) * 0.69314718055994531f;
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
  const QkvCols cols = qkv_cols(p.hl, p.G, d, jj);
  const int64_t ldq = cols.ld;
  const int64_t tok = ldq * p.b;
  const float* base = static_cast<const float*>(p.qkv) + (int64_t)bidx * ldq;
  const float* qv = base + cols.q + (int64_t)q * tok;
  float o[DMAX];
  for (int e = 0; e < d; ++e) o[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int nk = p.causal ? q + 1 : p.s;
  for (int k = 0; k < nk; ++k) {
    const float* kv = base + cols.k + (int64_t)k * tok;  // K at kv, V at kv + d
    float sdot = 0.f;
    for (int e = 0; e < d; ++e) sdot = fmaf(qv[e], kv[e], sdot);
    const float x = sdot * p.scale;
    const float mn = fmaxf(m, x);
    const float corr = expf(m - mn);
    const float pe = expf(x - mn);
    l = l * corr + pe;
    for (int e = 0; e < d; ++e) o[e] = o[e] * corr + pe * kv[d + e];
    m = mn;
  }
  float* out = static_cast<float*>(p.o) + ((int64_t)q * p.b + bidx) * ((int64_t)p.hl * d) + (int64_t)jj * d;
  for (int e = 0; e < d; ++e) out[e] = o[e] / l;
  if (p.lse != nullptr) p.lse[((int64_t)bidx * p.hl + jj) * p.s + q] = m + logf(l);
}

// ================================================================================================================
// Backward.  With P = exp(S scale - lse) recomputed from the forward's log-sum-exp and D[q] = sum_e dO[q,e] O[q,e]
// (equal to the row sum of P * dP, since O = P V): dV = P^T dO, dS = P * (dO V^T - D), dQ = dS K scale,
// dK = dS^T Q scale.  Two kernels share no accumulators, so no atomics and the results are deterministic:
//   * dK, dV: one workgroup = 64 keys of one (batch, head), 4 waves x 16 keys, walking the 64-query blocks that
//     see them (causal: from the diagonal block on); Q, dO tiles and the blocks' (lse, D) record come by direct
//     copies into a 3-stage ring.  S = Q K^T and dP = dO V^T take Q / dO rows from LDS and the wave's K / V
//     fragments from registers; dV^T += dO^T P and dK^T += Q^T dS read dO^T and Q^T with transposing LDS reads
//     whose row addresses follow the query order of the P / dS operand (the forward's V trick).
//   * dQ, run first: 64 queries per workgroup, 4 waves x 16, K and V tiles in the ring: S^T = K Q^T,
//     dP^T = V dO^T, and with K^T gathered by transposing reads A^T += K^T (P dP)^T, B^T += K^T P^T and
//     D += sum_k P dP, so dQ = (A - D B) scale comes out of one walk over the keys; D is written to the record.
// ================================================================================================================

// Per (batch, head, 64-query block) record: [-lse log2 e (64) | D (64) | padding (128)], read by the dK / dV pass.
// The fp32 backward's is written here, with D from the stored fp32 O (as good as the row sum of P dP); the bf16
// backward's by its dQ kernel, which gets D from its own walk over the keys (attn_bwd_dq_bf16_kernel).
__global__ __launch_bounds__(256) void attn_bwd_prep_f32_kernel(AttnBwdParams p) {
  const int nqb = (p.s + 63) / 64;
  const int rec_id = blockIdx.x;  // bh * nqb + qb
  const int bh = rec_id / nqb, qb = rec_id % nqb;
  const int bidx = bh / p.hl, jj = bh % p.hl;
  const int t = threadIdx.x;
  float* rec = p.rec + (int64_t)rec_id * 256;
  if (t < 64) {
    const int q = qb * 64 + t;
    rec[t] = q < p.s ? -p.lse[(int64_t)bh * p.s + q] * 1.4426950408889634f : 0.f;
  } else if (t < 128) {
    const int q = qb * 64 + (t - 64);
    float acc = 0.f;
    if (q < p.s) {
      const int64_t off = ((int64_t)q * p.b + bidx) * ((int64_t)p.hl * p.d) + (int64_t)jj * p.d;
      const float* dO = static_cast<const float*>(p.dout) + off;
      const float* O = static_cast<const float*>(p.o) + off;
      for (int e = 0; e < p.d; ++e) acc = fmaf(dO[e], O[e], acc);
    }
    rec[t] = acc;
  } else {
    rec[t] = 0.f;
  }
}

template <int DP>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkv_bf16_kernel(AttnBwdParams p) {
  constexpr int CH = DP / 8;
  constexpr int TILE_B = 64 * CH * 16;          // one Q (or dO) tile
  constexpr int STAGE_B = 2 * TILE_B + 1024;    // Q tile, dO tile, (lse, D) record
  constexpr int CPW = CH / 4;
  constexpr int NDS = DP / 32, NST = DP / 16;
  constexpr int NS = dkv_stages<DP>();
  constexpr int D = NS - 1;  // query blocks in flight ahead of the one being used
  __shared__ __attribute__((aligned(16))) char lds[NS * STAGE_B];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4;
  const int l16 = lane & 15;
  const int nqb = (p.s + 63) / 64;
  // one workgroup per (64-key block, batch, local KV group, head split): split sp walks query heads
  // sp*HS .. sp*HS + HS - 1 of the group (HS = G / splits) and, with more than one split, writes fp32 partial dK / dV
  // that attn_bwd_kv_sum_kernel adds up in split order
  const int gl = p.hl / p.G;
  const int splits = p.kvpart != nullptr ? p.G : 1;
  const int HS = p.G / splits;
  const int nbh = p.b * gl * splits;
  const int ktile = work_rank((int)blockIdx.x / nbh, nqb, p.fold);  // key block 0 sees the most queries
  const int bh = (int)blockIdx.x % nbh;
  const int sp = bh % splits;
  const int bidx = bh / splits / gl, jg = bh / splits % gl;
  const int d = p.d;
  const QkvCols kc = qkv_cols(p.hl, p.G, d, jg * p.G);
  const int64_t ldq = kc.ld;
  const int64_t tok_stride = ldq * p.b;
  const int64_t ldo = (int64_t)p.hl * d * p.b;  // dO row stride (consecutive sequence positions)
  const uint16_t* __restrict__ qkv0 = static_cast<const uint16_t*>(p.qkv) + (int64_t)bidx * ldq;
  const uint16_t* __restrict__ kvb = qkv0 + kc.k;  // the group's K, V at + d
  const uint16_t* __restrict__ dob0 = static_cast<const uint16_t*>(p.dout) + (int64_t)bidx * p.hl * d;

  // ---- this lane's key: K and V fragments (k = d: lane supplies d = 32u + 8g .. +8)
  const int key = ktile * 64 + wave * 16 + l16;
  bf16x8_t kf[NDS], vf[NDS];
#pragma unroll
  for (int u = 0; u < NDS; ++u) {
    const int dd = 32 * u + 8 * g;
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
    if (key < p.s && dd < d) {
      a = *reinterpret_cast<const uint4*>(kvb + (int64_t)key * tok_stride + dd);
      b = *reinterpret_cast<const uint4*>(kvb + (int64_t)key * tok_stride + d + dd);
    }
    kf[u] = __builtin_bit_cast(bf16x8_t, a);
    vf[u] = __builtin_bit_cast(bf16x8_t, b);
  }
  settle(kf);
  settle(vf);
  const int qb0 = p.causal ? ktile : 0;
  const int nblk = nqb - qb0;
  const int ntot = HS * nblk;  // (query head of the split, query block) steps, head by head

  // ---- copies (same chunk layout as the forward's K / V tiles); wave 0 also copies the block's record
  int crow[CPW], ccol[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int P = (wave + 4 * i) * 64 + lane;
    const int r = P / CH, slot = P % CH;
    const int c = tile_chunk<CH>(r, slot);
    crow[i] = r;
    ccol[i] = (c * 8 < d) ? c * 8 : 0;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)&lds[0];
  // this lane's byte offsets of copy c within a full 64-query tile of Q and of dO, from the tile's first row
  uint32_t qoff[CPW], doff[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    qoff[c] = (uint32_t)(((int64_t)crow[c] * tok_stride + ccol[c]) * 2);
    doff[c] = (uint32_t)(((int64_t)crow[c] * ldo + ccol[c]) * 2);
  }
  const bool off32 = (int64_t)64 * (tok_stride > ldo ? tok_stride : ldo) * 2 < (int64_t)1 << 32;
  // Q columns of the split's first query head (the group's heads follow d apart: qkv_cols)
  const uint16_t* __restrict__ qh0 = qkv0 + kc.q + (int64_t)sp * HS * d;
  // steps are copied in order, head by head: the next one's head within the split and query block, and its index
  int cp_hs = 0, cp_qb = qb0, cp_i = 0;
  auto issue_tile = [&](int st) {
    const int hs = cp_hs, qb = cp_qb;
    if (cp_i + 1 < ntot) {  // past the last step: a harmless re-copy of it
      ++cp_i;
      if (++cp_qb == nqb) {
        cp_qb = qb0;
        ++cp_hs;
      }
    }
    const int jh = jg * p.G + sp * HS + hs;  // the step's query head
    const uint16_t* qsrc = qh0 + (int64_t)hs * d;
    const uint16_t* dsrc = dob0 + (int64_t)jh * d;
    const float* rsrc = p.rec + ((int64_t)(bidx * p.hl + jh) * nqb + qb) * 256;
    const uint32_t sb = lds0 + st * STAGE_B;
    if (qb * 64 + 64 <= p.s && off32) {  // every row of the tile exists
      const uint16_t* qt = qsrc + (int64_t)qb * 64 * tok_stride;
      const uint16_t* dt = dsrc + (int64_t)qb * 64 * ldo;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const uint32_t dst = sb + (wave + 4 * c) * 1024;
        dma16s(qt, qoff[c], dst);
        dma16s(dt, doff[c], dst + TILE_B);
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int row = min(qb * 64 + crow[c], p.s - 1);
        const uint32_t dst = sb + (wave + 4 * c) * 1024;
        dma16(qsrc + (int64_t)row * tok_stride + ccol[c], __builtin_amdgcn_readfirstlane(dst));
        dma16(dsrc + (int64_t)row * ldo + ccol[c], __builtin_amdgcn_readfirstlane(dst + TILE_B));
      }
    }
    if (wave == 0) dma16s(rsrc, (uint32_t)lane * 16u, sb + 2 * TILE_B);
  };
  auto chunk_off = [&](int r, int c) { return r * CH * 16 + tile_chunk<CH>(r, c) * 16; };
  int roff[4][NDS];  // A fragments of Q / dO rows (queries 16 qs + l16), d = 32u + 8g
#pragma unroll
  for (int qs = 0; qs < 4; ++qs)
#pragma unroll
    for (int u = 0; u < NDS; ++u) roff[qs][u] = chunk_off(16 * qs + l16, 4 * u + g);
  int toff[2][NST][2];  // transposing reads: rows = queries in the P / dS operand's order, columns = d
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int R = 32 * u + 16 * hh + 4 * g + (l16 >> 2);
        const int dc = 16 * st + 4 * (l16 & 3);
        toff[u][st][hh] = chunk_off(R, dc >> 3) + ((dc >> 2) & 1) * 8;
      }
  auto trfrag = [&](const char* base, int u, int st) {
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + toff[u][st][0]));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + toff[u][st][1]));
    const v8i16_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, w);
  };

  const float c2 = p.scale * 1.4426950408889634f;
  f32x4_t dv[NST], dk[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) dv[st] = dk[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < D; ++i) issue_tile(i);
  // step 0 has landed (wave 0 also copies the record: one more copy per step)
  if (wave == 0) wait_vmcnt<(D - 1) * (2 * CPW + 1)>(); else wait_vmcnt<(D - 1) * 2 * CPW>();
  __syncthreads();

  // one query block; the ring stage is a template constant, as in the forward
  int cur_qb = qb0;  // the query block of the step being multiplied
  auto step = [&](int i, auto stage) {
    constexpr int st_cur = decltype(stage)::value;
    constexpr int st_new = (st_cur + D) % NS;
    issue_tile(st_new);  // step i + D
    const char* Qt = &lds[st_cur * STAGE_B];
    const char* Dt = Qt + TILE_B;
    const float* R = reinterpret_cast<const float*>(Qt + 2 * TILE_B);
    const int qbi = cur_qb;
    if (++cur_qb == nqb) cur_qb = qb0;
    const int q0 = qbi * 64;

    // S and dP in two halves of 32 queries, each half's Q and dO fragments read before its MFMAs (as in dQ)
    f32x4_t sc[4], dp[4];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      bf16x8_t qa[2][NDS], da[2][NDS];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int u = 0; u < NDS; ++u) {
          qa[i][u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(Qt + roff[2 * hq + i][u]));
          da[i][u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(Dt + roff[2 * hq + i][u]));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int qs = 2 * hq + i;
        sc[qs] = dp[qs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NDS; ++u) {
          sc[qs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[i][u], kf[u], sc[qs], 0, 0, 0);
          dp[qs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[i][u], vf[u], dp[qs], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // P and dS for queries q0 + 16 qs + 4 g + e and this lane's key; masked scores become -inf (P = 0), in a
    // branch of their own that only the diagonal block and a ragged last block take
    const bool diag = p.causal && qbi == ktile;
    const bool ragged = q0 + 64 > p.s;
    if (diag || ragged) {
#pragma unroll
      for (int qs = 0; qs < 4; ++qs)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q = q0 + 16 * qs + 4 * g + e;
          if (q >= p.s || (p.causal && key > q)) sc[qs][e] = -INFINITY;
        }
    }
    // P goes to the matrix cores as a bf16 pair hi + lo (lo = P - hi rounded again): with near-uniform weights
    // a single bf16 P carries 2^-9 relative error into every term of dV's sum over queries
    uint32_t pp[4][2], pl[4][2], dd2[4][2], dl2[4][2];
#pragma unroll
    for (int qs = 0; qs < 4; ++qs) {
      const f32x4_t nl4 = *reinterpret_cast<const f32x4_t*>(R + 16 * qs + 4 * g);  // -lse log2 e
      const f32x4_t D4 = *reinterpret_cast<const f32x4_t*>(R + 64 + 16 * qs + 4 * g);
      float pe[4], ds[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = __builtin_amdgcn_exp2f(fmaf(sc[qs][e], c2, nl4[e]));
        ds[e] = pe[e] * (dp[qs][e] - D4[e]);
      }
      split_hi_lo(pe, pp[qs], pl[qs]);
      split_hi_lo(ds, dd2[qs], dl2[qs]);
    }
    // dV^T += dO^T P, dK^T += Q^T dS over two 32-query steps (P and dS as hi + lo bf16 pairs)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pp[2 * u][0], pp[2 * u][1], pp[2 * u + 1][0], pp[2 * u + 1][1]));
      const bf16x8_t plf = __builtin_bit_cast(bf16x8_t, make_uint4(pl[2 * u][0], pl[2 * u][1], pl[2 * u + 1][0], pl[2 * u + 1][1]));
      const bf16x8_t sf = __builtin_bit_cast(bf16x8_t, make_uint4(dd2[2 * u][0], dd2[2 * u][1], dd2[2 * u + 1][0], dd2[2 * u + 1][1]));
      const bf16x8_t slf = __builtin_bit_cast(bf16x8_t, make_uint4(dl2[2 * u][0], dl2[2 * u][1], dl2[2 * u + 1][0], dl2[2 * u + 1][1]));
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const bf16x8_t dot = trfrag(Dt, u, st);
        dv[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dot, pf, dv[st], 0, 0, 0);
        dv[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dot, plf, dv[st], 0, 0, 0);
        const bf16x8_t qt = trfrag(Qt, u, st);
        dk[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt, sf, dk[st], 0, 0, 0);
        dk[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt, slf, dk[st], 0, 0, 0);
      }
    }
    if (wave == 0) wait_vmcnt<(D - 1) * (2 * CPW + 1)>(); else wait_vmcnt<(D - 1) * 2 * CPW>();
    __syncthreads();
  };
  for (int i0 = 0; i0 < ntot; i0 += NS) {
    step(i0, std::integral_constant<int, 0>{});
    if (i0 + 1 < ntot) step(i0 + 1, std::integral_constant<int, 1>{});
    if constexpr (NS > 2) {
      if (i0 + 2 < ntot) step(i0 + 2, std::integral_constant<int, 2 % NS>{});
    }
  }
  wait_vmcnt<0>();

  if (key < p.s && splits > 1) {
    // partial [split][token row][local group][dK (scaled) | dV], fp32
    float* part = p.kvpart + (((int64_t)sp * p.s * p.b + (int64_t)key * p.b + bidx) * gl + jg) * 2 * d;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int dd = st * 16 + 4 * g;
      if (dd < d) {
        *reinterpret_cast<f32x4_t*>(part + dd) = f32x4_t{dk[st][0] * p.scale, dk[st][1] * p.scale,
                                                          dk[st][2] * p.scale, dk[st][3] * p.scale};
        *reinterpret_cast<f32x4_t*>(part + d + dd) = dv[st];
      }
    }
  } else if (key < p.s) {
    uint16_t* out = static_cast<uint16_t*>(p.dqkv) + ((int64_t)key * p.b + bidx) * ldq + kc.k;  // dK; dV at + d
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int dd = st * 16 + 4 * g;
      if (dd < d) {
        uint2 w;
        w.x = pack_bf16x2_hw(dk[st][0] * p.scale, dk[st][1] * p.scale);
        w.y = pack_bf16x2_hw(dk[st][2] * p.scale, dk[st][3] * p.scale);
        *reinterpret_cast<uint2*>(out + dd) = w;
        w.x = pack_bf16x2_hw(dv[st][0], dv[st][1]);
        w.y = pack_bf16x2_hw(dv[st][2], dv[st][3]);
        *reinterpret_cast<uint2*>(out + d + dd) = w;
      }
    }
  }
}

// dQ without knowing D first: dQ = sum_k P (dP - D) K = A - D B with A = sum_k (P dP) K, B = sum_k P K and
// D = sum_k P dP, all three gathered in the one walk over the keys (P dP and P reach the matrix cores as bf16
// hi + lo pairs; with a single bf16 B the difference A - D B loses about 3e-2 of dQ's scale).  D goes into the
// record for the dK / dV pass, which runs after this one.  Taking D as the row sum of dO * O instead would use the
// forward's bf16-rounded O, whose rounding reaches every element of dS = P * (dP - D).
template <int DP>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_bf16_kernel(AttnBwdParams p) {
  constexpr int CH = DP / 8;
  constexpr int TILE_B = KT * CH * 16;
  constexpr int STAGE_B = 2 * TILE_B;   // K tile then V tile
  constexpr int CPW = CH / 4;
  constexpr int NC = 2 * CPW;
  constexpr int NDS = DP / 32, NST = DP / 16;
  constexpr int NS = kv_stages<DP>();
  constexpr int D = NS - 1;  // blocks in flight ahead of the one being multiplied
  __shared__ __attribute__((aligned(16))) char lds[NS * STAGE_B];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 4;
  const int l16 = lane & 15;
  const int nq = (p.s + QT - 1) / QT;
  const int nbh = p.b * p.hl;
  const int qtile = nq - 1 - work_rank((int)blockIdx.x / nbh, nq, p.fold);
  const int bh = (int)blockIdx.x % nbh;
  const int bidx = bh / p.hl, jj = bh % p.hl;
  const int d = p.d;
  const QkvCols cols = qkv_cols(p.hl, p.G, d, jj);
  const int64_t ldq = cols.ld;
  const int64_t tok_stride = ldq * p.b;
  const uint16_t* __restrict__ qkv = static_cast<const uint16_t*>(p.qkv) + (int64_t)bidx * ldq + cols.q;
  const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(p.qkv) + (int64_t)bidx * ldq + cols.k;

  // ---- this lane's query: Q and dO fragments, lse (log2 units) and D
  const int q = qtile * QT + wave * 16 + l16;
  bf16x8_t qf[NDS], df[NDS];
#pragma unroll
  for (int u = 0; u < NDS; ++u) {
    const int dd = 32 * u + 8 * g;
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
    if (q < p.s && dd < d) {
      a = *reinterpret_cast<const uint4*>(qkv + (int64_t)q * tok_stride + dd);
      b = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.dout) +
                                          ((int64_t)q * p.b + bidx) * ((int64_t)p.hl * d) + (int64_t)jj * d + dd);
    }
    qf[u] = __builtin_bit_cast(bf16x8_t, a);
    df[u] = __builtin_bit_cast(bf16x8_t, b);
  }
  const float lse2 = q < p.s ? p.lse[(int64_t)bh * p.s + q] * 1.4426950408889634f : 0.f;
  settle(qf);
  settle(df);
  asm volatile("" ::"v"(lse2));
  float* const drec = p.rec + ((int64_t)bh * ((p.s + 63) / 64) + q / 64) * 256 + 64 + (q % 64);
  float dsum = 0.f;

  const int nkt_all = (p.s + KT - 1) / KT;
  const int nkt = p.causal ? min(nkt_all, qtile + 1) : nkt_all;

  int crow[CPW], ccol[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int P = (wave + 4 * i) * 64 + lane;
    const int r = P / CH, slot = P % CH;
    const int c = tile_chunk<CH>(r, slot);
    crow[i] = r;
    ccol[i] = (c * 8 < d) ? c * 8 : 0;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)&lds[0];
  // this lane's byte offset of copy i within a full key tile (the keys; the values at 2 d bytes further)
  uint32_t coff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) coff[i] = (uint32_t)(((int64_t)crow[i] * tok_stride + ccol[i]) * 2);
  const bool off32 = (int64_t)KT * tok_stride * 2 < (int64_t)1 << 32;
  auto issue_tile = [&](int kt, int st) {
    const int ktc = min(kt, nkt - 1);
    const int kv0 = ktc * KT;
    const uint32_t sb = lds0 + st * STAGE_B;
    if (kv0 + KT <= p.s && off32) {  // every row of the tile exists
      const uint16_t* tb = kbase + (int64_t)kv0 * tok_stride;
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const uint32_t dst = sb + (wave + 4 * i) * 1024;
        dma16s(tb, coff[i], dst);
        dma16s(tb + d, coff[i], dst + TILE_B);
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int row = min(kv0 + crow[i], p.s - 1);
        const uint16_t* src = kbase + (int64_t)row * tok_stride + ccol[i];
        const uint32_t dst = sb + (wave + 4 * i) * 1024;
        dma16(src, __builtin_amdgcn_readfirstlane(dst));
        dma16(src + d, __builtin_amdgcn_readfirstlane(dst + TILE_B));
      }
    }
  };
  auto chunk_off = [&](int r, int c) { return r * CH * 16 + tile_chunk<CH>(r, c) * 16; };
  int koff[4][NDS];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int u = 0; u < NDS; ++u) koff[ks][u] = chunk_off(16 * ks + l16, 4 * u + g);
  int toff[2][NST][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int R = 32 * u + 16 * hh + 4 * g + (l16 >> 2);
        const int dc = 16 * st + 4 * (l16 & 3);
        toff[u][st][hh] = chunk_off(R, dc >> 3) + ((dc >> 2) & 1) * 8;
      }

  const float c2 = p.scale * 1.4426950408889634f;
  f32x4_t dq[NST], bq[NST];  // A^T and B^T
#pragma unroll
  for (int st = 0; st < NST; ++st) dq[st] = bq[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < D; ++i) issue_tile(i, i);
  wait_vmcnt<(D - 1) * NC>();  // block 0 has landed
  __syncthreads();

  // one key block; the ring stage is a template constant, as in the forward
  auto step = [&](int kt, auto stage) {
    constexpr int st_cur = decltype(stage)::value;
    constexpr int st_new = (st_cur + D) % NS;
    issue_tile(kt + D, st_new);
    const char* Kt = &lds[st_cur * STAGE_B];
    const char* Vt = Kt + TILE_B;
    const int kv0 = kt * KT;
    // S^T and dP^T in two halves of 32 keys: the half's K and V fragments are all read before its MFMAs, so only
    // the first MFMA waits on LDS (read one by one, each MFMA waited on the read just before it)
    f32x4_t sc[4], dp[4];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      bf16x8_t ka[2][NDS], va[2][NDS];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int u = 0; u < NDS; ++u) {
          ka[i][u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(Kt + koff[2 * hk + i][u]));
          va[i][u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(Vt + koff[2 * hk + i][u]));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ks = 2 * hk + i;
        sc[ks] = dp[ks] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NDS; ++u) {
          sc[ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i][u], qf[u], sc[ks], 0, 0, 0);
          dp[ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[i][u], df[u], dp[ks], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // masked scores become -inf (P = 0), in a branch of their own: the diagonal block and a ragged last block only
    if ((p.causal && kt == qtile) || (kv0 + KT > p.s)) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kv = kv0 + ks * 16 + 4 * g + e;
          if (kv >= p.s || (p.causal && kv > q)) sc[ks][e] = -INFINITY;
        }
    }
    uint32_t gh[4][2], gl[4][2], ph[4][2], pl[4][2];  // P dP and P as hi + lo bf16 pairs
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float gv[4], pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[ks][e], c2, -lse2));
        gv[e] = pv[e] * dp[ks][e];
        dsum += gv[e];
      }
      split_hi_lo(gv, gh[ks], gl[ks]);
      split_hi_lo(pv, ph[ks], pl[ks]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8_t gf = __builtin_bit_cast(bf16x8_t, make_uint4(gh[2 * u][0], gh[2 * u][1], gh[2 * u + 1][0], gh[2 * u + 1][1]));
      const bf16x8_t glf = __builtin_bit_cast(bf16x8_t, make_uint4(gl[2 * u][0], gl[2 * u][1], gl[2 * u + 1][0], gl[2 * u + 1][1]));
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(ph[2 * u][0], ph[2 * u][1], ph[2 * u + 1][0], ph[2 * u + 1][1]));
      const bf16x8_t plf = __builtin_bit_cast(bf16x8_t, make_uint4(pl[2 * u][0], pl[2 * u][1], pl[2 * u + 1][0], pl[2 * u + 1][1]));
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(Kt + toff[u][st][0]));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(Kt + toff[u][st][1]));
        const v8i16_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8_t kt_ = __builtin_bit_cast(bf16x8_t, w);
        dq[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt_, gf, dq[st], 0, 0, 0);
        dq[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt_, glf, dq[st], 0, 0, 0);
        bq[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt_, pf, bq[st], 0, 0, 0);
        bq[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt_, plf, bq[st], 0, 0, 0);
      }
    }
    wait_vmcnt<(D - 1) * NC>();  // block kt+1 has landed
    __syncthreads();
  };
  for (int kt0 = 0; kt0 < nkt; kt0 += NS) {
    step(kt0, std::integral_constant<int, 0>{});
    if (kt0 + 1 < nkt) step(kt0 + 1, std::integral_constant<int, 1>{});
    if constexpr (NS > 2) {
      if (kt0 + 2 < nkt) step(kt0 + 2, std::integral_constant<int, 2 % NS>{});
    }
  }
  wait_vmcnt<0>();

  dsum = sum_over_groups(dsum);  // D for this lane's query
  if (g == 0) {  // this query's record entries: -lse log2 e and D (zeros past the sequence, which dK / dV masks)
    drec[-64] = -lse2;
    *drec = q < p.s ? dsum : 0.f;
  }
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int e = 0; e < 4; ++e) dq[st][e] = fmaf(-dsum, bq[st][e], dq[st][e]);  // A - D B
  if (q < p.s) {
    uint16_t* out = static_cast<uint16_t*>(p.dqkv) + ((int64_t)q * p.b + bidx) * ldq + cols.q;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int dd = st * 16 + 4 * g;
      if (dd < d) {
        uint2 w;
        w.x = pack_bf16x2_hw(dq[st][0] * p.scale, dq[st][1] * p.scale);
        w.y = pack_bf16x2_hw(dq[st][2] * p.scale, dq[st][3] * p.scale);
        *reinterpret_cast<uint2*>(out + dd) = w;
      }
    }
  }
}

// fp32 backward: one thread per query (dQ) or per key (dK, dV), plain loops over the other side.
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(AttnBwdParams p) {
  constexpr int DMAX = 128;
  const int q = blockIdx.x * 64 + threadIdx.x;
  const int bh = blockIdx.y;
  const int bidx = bh / p.hl, jj = bh % p.hl;
  if (q >= p.s) return;
  const int d = p.d;
  const QkvCols cols = qkv_cols(p.hl, p.G, d, jj);
  const int64_t ldq = cols.ld, tok = ldq * p.b;
  const float* base = static_cast<const float*>(p.qkv) + (int64_t)bidx * ldq;
  const float* qv = base + cols.q + (int64_t)q * tok;
  const float* dov = static_cast<const float*>(p.dout) + ((int64_t)q * p.b + bidx) * ((int64_t)p.hl * d) + (int64_t)jj * d;
  const float lse = p.lse[(int64_t)bh * p.s + q];
  const float D = p.rec[((int64_t)bh * ((p.s + 63) / 64) + q / 64) * 256 + 64 + (q % 64)];
  float acc[DMAX];
  for (int e = 0; e < d; ++e) acc[e] = 0.f;
  const int nk = p.causal ? q + 1 : p.s;
  for (int k = 0; k < nk; ++k) {
    const float* kv = base + cols.k + (int64_t)k * tok;  // K at kv, V at kv + d
    float sdot = 0.f, dpv = 0.f;
    for (int e = 0; e < d; ++e) {
      sdot = fmaf(qv[e], kv[e], sdot);
      dpv = fmaf(dov[e], kv[d + e], dpv);
    }
    const float ds = expf(sdot * p.scale - lse) * (dpv - D);
    for (int e = 0; e < d; ++e) acc[e] = fmaf(ds, kv[e], acc[e]);
  }
  float* out = static_cast<float*>(p.dqkv) + ((int64_t)q * p.b + bidx) * ldq + cols.q;
  for (int e = 0; e < d; ++e) out[e] = acc[e] * p.scale;
}

__global__ __launch_bounds__(64) void attn_bwd_dkv_f32_kernel(AttnBwdParams p) {
  constexpr int DMAX = 128;
  const int k = blockIdx.x * 64 + threadIdx.x;
  const int gl = p.hl / p.G;  // one thread per (key, batch, local KV group); the group's query heads summed
  const int bh = blockIdx.y;
  const int bidx = bh / gl, jg = bh % gl;
  if (k >= p.s) return;
  const int d = p.d;
  const QkvCols kc = qkv_cols(p.hl, p.G, d, jg * p.G);
  const int64_t ldq = kc.ld, tok = ldq * p.b;
  const float* base = static_cast<const float*>(p.qkv) + (int64_t)bidx * ldq;
  const float* kv = base + kc.k + (int64_t)k * tok;  // K at kv, V at kv + d
  const int nqb = (p.s + 63) / 64;
  float dk[DMAX], dv[DMAX];
  for (int e = 0; e < d; ++e) dk[e] = dv[e] = 0.f;
  for (int hs = 0; hs < p.G; ++hs) {
    const int jh = jg * p.G + hs;
    const int64_t qcol = qkv_cols(p.hl, p.G, d, jh).q;
    const int64_t hrow = (int64_t)bidx * p.hl + jh;
    for (int q = p.causal ? k : 0; q < p.s; ++q) {
      const float* qv = base + qcol + (int64_t)q * tok;
      const float* dov = static_cast<const float*>(p.dout) + ((int64_t)q * p.b + bidx) * ((int64_t)p.hl * d) + (int64_t)jh * d;
      const float lse = p.lse[hrow * p.s + q];
      const float D = p.rec[(hrow * nqb + q / 64) * 256 + 64 + (q % 64)];
      float sdot = 0.f, dpv = 0.f;
      for (int e = 0; e < d; ++e) {
        sdot = fmaf(qv[e], kv[e], sdot);
        dpv = fmaf(dov[e], kv[d + e], dpv);
      }
      const float pe = expf(sdot * p.scale - lse);
      const float ds = pe * (dpv - D);
      for (int e = 0; e < d; ++e) {
        dv[e] = fmaf(pe, dov[e], dv[e]);
        dk[e] = fmaf(ds, qv[e], dk[e]);
      }
    }
  }
  float* out = static_cast<float*>(p.dqkv) + ((int64_t)k * p.b + bidx) * ldq + kc.k;
  for (int e = 0; e < d; ++e) {
    out[e] = dk[e] * p.scale;
    out[d + e] = dv[e];
  }
}

// dK | dV of every (token row, local KV group) = the sum of the head splits' fp32 partials, in split order, rounded
// once to bf16 into the group's key and value columns (adjacent in dQKV).  One thread per 4 columns.
__global__ __launch_bounds__(256) void attn_bwd_kv_sum_kernel(AttnBwdParams p) {
  const int gl = p.hl / p.G, d = p.d, w4 = d / 2;  // 2d columns per (row, group), in 4-column quads
  const int64_t rows = (int64_t)p.s * p.b;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * gl * w4) return;
  const int c4 = (int)(idx % w4);
  const int64_t rg = idx / w4;  // token row * gl + group
  const int jg = (int)(rg % gl);
  const int64_t m = rg / gl;
  const int64_t split_stride = rows * gl * 2 * d;
  const float* part = p.kvpart + rg * 2 * d + 4 * c4;
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(part);
  for (int sp = 1; sp < p.G; ++sp) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + sp * split_stride);
    acc[0] += v[0];
    acc[1] += v[1];
    acc[2] += v[2];
    acc[3] += v[3];
  }
  const QkvCols kc = qkv_cols(p.hl, p.G, d, jg * p.G);
  uint16_t* out = static_cast<uint16_t*>(p.dqkv) + m * kc.ld + kc.k + 4 * c4;
  uint2 w;
  w.x = pack_bf16x2_hw(acc[0], acc[1]);
  w.y = pack_bf16x2_hw(acc[2], acc[3]);
  *reinterpret_cast<uint2*>(out) = w;
}

// Workgroups of Kernel (256 threads) resident on the current device at once; 0 when the runtime cannot say.  A
// template on the kernel itself, so each kernel has its own cache (kernels of one signature share a type).
template <auto Kernel, int NT = 256>
int64_t resident_limit() {
  const void* const kernel = reinterpret_cast<const void*>(Kernel);
  constexpr int kMaxDevices = 64;
  static std::atomic<int64_t> cache[kMaxDevices];  // 0: not yet asked
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    // the runtime's occupancy figure, capped by the LDS count (the runtime has reported 2 per CU for kernels of
    // 96 KB of static LDS on a 160 KB CU)
    int per_cu = 0, cus = 0, lds_cu = 0;
    hipFuncAttributes fa;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, NT, 0) != hipSuccess ||
        hipFuncGetAttributes(&fa, kernel) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      per_cu = 0;
    } else if (fa.sharedSizeBytes > 0) {
      per_cu = std::min<int64_t>(per_cu, (int64_t)lds_cu / (int64_t)fa.sharedSizeBytes);
    }
    v = (int64_t)per_cu * cus + 1;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v - 1;
}

template <auto Kernel, int NT = 256>
int fold_for(unsigned grid, int causal) {
  return causal && (int64_t)grid <= resident_limit<Kernel, NT>() ? 1 : 0;
}

template <int DP>
hipError_t launch_bwd_bf16(const AttnBwdParams& p0, hipStream_t st) {
  AttnBwdParams p = p0;
  const int nq = (p.s + 63) / 64;
  const unsigned grid = (unsigned)(nq * p.b * p.hl);
  static const std::string n1 = "attn_bwd_dkv_bf16_d" + std::to_string(DP);
  static const std::string n2 = "attn_bwd_dq_bf16_d" + std::to_string(DP);
  const int splits = p.kvpart != nullptr ? p.G : 1;
  // one workgroup per (64 keys, batch, KV group, head split)
  const unsigned grid_kv = (unsigned)(nq * p.b * (p.hl / p.G) * splits);
  // dQ first: it also writes each query's D, which the dK / dV pass reads
  p.fold = fold_for<attn_bwd_dq_bf16_kernel<DP>>(grid, p.causal);
  hipError_t e = TP_LAUNCH(n2.c_str(), (attn_bwd_dq_bf16_kernel<DP>), dim3(grid), dim3(256), 0, st, p);
  p.fold = fold_for<attn_bwd_dkv_bf16_kernel<DP>>(grid_kv, p.causal);
  if (e == hipSuccess) e = TP_LAUNCH(n1.c_str(), (attn_bwd_dkv_bf16_kernel<DP>), dim3(grid_kv), dim3(256), 0, st, p);
  if (e == hipSuccess && splits > 1) {
    const int64_t n = (int64_t)p.s * p.b * (p.hl / p.G) * (p.d / 2);
    e = TP_LAUNCH("attn_bwd_kv_sum_bf16", attn_bwd_kv_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                  st, p);
  }

  return e;
}

template <int DP>
hipError_t launch_bf16(const AttnParams& p0, hipStream_t st) {
  AttnParams p = p0;
  const int nq = (p.s + QT - 1) / QT;
  const unsigned grid = (unsigned)(nq * p.b * p.hl);
  static const std::string name = "attn_fwd_bf16_d" + std::to_string(DP);
  p.fold = fold_for<attn_fwd_bf16_ks_kernel<DP>, 512>(grid, p.causal);
  return TP_LAUNCH(name.c_str(), (attn_fwd_bf16_ks_kernel<DP>), dim3(grid), dim3(512), 0, st, p);
}

}  // namespace

hipError_t attention_bf16(const AttnParams& p, hipStream_t st) {
  if (p.s <= 0 || p.b <= 0 || p.hl <= 0) return hipSuccess;
  if (p.d <= 32) return launch_bf16<32>(p, st);
  if (p.d <= 64) return launch_bf16<64>(p, st);
  if (p.d <= 96) return launch_bf16<96>(p, st);
  return launch_bf16<128>(p, st);
}

hipError_t attention_bwd(tp_dtype dt, const AttnBwdParams& p, hipStream_t st) {
  if (p.s <= 0 || p.b <= 0 || p.hl <= 0) return hipSuccess;
  const int nqb = (p.s + 63) / 64;
  hipError_t e;
  if (dt == TP_BF16) {  // the dQ kernel writes the records
    if (p.d <= 32) return launch_bwd_bf16<32>(p, st);
    if (p.d <= 64) return launch_bwd_bf16<64>(p, st);
    if (p.d <= 96) return launch_bwd_bf16<96>(p, st);
    return launch_bwd_bf16<128>(p, st);
  }
  e = TP_LAUNCH("attn_bwd_prep_f32", attn_bwd_prep_f32_kernel, dim3((unsigned)(nqb * p.b * p.hl)), dim3(256), 0, st,
                p);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((p.s + 63) / 64), (unsigned)(p.b * p.hl));
  const dim3 grid_kv((unsigned)((p.s + 63) / 64), (unsigned)(p.b * (p.hl / p.G)));
  e = TP_LAUNCH("attn_bwd_dkv_f32", attn_bwd_dkv_f32_kernel, grid_kv, dim3(64), 0, st, p);
  if (e == hipSuccess) e = TP_LAUNCH("attn_bwd_dq_f32", attn_bwd_dq_f32_kernel, grid, dim3(64), 0, st, p);
  return e;
}

hipError_t attention_f32(const AttnParams& p, hipStream_t st) {
  if (p.s <= 0 || p.b <= 0 || p.hl <= 0) return hipSuccess;
  return TP_LAUNCH("attn_fwd_f32", attn_fwd_f32_kernel, dim3((unsigned)((p.s + 63) / 64), (unsigned)(p.b * p.hl)),
                   dim3(64), 0, st, p);
}

}  // namespace tp
