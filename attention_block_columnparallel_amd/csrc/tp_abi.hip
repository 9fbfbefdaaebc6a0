// The C ABI of libtpshard: host-side validation of every argument (before any HIP call, so it is testable on a
// machine without a GPU) and the launch sequence of each entry point.  Divisibility rules follow the pages: the
// sequence dim must split evenly across the t ranks for the dim-0 split / gather / reduce-scatter
// ("Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" §1); output columns, input rows and heads must divide by
// t, and h = a * d (Megatron-LM visual reading, divisibility rules; §1 of the same atlas page for h = a * d).
#include <stdio.h>
#include <string.h>

#include "tp_common.h"

namespace {

thread_local int g_last_hip_error = 0;

struct TimingLog {
  hipEvent_t* starts = nullptr;
  hipEvent_t* stops = nullptr;
  int cap = 0;
  int n = 0;
  bool armed = false;
  bool open = false;  // a start was recorded for slot n
  char only[64] = {0};  // when non-empty, only launches whose name starts with this are recorded
  const char* names[4096];
};
thread_local TimingLog g_timing;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return TP_OK;
  g_last_hip_error = (int)e;
  return TP_E_HIP;
}

bool bad_dtype(tp_dtype dt) { return dt != TP_F32 && dt != TP_BF16; }
int64_t esize(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }

struct Buf {
  const void* p;
  int64_t bytes;
};

bool overlaps(const Buf& a, const Buf& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + (uintptr_t)a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + (uintptr_t)b.bytes;
  return a0 < b1 && b0 < a1;
}

// Any output overlapping any input, or two outputs overlapping each other.
bool any_alias(const Buf* outs, int no, const Buf* ins, int ni) {
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j)
      if (overlaps(outs[i], ins[j])) return true;
    for (int j = i + 1; j < no; ++j)
      if (overlaps(outs[i], outs[j])) return true;
  }
  return false;
}

bool misaligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p != nullptr && ((uintptr_t)p & 15u) != 0) return true;
  return false;
}

// 2^31 elements is the largest single tensor the kernels index with 32-bit row / column counts.
constexpr int64_t kMaxDim = (int64_t)1 << 31;

}  // namespace

namespace tp {
void timing_start(hipStream_t st, const char* name) {
  TimingLog& T = g_timing;
  T.open = false;
  if (!T.armed || T.n >= T.cap) return;
  if (T.only[0] != 0 && strncmp(name, T.only, strlen(T.only)) != 0) return;
  if (hipEventRecord(T.starts[T.n], st) == hipSuccess) T.open = true;
}
void timing_stop(hipStream_t st, const char* name) {
  TimingLog& T = g_timing;
  if (!T.open) return;
  T.open = false;
  if (hipEventRecord(T.stops[T.n], st) == hipSuccess) {
    if (T.n < (int)(sizeof(T.names) / sizeof(T.names[0]))) T.names[T.n] = name;
    ++T.n;
  }
}
}  // namespace tp

extern "C" {

int tp_timing_begin(hipEvent_t* starts, hipEvent_t* stops, int capacity) {
  if (starts == nullptr || stops == nullptr) return TP_E_NULL;
  if (capacity <= 0) return TP_E_SHAPE;
  TimingLog& T = g_timing;
  T.starts = starts;
  T.stops = stops;
  T.cap = capacity < 4096 ? capacity : 4096;
  T.n = 0;
  T.open = false;
  T.armed = true;
  return TP_OK;
}

int tp_timing_end(void) {
  g_timing.armed = false;
  return g_timing.n;
}

int tp_timing_filter(const char* prefix) {
  TimingLog& T = g_timing;
  if (prefix == nullptr) {
    T.only[0] = 0;
    return TP_OK;
  }
  const size_t n = strlen(prefix);
  if (n >= sizeof(T.only)) return TP_E_SHAPE;
  memcpy(T.only, prefix, n + 1);
  return TP_OK;
}

const char* tp_timing_kernel(int i) {
  if (i < 0 || i >= g_timing.n) return nullptr;
  return g_timing.names[i];
}

const char* tp_status_str(int status) {
  switch (status) {
    case TP_OK: return "ok";
    case TP_E_NULL: return "a required pointer is NULL";
    case TP_E_SHAPE: return "a size is non-positive or out of range";
    case TP_E_DIVISIBILITY: return "divisibility rule violated (s, ffn or heads not divisible by t, or h != a*d)";
    case TP_E_DTYPE: return "unknown dtype";
    case TP_E_RANK: return "rank outside [0, t)";
    case TP_E_ALIAS: return "an output buffer overlaps an input buffer";
    case TP_E_UNSUPPORTED: return "unsupported combination (activation/dtype, alignment or head dim)";
    case TP_E_HIP: return "HIP launch failed";
    case TP_E_SCRATCH: return "the call needs more scratch than the library's fixed no-allocation buffer holds";
    default: return "unknown status";
  }
}

int tp_last_hip_error(void) { return g_last_hip_error; }

int tp_abi_version(void) { return TPSHARD_ABI_VERSION; }

int tp_shard_weights(const tp_dims* dims, int rank, tp_wkind kind, tp_dtype dtype, const void* full, void* shard,
                     hipStream_t stream) {
  if (dims == nullptr || full == nullptr || shard == nullptr) return TP_E_NULL;
  const int64_t h = dims->h, t = dims->t, ffn = dims->ffn, a = dims->a, d = dims->d;
  const int64_t g = dims->g == 0 ? a : dims->g;  // KV heads (0: as many as query heads)
  const bool mlp = kind == TP_W_FC1 || kind == TP_W_FC1_GATE_UP || kind == TP_W_FC2 || kind == TP_B_FC1 ||
                   kind == TP_B_FC1_GATE_UP;
  const bool att = kind == TP_W_QKV || kind == TP_W_PROJ || kind == TP_B_QKV;
  if (!mlp && !att) return TP_E_UNSUPPORTED;
  if (t <= 0 || h <= 0 || (mlp && ffn <= 0) || (att && (a <= 0 || d <= 0 || g <= 0))) return TP_E_SHAPE;
  if (h >= kMaxDim || ffn >= kMaxDim) return TP_E_SHAPE;
  if (mlp && ffn % t != 0) return TP_E_DIVISIBILITY;
  if (att && (a % t != 0 || h != a * d || a % g != 0 || g % t != 0)) return TP_E_DIVISIBILITY;
  if (rank < 0 || rank >= t) return TP_E_RANK;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  const int64_t es = esize(dtype);
  const int64_t f_l = mlp ? ffn / t : 0, hl = att ? a / t : 0, ad = a * d;
  const int64_t gl = att ? g / t : 0, G = att ? a / g : 1;  // local KV groups, query heads per group
  int64_t rows = 0, full_cols = 0, shard_cols = 0;
  switch (kind) {
    case TP_W_FC1: rows = h; full_cols = ffn; shard_cols = f_l; break;
    case TP_W_FC1_GATE_UP: rows = h; full_cols = 2 * ffn; shard_cols = 2 * f_l; break;
    case TP_W_FC2: rows = ffn; full_cols = h; shard_cols = h; break;
    case TP_W_QKV: rows = h; full_cols = ad + 2 * g * d; shard_cols = (hl + 2 * gl) * d; break;
    case TP_W_PROJ: rows = ad; full_cols = h; shard_cols = h; break;
    case TP_B_FC1: rows = 1; full_cols = ffn; shard_cols = f_l; break;
    case TP_B_FC1_GATE_UP: rows = 1; full_cols = 2 * ffn; shard_cols = 2 * f_l; break;
    case TP_B_QKV: rows = 1; full_cols = ad + 2 * g * d; shard_cols = (hl + 2 * gl) * d; break;
  }
  const Buf out[] = {{shard, (kind == TP_W_FC2 ? f_l : kind == TP_W_PROJ ? hl * d : rows) * shard_cols * es}};
  const Buf in[] = {{full, rows * full_cols * es}};
  if (any_alias(out, 1, in, 1)) return TP_E_ALIAS;
  if (kind == TP_W_FC2 || kind == TP_W_PROJ) {
    // row-parallel shards are a contiguous run of rows
    const int64_t rl = kind == TP_W_FC2 ? f_l : hl * d;
    const uint8_t* src = static_cast<const uint8_t*>(full) + (int64_t)rank * rl * h * es;
    return hip_status(tp::copy_bytes(src, shard, rl * h * es, stream));
  }
  return hip_status(tp::pack_columns(dtype, full, rows, full_cols, shard, shard_cols, (int)kind, f_l, ffn, rank, hl,
                                     d, ad, G, g * d, stream));
}

int tp_mlp_fwd(const tp_dims* dims, int rank, tp_act act, tp_dtype dtype, const void* X, const void* A_i,
               const void* a_i, const void* B_i, void* U_i, void* Y_i, void* Z_i, hipStream_t stream) {
  if (dims == nullptr || X == nullptr || A_i == nullptr || B_i == nullptr || U_i == nullptr || Y_i == nullptr ||
      Z_i == nullptr)
    return TP_E_NULL;
  const int64_t s = dims->s, b = dims->b, h = dims->h, ffn = dims->ffn, t = dims->t;
  if (s <= 0 || b <= 0 || h <= 0 || ffn <= 0 || t <= 0) return TP_E_SHAPE;
  if (s * b >= kMaxDim || h >= kMaxDim || ffn >= kMaxDim) return TP_E_SHAPE;
  if (ffn % t != 0) return TP_E_DIVISIBILITY;
  if (rank < 0 || rank >= t) return TP_E_RANK;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  if (act != TP_ACT_GELU && act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU && act != TP_ACT_RELU)
    return TP_E_UNSUPPORTED;
  const int64_t M = s * b, f = ffn / t, n1 = act == TP_ACT_SWIGLU ? 2 * f : f, es = esize(dtype);
  if (dtype == TP_BF16 && (h % 8 != 0 || f % 8 != 0 || misaligned16({X, A_i, a_i, B_i, U_i, Y_i, Z_i})))
    return TP_E_UNSUPPORTED;
  const Buf outs[] = {{U_i, M * n1 * es}, {Y_i, M * f * es}, {Z_i, M * h * es}};
  const Buf ins[] = {{X, M * h * es}, {A_i, h * n1 * es}, {a_i, n1 * es}, {B_i, f * h * es}};
  if (any_alias(outs, 3, ins, 4)) return TP_E_ALIAS;

  tp::GemmParams g1 = {};
  g1.A = X; g1.lda = h;
  g1.B = A_i; g1.ldb = n1;
  g1.M = (int)M; g1.N = (int)n1; g1.K = (int)h;
  g1.C = U_i; g1.ldc = n1;
  g1.C2 = Y_i; g1.ldc2 = f;
  g1.bias = a_i;
  g1.fhalf = (int)f;
  g1.act = (int)act;
  const int epi1 = act == TP_ACT_SWIGLU ? tp::EPI_SWIGLU_FWD : tp::EPI_BIAS_ACT;
  tp::GemmParams g2 = {};
  g2.A = Y_i; g2.lda = f;
  g2.B = B_i; g2.ldb = h;
  g2.M = (int)M; g2.N = (int)h; g2.K = (int)f;
  g2.C = Z_i; g2.ldc = h;
  hipError_t e;
  if (dtype == TP_BF16) {
    e = tp::gemm_bf16(g1, true, false, epi1, stream);
    if (e == hipSuccess) e = tp::gemm_bf16(g2, true, false, tp::EPI_STORE, stream);
  } else {
    e = tp::gemm_f32(g1, true, false, epi1, stream);
    if (e == hipSuccess) e = tp::gemm_f32(g2, true, false, tp::EPI_STORE, stream);
  }
  return hip_status(e);
}

int tp_mlp_bwd_phase(const tp_dims* dims, int rank, tp_act act, tp_dtype dtype, tp_bwd_phase phase, const void* X,
                     const void* A_i, const void* B_i, const void* U_i, const void* Y_i, const void* dZ, void* dU_ws,
                     void* dA_i, void* da_i, void* dB_i, void* dX_i, hipStream_t stream) {
  const bool dgrad = phase == TP_BWD_ALL || phase == TP_BWD_DGRAD;
  const bool wgrad = phase == TP_BWD_ALL || phase == TP_BWD_WGRAD;
  if (dims == nullptr || dZ == nullptr || dU_ws == nullptr) return TP_E_NULL;
  if (dgrad && (A_i == nullptr || B_i == nullptr || U_i == nullptr || dX_i == nullptr)) return TP_E_NULL;
  if (wgrad && (X == nullptr || Y_i == nullptr || dA_i == nullptr || dB_i == nullptr)) return TP_E_NULL;
  const int64_t s = dims->s, b = dims->b, h = dims->h, ffn = dims->ffn, t = dims->t;
  if (s <= 0 || b <= 0 || h <= 0 || ffn <= 0 || t <= 0) return TP_E_SHAPE;
  if (s * b >= kMaxDim || h >= kMaxDim || ffn >= kMaxDim) return TP_E_SHAPE;
  if (ffn % t != 0) return TP_E_DIVISIBILITY;
  if (rank < 0 || rank >= t) return TP_E_RANK;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  if (act != TP_ACT_GELU && act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU && act != TP_ACT_RELU)
    return TP_E_UNSUPPORTED;
  if (phase != TP_BWD_ALL && phase != TP_BWD_DGRAD && phase != TP_BWD_WGRAD) return TP_E_UNSUPPORTED;
  const int64_t M = s * b, f = ffn / t, n1 = act == TP_ACT_SWIGLU ? 2 * f : f, es = esize(dtype);
  // a phase reads only its own operands; the others may be anything (they are not checked or touched)
  const void* Xp = wgrad ? X : nullptr;
  const void* Yp = wgrad ? Y_i : nullptr;
  const void* Ap = dgrad ? A_i : nullptr;
  const void* Bp = dgrad ? B_i : nullptr;
  const void* Up = dgrad ? U_i : nullptr;
  void* dAp = wgrad ? dA_i : nullptr;
  void* dap = wgrad ? da_i : nullptr;
  void* dBp = wgrad ? dB_i : nullptr;
  void* dXp = dgrad ? dX_i : nullptr;
  if (dtype == TP_BF16 &&
      (h % 8 != 0 || f % 8 != 0 || misaligned16({Xp, Ap, Bp, Up, Yp, dZ, dU_ws, dAp, dap, dBp, dXp})))
    return TP_E_UNSUPPORTED;
  // dU_ws is an output of the dgrad phase and an input of the wgrad-only phase
  const Buf dU = {dU_ws, M * n1 * es};
  const Buf outs[] = {{dAp, h * n1 * es}, {dap, n1 * es}, {dBp, f * h * es}, {dXp, M * h * es},
                      dgrad ? dU : Buf{nullptr, 0}};
  const Buf ins[] = {{Xp, M * h * es}, {Ap, h * n1 * es}, {Bp, f * h * es}, {Up, M * n1 * es},
                     {Yp, M * f * es}, {dZ, M * h * es}, dgrad ? Buf{nullptr, 0} : dU};
  if (any_alias(outs, 5, ins, 7)) return TP_E_ALIAS;

  // dU = (dZ B_i^T) * act'(U):  A = dZ [M,h] K-major, B = B_i [f,h] read as rows n, K-major.
  tp::GemmParams gy = {};
  gy.A = dZ; gy.lda = h;
  gy.B = Bp; gy.ldb = h;
  gy.M = (int)M; gy.N = (int)f; gy.K = (int)h;
  gy.C = dU_ws; gy.ldc = n1;
  gy.aux = Up; gy.ldaux = n1;
  gy.fhalf = (int)f;
  gy.act = (int)act;
  const int epiy = act == TP_ACT_SWIGLU ? tp::EPI_SWIGLU_BWD : tp::EPI_ACT_BWD;
  // dB = Y^T dZ: C [f,h], A(m=f, k=tok) = Y [tok,f] MN-major, B(n=h, k=tok) = dZ [tok,h] MN-major.
  tp::GemmParams gb = {};
  gb.A = Yp; gb.lda = f;
  gb.B = dZ; gb.ldb = h;
  gb.M = (int)f; gb.N = (int)h; gb.K = (int)M;
  gb.C = dBp; gb.ldc = h;
  // dA = X^T dU: C [h,n1], A(m=h, k=tok) = X MN-major, B(n, k=tok) = dU MN-major.
  tp::GemmParams ga = {};
  ga.A = Xp; ga.lda = h;
  ga.B = dU_ws; ga.ldb = n1;
  ga.M = (int)h; ga.N = (int)n1; ga.K = (int)M;
  ga.C = dAp; ga.ldc = n1;
  // dX = dU A^T: C [tok,h], A = dU [tok,n1] K-major, B(n=h, k=n1) = A_i [h,n1] K-major.
  tp::GemmParams gx = {};
  gx.A = dU_ws; gx.lda = n1;
  gx.B = Ap; gx.ldb = n1;
  gx.M = (int)M; gx.N = (int)h; gx.K = (int)n1;
  gx.C = dXp; gx.ldc = h;

  // Order within one call: dU, then the weight gradients, then dX (the full backward keeps the launch order it
  // always had; the split phases run dU + dX, or the weight gradients, alone).
  auto gemm = dtype == TP_BF16 ? tp::gemm_bf16 : tp::gemm_f32;
  hipError_t e = hipSuccess;
  if (dgrad) e = gemm(gy, true, true, epiy, stream);
  if (e == hipSuccess && wgrad) {
    if (dtype == TP_BF16) {
      e = tp::gemm_bf16_wgrad_pair(gb, ga, stream);
    } else {
      e = gemm(gb, false, false, tp::EPI_STORE, stream);
      if (e == hipSuccess) e = gemm(ga, false, false, tp::EPI_STORE, stream);
    }
    if (e == hipSuccess && dap != nullptr) e = tp::colsum(dtype, dU_ws, M, n1, dap, stream);
  }
  if (e == hipSuccess && dgrad) e = gemm(gx, true, true, tp::EPI_STORE, stream);
  return hip_status(e);
}

int tp_mlp_bwd(const tp_dims* dims, int rank, tp_act act, tp_dtype dtype, const void* X, const void* A_i,
               const void* B_i, const void* U_i, const void* Y_i, const void* dZ, void* dU_ws, void* dA_i,
               void* da_i, void* dB_i, void* dX_i, hipStream_t stream) {
  return tp_mlp_bwd_phase(dims, rank, act, dtype, TP_BWD_ALL, X, A_i, B_i, U_i, Y_i, dZ, dU_ws, dA_i, da_i, dB_i,
                          dX_i, stream);
}

int tp_attn_fwd(const tp_dims* dims, int rank, tp_dtype dtype, int causal, const void* X, const void* Wqkv_i,
                const void* bqkv_i, const void* Wo_i, void* QKV_i, void* O_i, float* lse_i, void* Z_i,
                hipStream_t stream) {
  if (dims == nullptr || X == nullptr || Wqkv_i == nullptr || Wo_i == nullptr || QKV_i == nullptr ||
      O_i == nullptr || Z_i == nullptr)
    return TP_E_NULL;
  const int64_t s = dims->s, b = dims->b, h = dims->h, a = dims->a, d = dims->d, t = dims->t;
  const int64_t g = dims->g == 0 ? a : dims->g;  // KV heads (0: as many as query heads)
  if (s <= 0 || b <= 0 || h <= 0 || a <= 0 || d <= 0 || t <= 0 || g <= 0) return TP_E_SHAPE;
  if (s * b >= kMaxDim || h >= kMaxDim) return TP_E_SHAPE;
  if (a % t != 0 || h != a * d || a % g != 0 || g % t != 0) return TP_E_DIVISIBILITY;
  if (rank < 0 || rank >= t) return TP_E_RANK;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  if (d > 128) return TP_E_UNSUPPORTED;
  const int64_t M = s * b, hl = a / t, n = (hl + 2 * (g / t)) * d, es = esize(dtype);
  if (dtype == TP_BF16 && (h % 8 != 0 || d % 8 != 0 || misaligned16({X, Wqkv_i, bqkv_i, Wo_i, QKV_i, O_i, Z_i})))
    return TP_E_UNSUPPORTED;
  const Buf outs[] = {{QKV_i, M * n * es}, {O_i, M * hl * d * es}, {lse_i, b * hl * s * 4}, {Z_i, M * h * es}};
  const Buf ins[] = {{X, M * h * es}, {Wqkv_i, h * n * es}, {bqkv_i, n * es}, {Wo_i, hl * d * h * es}};
  if (any_alias(outs, 4, ins, 4)) return TP_E_ALIAS;

  tp::GemmParams gq = {};
  gq.A = X; gq.lda = h;
  gq.B = Wqkv_i; gq.ldb = n;
  gq.M = (int)M; gq.N = (int)n; gq.K = (int)h;
  gq.C = QKV_i; gq.ldc = n;
  gq.bias = bqkv_i;
  tp::AttnParams ap = {};
  ap.qkv = QKV_i; ap.o = O_i; ap.lse = lse_i;
  ap.s = (int)s; ap.b = (int)b; ap.hl = (int)hl; ap.d = (int)d; ap.G = (int)(a / g);
  ap.causal = causal ? 1 : 0;
  ap.scale = (float)(1.0 / __builtin_sqrt((double)d));
  tp::GemmParams go = {};
  go.A = O_i; go.lda = hl * d;
  go.B = Wo_i; go.ldb = h;
  go.M = (int)M; go.N = (int)h; go.K = (int)(hl * d);
  go.C = Z_i; go.ldc = h;
  hipError_t e;
  if (dtype == TP_BF16) {
    // Z_i is not written until the projection: it holds the QKV GEMM's split-K partials
    e = tp::gemm_bf16_splitk(gq, true, false, tp::EPI_BIAS, static_cast<float*>(Z_i), M * h * es / 4, stream);
    if (e == hipSuccess) e = tp::attention_bf16(ap, stream);
    if (e == hipSuccess) e = tp::gemm_bf16(go, true, false, tp::EPI_STORE, stream);
  } else {
    e = tp::gemm_f32(gq, true, false, tp::EPI_BIAS, stream);
    if (e == hipSuccess) e = tp::attention_f32(ap, stream);
    if (e == hipSuccess) e = tp::gemm_f32(go, true, false, tp::EPI_STORE, stream);
  }
  return hip_status(e);
}

int tp_attn_bwd(const tp_dims* dims, int rank, tp_dtype dtype, int causal, const void* X, const void* Wqkv_i,
                const void* Wo_i, const void* QKV_i, const void* O_i, const float* lse_i, const void* dZ, void* dO_ws,
                float* rec_ws, void* dQKV_i, void* dWqkv_i, void* dbqkv_i, void* dWo_i, void* dX_i,
                hipStream_t stream) {
  if (dims == nullptr || X == nullptr || Wqkv_i == nullptr || Wo_i == nullptr || QKV_i == nullptr ||
      O_i == nullptr || lse_i == nullptr || dZ == nullptr || dO_ws == nullptr || rec_ws == nullptr ||
      dQKV_i == nullptr || dWqkv_i == nullptr || dWo_i == nullptr || dX_i == nullptr)
    return TP_E_NULL;
  const int64_t s = dims->s, b = dims->b, h = dims->h, a = dims->a, d = dims->d, t = dims->t;
  const int64_t g = dims->g == 0 ? a : dims->g;  // KV heads (0: as many as query heads)
  if (s <= 0 || b <= 0 || h <= 0 || a <= 0 || d <= 0 || t <= 0 || g <= 0) return TP_E_SHAPE;
  if (s * b >= kMaxDim || h >= kMaxDim) return TP_E_SHAPE;
  if (a % t != 0 || h != a * d || a % g != 0 || g % t != 0) return TP_E_DIVISIBILITY;
  if (rank < 0 || rank >= t) return TP_E_RANK;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  if (d > 128) return TP_E_UNSUPPORTED;
  const int64_t M = s * b, hl = a / t, n = (hl + 2 * (g / t)) * d, es = esize(dtype), nqb = (s + 63) / 64;
  if (dtype == TP_BF16 && (h % 8 != 0 || d % 8 != 0 ||
                           misaligned16({X, Wqkv_i, Wo_i, QKV_i, O_i, dZ, dO_ws, rec_ws, dQKV_i, dWqkv_i, dbqkv_i,
                                         dWo_i, dX_i})))
    return TP_E_UNSUPPORTED;
  const int64_t G = a / g, rec_floats = b * hl * nqb * 256;
  const int64_t ws_floats = rec_floats + (G > 1 ? M * (g / t) * 2 * d * G : 0);
  const Buf outs[] = {{dO_ws, M * hl * d * es}, {rec_ws, ws_floats * 4}, {dQKV_i, M * n * es},
                      {dWqkv_i, h * n * es},     {dbqkv_i, n * es},                  {dWo_i, hl * d * h * es},
                      {dX_i, M * h * es}};
  const Buf ins[] = {{X, M * h * es},     {Wqkv_i, h * n * es},     {Wo_i, hl * d * h * es}, {QKV_i, M * n * es},
                     {O_i, M * hl * d * es}, {lse_i, b * hl * s * 4}, {dZ, M * h * es}};
  if (any_alias(outs, 7, ins, 7)) return TP_E_ALIAS;

  // dO = dZ Wo_i^T (the projection's data gradient)
  tp::GemmParams gd = {};
  gd.A = dZ; gd.lda = h;
  gd.B = Wo_i; gd.ldb = h;
  gd.M = (int)M; gd.N = (int)(hl * d); gd.K = (int)h;
  gd.C = dO_ws; gd.ldc = hl * d;
  // attention core backward into dQKV_i
  tp::AttnBwdParams bp = {};
  bp.qkv = QKV_i; bp.o = O_i; bp.dout = dO_ws; bp.lse = lse_i; bp.rec = rec_ws; bp.dqkv = dQKV_i;
  bp.s = (int)s; bp.b = (int)b; bp.hl = (int)hl; bp.d = (int)d; bp.G = (int)G;
  bp.kvpart = (G > 1 && dtype == TP_BF16) ? rec_ws + rec_floats : nullptr;
  bp.causal = causal ? 1 : 0;
  bp.scale = (float)(1.0 / __builtin_sqrt((double)d));
  // weight gradients dWo_i = O_i^T dZ and dWqkv_i = X^T dQKV_i (both over K = s*b)
  tp::GemmParams gwo = {};
  gwo.A = O_i; gwo.lda = hl * d;
  gwo.B = dZ; gwo.ldb = h;
  gwo.M = (int)(hl * d); gwo.N = (int)h; gwo.K = (int)M;
  gwo.C = dWo_i; gwo.ldc = h;
  tp::GemmParams gwq = {};
  gwq.A = X; gwq.lda = h;
  gwq.B = dQKV_i; gwq.ldb = n;
  gwq.M = (int)h; gwq.N = (int)n; gwq.K = (int)M;
  gwq.C = dWqkv_i; gwq.ldc = n;
  // the partial dX_i = dQKV_i Wqkv_i^T
  tp::GemmParams gx = {};
  gx.A = dQKV_i; gx.lda = n;
  gx.B = Wqkv_i; gx.ldb = n;
  gx.M = (int)M; gx.N = (int)h; gx.K = (int)n;
  gx.C = dX_i; gx.ldc = h;

  auto gemm = dtype == TP_BF16 ? tp::gemm_bf16 : tp::gemm_f32;
  // dX_i is not written until the last GEMM: it holds the dO GEMM's split-K partials
  hipError_t e = dtype == TP_BF16 ? tp::gemm_bf16_splitk(gd, true, true, tp::EPI_STORE, static_cast<float*>(dX_i),
                                                         M * h * es / 4, stream)
                                  : gemm(gd, true, true, tp::EPI_STORE, stream);
  if (e == hipSuccess) e = tp::attention_bwd(dtype, bp, stream);
  if (e == hipSuccess) {
    if (dtype == TP_BF16) {  // dX_i again lends its memory: split-K partials of the pair's tail tiles
      e = tp::gemm_bf16_wgrad_pair_splitk(gwo, gwq, static_cast<float*>(dX_i), M * h * es / 4, stream);
    } else {
      e = gemm(gwo, false, false, tp::EPI_STORE, stream);
      if (e == hipSuccess) e = gemm(gwq, false, false, tp::EPI_STORE, stream);
    }
  }
  if (e == hipSuccess && dbqkv_i != nullptr) e = tp::colsum(dtype, dQKV_i, M, n, dbqkv_i, stream);
  if (e == hipSuccess) e = gemm(gx, true, true, tp::EPI_STORE, stream);
  return hip_status(e);
}

int64_t tp_attn_bwd_workspace(const tp_dims* dims) {
  if (dims == nullptr) return 0;
  const int64_t s = dims->s, b = dims->b, a = dims->a, d = dims->d, t = dims->t;
  const int64_t g = dims->g == 0 ? a : dims->g;
  if (s <= 0 || b <= 0 || a <= 0 || d <= 0 || t <= 0 || g <= 0 || a % t != 0 || a % g != 0 || g % t != 0) return 0;
  const int64_t hl = a / t, G = a / g, nqb = (s + 63) / 64;
  return (b * hl * nqb * 256 + (G > 1 ? s * b * (g / t) * 2 * d * G : 0)) * 4;
}

int tp_partial_reduce(int64_t n, int64_t h, int t, tp_dtype dtype, const void* partials, const void* bias_c,
                      void* out, hipStream_t stream) {
  if (partials == nullptr || out == nullptr) return TP_E_NULL;
  if (n <= 0 || h <= 0 || t <= 0) return TP_E_SHAPE;
  if (n % h != 0) return TP_E_SHAPE;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  const int64_t es = esize(dtype);
  const Buf outs[] = {{out, n * es}};
  const Buf ins[] = {{partials, (int64_t)t * n * es}, {bias_c, h * es}};
  if (any_alias(outs, 1, ins, 2)) return TP_E_ALIAS;
  return hip_status(tp::reduce_partials(dtype, partials, t, n, 0, n, bias_c, h, out, stream));
}

int tp_reduce_scatter_dim0(const tp_dims* dims, int rank, tp_dtype dtype, const void* partials, const void* bias_c,
                           void* out, hipStream_t stream) {
  if (dims == nullptr || partials == nullptr || out == nullptr) return TP_E_NULL;
  const int64_t s = dims->s, b = dims->b, h = dims->h, t = dims->t;
  if (s <= 0 || b <= 0 || h <= 0 || t <= 0) return TP_E_SHAPE;
  if (s % t != 0) return TP_E_DIVISIBILITY;
  if (rank < -1 || rank >= t) return TP_E_RANK;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  const int64_t es = esize(dtype), n = s * b * h, slice = (s / t) * b * h;
  const int64_t count = rank < 0 ? n : slice;
  const Buf outs[] = {{out, count * es}};
  const Buf ins[] = {{partials, t * n * es}, {bias_c, h * es}};
  if (any_alias(outs, 1, ins, 2)) return TP_E_ALIAS;
  const int64_t in_off = rank < 0 ? 0 : (int64_t)rank * slice;
  return hip_status(tp::reduce_partials(dtype, partials, (int)t, n, in_off, count, bias_c, h, out, stream));
}

int tp_gather_dim0(const tp_dims* dims, tp_dtype dtype, const void* slices, void* out, hipStream_t stream) {
  if (dims == nullptr || slices == nullptr || out == nullptr) return TP_E_NULL;
  const int64_t s = dims->s, b = dims->b, h = dims->h, t = dims->t;
  if (s <= 0 || b <= 0 || h <= 0 || t <= 0) return TP_E_SHAPE;
  if (s % t != 0) return TP_E_DIVISIBILITY;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  const int64_t bytes = s * b * h * esize(dtype);
  const Buf outs[] = {{out, bytes}};
  const Buf ins[] = {{slices, bytes}};
  if (any_alias(outs, 1, ins, 1)) return TP_E_ALIAS;
  return hip_status(tp::copy_bytes(slices, out, bytes, stream));
}

int64_t tp_sp_ln_bwd_workspace(int64_t rows, int64_t h) {
  if (rows <= 0 || h <= 0) return 0;
  return tp::sp_bwd_blocks(rows) * 2 * h * (int64_t)sizeof(float);
}

namespace {
// Size / dtype / alignment rules shared by the two sequence-parallel region calls.
int sp_check_sizes(int64_t rows, int64_t h, tp_dtype dtype, double p) {
  if (rows <= 0 || h <= 0 || rows >= kMaxDim || !(p >= 0.0 && p < 1.0)) return TP_E_SHAPE;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  if (h % 8 != 0 || h > tp::SP_MAX_H) return TP_E_UNSUPPORTED;
  return TP_OK;
}
}  // namespace

int tp_sp_dropout_add_ln_fwd(int64_t rows, int64_t h, tp_dtype dtype, double p, double eps, const void* z,
                             const void* residual, const uint32_t* bits, const void* gamma, const void* beta,
                             void* out, void* y, float* mean, float* rstd, uint8_t* mask, hipStream_t stream) {
  if (z == nullptr || gamma == nullptr || beta == nullptr) return TP_E_NULL;
  // without y the call is the first half of the LayerNorm-folded column GEMM: u and the statistics are its outputs
  if (y == nullptr && (out == nullptr || mean == nullptr || rstd == nullptr)) return TP_E_NULL;
  if (p > 0.0 && bits == nullptr) return TP_E_NULL;
  if (!(eps >= 0.0) || eps > 1e30) return TP_E_SHAPE;
  int st = sp_check_sizes(rows, h, dtype, p);
  if (st != TP_OK) return st;
  const uint32_t* bits_used = p > 0.0 ? bits : nullptr;
  if (misaligned16({z, residual, (const void*)bits_used, gamma, beta, out, y})) return TP_E_UNSUPPORTED;
  const int64_t es = esize(dtype), n = rows * h;
  const Buf outs[] = {{out, n * es}, {y, n * es}, {mean, rows * 4}, {rstd, rows * 4}, {mask, n / 8}};
  const Buf ins[] = {{z, n * es}, {residual, n * es}, {bits_used, n * 4}, {gamma, h * es}, {beta, h * es}};
  if (any_alias(outs, 5, ins, 5)) return TP_E_ALIAS;
  tp::SpFwdArgs a;
  a.z = z;
  a.residual = residual;
  a.bits = bits_used;
  a.gamma = gamma;
  a.beta = beta;
  a.out = out;
  a.y = y;
  a.mean = mean;
  a.rstd = rstd;
  a.mask = mask;
  a.rows = rows;
  a.h = h;
  a.p = p;
  a.eps = eps;
  return hip_status(tp::sp_dropout_add_ln_fwd(dtype, a, stream));
}

namespace {
// The backward's checks and launch, shared by the workspace and the no-allocation entry points.  noalloc: ws is
// ignored (may be NULL) and the library's fixed scratch takes its place.
int sp_bwd_entry(int64_t rows, int64_t h, tp_dtype dtype, double p, const void* u, const void* gamma,
                 const float* mean, const float* rstd, const void* dy, const void* dres_in, const uint8_t* mask,
                 void* dres, void* dz, float* dgamma, float* dbeta, float* ws, bool noalloc, hipStream_t stream) {
  if (u == nullptr || gamma == nullptr || mean == nullptr || rstd == nullptr || dy == nullptr ||
      dgamma == nullptr || dbeta == nullptr || (!noalloc && ws == nullptr))
    return TP_E_NULL;
  if (p > 0.0 && mask == nullptr) return TP_E_NULL;
  int st = sp_check_sizes(rows, h, dtype, p);
  if (st != TP_OK) return st;
  if (noalloc) ws = nullptr;
  if (misaligned16({u, gamma, dy, dres_in, dres, dz, (const void*)dgamma, (const void*)dbeta, (const void*)ws}))
    return TP_E_UNSUPPORTED;
  if (noalloc && tp_sp_ln_bwd_workspace(rows, h) > tp::SP_NOALLOC_SCRATCH_BYTES) return TP_E_SCRATCH;
  const uint8_t* mask_used = p > 0.0 ? mask : nullptr;
  const int64_t es = esize(dtype), n = rows * h;
  const Buf outs[] = {{dres, n * es}, {dz, n * es}, {dgamma, h * 4}, {dbeta, h * 4},
                      {ws, tp_sp_ln_bwd_workspace(rows, h)}};
  const Buf ins[] = {{u, n * es}, {gamma, h * es}, {mean, rows * 4}, {rstd, rows * 4}, {dy, n * es},
                     {dres_in, n * es}, {mask_used, n / 8}};
  if (any_alias(outs, 5, ins, 7)) return TP_E_ALIAS;
  if (noalloc) {
    const hipError_t e = tp::sp_noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
  }
  tp::SpBwdArgs a;
  a.u = u;
  a.gamma = gamma;
  a.mean = mean;
  a.rstd = rstd;
  a.dy = dy;
  a.dres_in = dres_in;
  a.mask = mask_used;
  a.dres = dres;
  a.dz = dz;
  a.dgamma = dgamma;
  a.dbeta = dbeta;
  a.ws = ws;
  a.rows = rows;
  a.h = h;
  a.p = p;
  return hip_status(tp::sp_dropout_add_ln_bwd(dtype, a, stream));
}
}  // namespace

int tp_sp_dropout_add_ln_bwd(int64_t rows, int64_t h, tp_dtype dtype, double p, const void* u, const void* gamma,
                             const float* mean, const float* rstd, const void* dy, const void* dres_in,
                             const uint8_t* mask, void* dres, void* dz, float* dgamma, float* dbeta, float* ws,
                             hipStream_t stream) {
  return sp_bwd_entry(rows, h, dtype, p, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz, dgamma, dbeta, ws, false,
                      stream);
}

int tp_sp_dropout_add_ln_bwd_noalloc(int64_t rows, int64_t h, tp_dtype dtype, double p, const void* u,
                                     const void* gamma, const float* mean, const float* rstd, const void* dy,
                                     const void* dres_in, const uint8_t* mask, void* dres, void* dz, float* dgamma,
                                     float* dbeta, hipStream_t stream) {
  return sp_bwd_entry(rows, h, dtype, p, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz, dgamma, dbeta, nullptr,
                      true, stream);
}

namespace {
int ce_check(int64_t rows, int64_t v_local, int rank, tp_dtype dtype) {
  if (rows <= 0 || v_local <= 0 || rows >= kMaxDim || v_local >= kMaxDim || rows * v_local >= ((int64_t)1 << 40))
    return TP_E_SHAPE;
  if (rank < 0) return TP_E_RANK;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  if (v_local % 8 != 0) return TP_E_UNSUPPORTED;
  return TP_OK;
}
}  // namespace

int tp_vocab_ce_fwd_local(int64_t rows, int64_t v_local, int rank, tp_dtype dtype, const void* logits_i,
                          const int32_t* targets, float* stats_i, hipStream_t stream) {
  if (logits_i == nullptr || targets == nullptr || stats_i == nullptr) return TP_E_NULL;
  const int st = ce_check(rows, v_local, rank, dtype);
  if (st != TP_OK) return st;
  if (misaligned16({logits_i, (const void*)stats_i})) return TP_E_UNSUPPORTED;
  const Buf outs[] = {{stats_i, rows * 16}};
  const Buf ins[] = {{logits_i, rows * v_local * esize(dtype)}, {targets, rows * 4}};
  if (any_alias(outs, 1, ins, 2)) return TP_E_ALIAS;
  return hip_status(tp::vocab_ce_local(dtype, logits_i, targets, rows, (int)v_local, rank, stats_i, stream));
}

int tp_vocab_ce_combine(int64_t rows, int t, const float* stats, const int32_t* targets, float* loss, float* lse,
                        hipStream_t stream) {
  if (stats == nullptr || targets == nullptr || loss == nullptr) return TP_E_NULL;
  if (rows <= 0 || t <= 0 || rows >= kMaxDim) return TP_E_SHAPE;
  if (misaligned16({(const void*)stats})) return TP_E_UNSUPPORTED;
  const Buf outs[] = {{loss, rows * 4}, {lse, rows * 4}};
  const Buf ins[] = {{stats, (int64_t)t * rows * 16}, {targets, rows * 4}};
  if (any_alias(outs, 2, ins, 2)) return TP_E_ALIAS;
  return hip_status(tp::vocab_ce_combine(stats, t, rows, targets, loss, lse, stream));
}

int tp_vocab_ce_bwd(int64_t rows, int64_t v_local, int rank, tp_dtype dtype, const void* logits_i,
                    const int32_t* targets, const float* lse, const float* dloss, void* dlogits_i,
                    hipStream_t stream) {
  if (logits_i == nullptr || targets == nullptr || lse == nullptr || dloss == nullptr || dlogits_i == nullptr)
    return TP_E_NULL;
  const int st = ce_check(rows, v_local, rank, dtype);
  if (st != TP_OK) return st;
  if (misaligned16({logits_i, (const void*)dlogits_i})) return TP_E_UNSUPPORTED;
  const int64_t bytes = rows * v_local * esize(dtype);
  const Buf outs[] = {{dlogits_i, bytes}};
  const Buf ins[] = {{logits_i, bytes}, {targets, rows * 4}, {lse, rows * 4}, {dloss, rows * 4}};
  if (any_alias(outs, 1, ins, 4)) return TP_E_ALIAS;
  return hip_status(tp::vocab_ce_bwd(dtype, logits_i, targets, lse, dloss, rows, (int)v_local, rank, dlogits_i,
                                     stream));
}

namespace {
// Sizes, dtype and alignment shared by the two LayerNorm-folded calls; the large-tile kernel needs h % 64 == 0.
int ln_check(const tp_dims* dims, tp_act act, tp_dtype dtype) {
  const int64_t s = dims->s, b = dims->b, h = dims->h, ffn = dims->ffn, t = dims->t;
  if (h <= 0 || ffn <= 0 || t <= 0 || s < 0 || b < 0) return TP_E_SHAPE;
  if (s * b >= kMaxDim || h >= kMaxDim || ffn >= kMaxDim) return TP_E_SHAPE;
  if (ffn % t != 0) return TP_E_DIVISIBILITY;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  if (dtype != TP_BF16) return TP_E_UNSUPPORTED;
  if (act != TP_ACT_GELU && act != TP_ACT_GELU_TANH && act != TP_ACT_SWIGLU && act != TP_ACT_RELU)
    return TP_E_UNSUPPORTED;
  if (h % 64 != 0 || h < 128 || (ffn / t) % 8 != 0) return TP_E_UNSUPPORTED;
  return TP_OK;
}
}  // namespace

int tp_ln_fold_weights(const tp_dims* dims, tp_act act, tp_dtype dtype, const void* gamma, const void* beta,
                       const void* A_i, const void* a_i, void* A_ln, float* c_ln, float* b_ln, hipStream_t stream) {
  if (dims == nullptr || gamma == nullptr || beta == nullptr || A_i == nullptr || A_ln == nullptr ||
      c_ln == nullptr || b_ln == nullptr)
    return TP_E_NULL;
  const int st = ln_check(dims, act, dtype);
  if (st != TP_OK) return st;
  const int64_t h = dims->h, f = dims->ffn / dims->t, n1 = act == TP_ACT_SWIGLU ? 2 * f : f;
  if (misaligned16({gamma, beta, A_i, a_i, A_ln})) return TP_E_UNSUPPORTED;
  const Buf outs[] = {{A_ln, h * n1 * 2}, {c_ln, n1 * 4}, {b_ln, n1 * 4}};
  const Buf ins[] = {{gamma, h * 2}, {beta, h * 2}, {A_i, h * n1 * 2}, {a_i, n1 * 2}};
  if (any_alias(outs, 3, ins, 4)) return TP_E_ALIAS;
  return hip_status(tp::ln_fold_weights(gamma, beta, A_i, a_i, h, n1, A_ln, c_ln, b_ln, stream));
}

int tp_ln_mlp_fwd(const tp_dims* dims, int rank, tp_act act, tp_dtype dtype, const void* X, const float* ln_mean,
                  const float* ln_rstd, const void* A_ln, const float* c_ln, const float* b_ln, const void* B_i,
                  void* U_i, void* Y_i, void* Z_i, hipStream_t stream) {
  if (dims == nullptr || X == nullptr || ln_mean == nullptr || ln_rstd == nullptr || A_ln == nullptr ||
      c_ln == nullptr || b_ln == nullptr || B_i == nullptr || U_i == nullptr || Y_i == nullptr || Z_i == nullptr)
    return TP_E_NULL;
  int st = ln_check(dims, act, dtype);
  if (st != TP_OK) return st;
  if (dims->s <= 0 || dims->b <= 0) return TP_E_SHAPE;
  if (rank < 0 || rank >= dims->t) return TP_E_RANK;
  const int64_t M = dims->s * dims->b, h = dims->h, f = dims->ffn / dims->t;
  const int64_t n1 = act == TP_ACT_SWIGLU ? 2 * f : f;
  if (misaligned16({X, A_ln, B_i, U_i, Y_i, Z_i})) return TP_E_UNSUPPORTED;
  const Buf outs[] = {{U_i, M * n1 * 2}, {Y_i, M * f * 2}, {Z_i, M * h * 2}};
  const Buf ins[] = {{X, M * h * 2}, {ln_mean, M * 4}, {ln_rstd, M * 4}, {A_ln, h * n1 * 2}, {c_ln, n1 * 4},
                     {b_ln, n1 * 4}, {B_i, f * h * 2}};
  if (any_alias(outs, 3, ins, 7)) return TP_E_ALIAS;
  tp::GemmParams g1 = {};
  g1.A = X; g1.lda = h;
  g1.B = A_ln; g1.ldb = n1;
  g1.M = (int)M; g1.N = (int)n1; g1.K = (int)h;
  g1.C = U_i; g1.ldc = n1;
  g1.C2 = Y_i; g1.ldc2 = f;
  g1.fhalf = (int)f;
  g1.act = (int)act;
  g1.ln_mean = ln_mean; g1.ln_rstd = ln_rstd; g1.ln_c = c_ln; g1.ln_b = b_ln;
  tp::GemmParams g2 = {};
  g2.A = Y_i; g2.lda = f;
  g2.B = B_i; g2.ldb = h;
  g2.M = (int)M; g2.N = (int)h; g2.K = (int)f;
  g2.C = Z_i; g2.ldc = h;
  hipError_t e = tp::gemm_bf16_ln(g1, act == TP_ACT_SWIGLU ? tp::EPI_LN_SWIGLU : tp::EPI_LN_ACT, stream);
  if (e == hipSuccess) e = tp::gemm_bf16(g2, true, false, tp::EPI_STORE, stream);
  return hip_status(e);
}

namespace {
int logits_check(int64_t rows, int64_t h, int64_t v_local, tp_dtype dtype) {
  if (rows <= 0 || h <= 0 || v_local <= 0 || rows >= kMaxDim || h >= kMaxDim || v_local >= kMaxDim)
    return TP_E_SHAPE;
  if (bad_dtype(dtype)) return TP_E_DTYPE;
  if (dtype == TP_BF16 && (h % 8 != 0 || v_local % 8 != 0)) return TP_E_UNSUPPORTED;
  return TP_OK;
}
}  // namespace

int tp_vocab_logits_fwd(int64_t rows, int64_t h, int64_t v_local, tp_dtype dtype, const void* X, const void* E_i,
                        void* logits_i, hipStream_t stream) {
  if (X == nullptr || E_i == nullptr || logits_i == nullptr) return TP_E_NULL;
  const int st = logits_check(rows, h, v_local, dtype);
  if (st != TP_OK) return st;
  if (dtype == TP_BF16 && misaligned16({X, E_i, logits_i})) return TP_E_UNSUPPORTED;
  const int64_t es = esize(dtype);
  const Buf outs[] = {{logits_i, rows * v_local * es}};
  const Buf ins[] = {{X, rows * h * es}, {E_i, v_local * h * es}};
  if (any_alias(outs, 1, ins, 2)) return TP_E_ALIAS;
  // logits = X E_i^T: A = X [rows, h] K-major; B(n = vocab row, k) = E_i [v_local, h] K-major
  tp::GemmParams g = {};
  g.A = X; g.lda = h;
  g.B = E_i; g.ldb = h;
  g.M = (int)rows; g.N = (int)v_local; g.K = (int)h;
  g.C = logits_i; g.ldc = v_local;
  auto gemm = dtype == TP_BF16 ? tp::gemm_bf16 : tp::gemm_f32;
  return hip_status(gemm(g, true, true, tp::EPI_STORE, stream));
}

int tp_vocab_logits_bwd(int64_t rows, int64_t h, int64_t v_local, tp_dtype dtype, const void* X, const void* E_i,
                        const void* dlogits_i, void* dX_i, void* dE_i, hipStream_t stream) {
  if (dlogits_i == nullptr || (dX_i == nullptr && dE_i == nullptr)) return TP_E_NULL;
  if (dX_i != nullptr && E_i == nullptr) return TP_E_NULL;
  if (dE_i != nullptr && X == nullptr) return TP_E_NULL;
  const int st = logits_check(rows, h, v_local, dtype);
  if (st != TP_OK) return st;
  const void* Xp = dE_i != nullptr ? X : nullptr;    // each output reads only its own operands
  const void* Ep = dX_i != nullptr ? E_i : nullptr;
  if (dtype == TP_BF16 && misaligned16({Xp, Ep, dlogits_i, dX_i, dE_i})) return TP_E_UNSUPPORTED;
  const int64_t es = esize(dtype);
  const Buf outs[] = {{dX_i, rows * h * es}, {dE_i, v_local * h * es}};
  const Buf ins[] = {{Xp, rows * h * es}, {Ep, v_local * h * es}, {dlogits_i, rows * v_local * es}};
  if (any_alias(outs, 2, ins, 3)) return TP_E_ALIAS;
  auto gemm = dtype == TP_BF16 ? tp::gemm_bf16 : tp::gemm_f32;
  hipError_t e = hipSuccess;
  if (dE_i != nullptr) {
    // dE_i = dlogits^T X: C [v_local, h]; A(m = vocab row, k = token) = dlogits MN-major; B(n, k) = X MN-major
    tp::GemmParams g = {};
    g.A = dlogits_i; g.lda = v_local;
    g.B = Xp; g.ldb = h;
    g.M = (int)v_local; g.N = (int)h; g.K = (int)rows;
    g.C = dE_i; g.ldc = h;
    e = gemm(g, false, false, tp::EPI_STORE, stream);
  }
  if (e == hipSuccess && dX_i != nullptr) {
    // dX_i = dlogits E_i: A = dlogits [rows, v_local] K-major; B(n = h, k = vocab row) = E_i [v_local, h] MN-major
    tp::GemmParams g = {};
    g.A = dlogits_i; g.lda = v_local;
    g.B = Ep; g.ldb = h;
    g.M = (int)rows; g.N = (int)h; g.K = (int)v_local;
    g.C = dX_i; g.ldc = h;
    e = gemm(g, true, false, tp::EPI_STORE, stream);
  }
  return hip_status(e);
}

}  // extern "C"
