/* tpshard.h -- C ABI of libtpshard: one tensor-parallel rank's compute of a Megatron-style column->row block on an
 * AMD Instinct MI355X (gfx950), plus the on-device g / g-bar / f reductions over t partial-sum buffers.
 *
 * Pages cited (by title and section):
 *   [ATLAS] "Tensor Parallelism (TP) 与 Sequence Parallelism (SP)", llm-infra-atlas parallel/02_tp_sp
 *   [SPLIT] 111qqz.com "tensor-parallelism-matrix-split" (column / row split of one linear layer and its backward)
 *   [MEGA]  blog.vllbc.top visual reading of Megatron-LM tensor parallelism
 *   [SPCP]  blog.vllbc.top "Sequence Parallel 与 Context Parallel"
 *
 * Notation follows the pages: s sequence length, b micro-batch, h hidden size, ffn the MLP inner width, a heads,
 * d head dim (h = a*d), t the tensor-parallel degree.  Activations are sequence-first [s, b, h] ([ATLAS] §1): a
 * GEMM sees them as M = s*b rows of h, in s-major order.  Weights use the math layout [in, out] ([SPLIT], the
 * remark on nn.Linear storage): a column shard is [h, ffn/t], a row shard [ffn/t, h].
 *
 * Conventions shared by every entry point:
 *   - Tensors are caller-owned, device-resident, dense row-major.  The library allocates nothing, frees nothing
 *     and keeps no state between calls (apart from the opt-in, thread-local launch-timing log below, and the fixed
 *     per-GPU scratch of tp_sp_dropout_add_ln_bwd_noalloc); code objects are linked into the shared object.
 *   - bf16 (TP_BF16) tensors hold bfloat16 values; the bf16 path needs every row length that is a GEMM K or N
 *     dimension (h, ffn/t, d, 3*(a/t)*d) to be a multiple of 8 and every pointer 16-byte aligned.  fp32 (TP_F32)
 *     tensors hold IEEE binary32 and have no alignment rule.
 *   - Every call only enqueues kernels on `stream` (0 = the null stream) and returns; nothing synchronises.
 *     The status is that of host validation and of the launches (hipGetLastError right after them).
 *   - Validation happens before any HIP call, in this order: null dims / pointers (TP_E_NULL), non-positive sizes
 *     (TP_E_SHAPE), divisibility rules of the pages (TP_E_DIVISIBILITY), rank (TP_E_RANK), dtype / activation
 *     (TP_E_DTYPE, TP_E_UNSUPPORTED), alignment (TP_E_UNSUPPORTED), output-aliases-input (TP_E_ALIAS).
 *   - Calls are stateless and re-entrant; two calls that write the same buffer on different streams race.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPSHARD_ABI_VERSION 2

/* Sizes in the pages' notation.  MLP calls read s, b, h, ffn, t; attention calls read s, b, h, a, d, t and g; the
 * reductions read s, b, h, t.  g is the number of KV heads (query groups) of grouped-query attention ([MEGA] QKV
 * remark: the fused QKV weight is h + 2*hkv wide); 0 means g = a (multi-head attention).  Needs a % g == 0 and
 * g % t == 0: each rank owns whole groups (with g < t a rank would need other ranks' KV heads). */
typedef struct {
  int64_t s, b, h, ffn, a, d, t, g;
} tp_dims;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Element-wise activation between the column and the row GEMM ([ATLAS] §2, [MEGA]: GeLU; [ATLAS] §1: SwiGLU
 * computes over 2 x ffn; [SPLIT] two-layer example: ReLU).  TP_ACT_GELU is the erf form x*Phi(x); TP_ACT_SWIGLU
 * is SiLU(gate) * up with the fc1 weight [h, 2*ffn] = [gate | up]. */
typedef enum { TP_ACT_GELU = 0, TP_ACT_GELU_TANH = 1, TP_ACT_SWIGLU = 2, TP_ACT_RELU = 3 } tp_act;

/* Which full weight (or bias) tp_shard_weights slices. */
typedef enum {
  TP_W_FC1 = 0,         /* full [h, ffn]            -> shard [h, ffn/t]  (column-parallel)                    */
  TP_W_FC1_GATE_UP = 1, /* full [h, 2ffn]=[Wg|Wu]   -> shard [h, 2ffn/t] = [Wg_i | Wu_i]                      */
  TP_W_FC2 = 2,         /* full [ffn, h]            -> shard [ffn/t, h]  (row-parallel)                       */
  TP_W_QKV = 3,         /* full [h, (a+2g)d] = [Wq|Wk|Wv] -> shard [h, (a/t + 2g/t)d]: per local KV group its
                           a/g query heads, then its k and v ([MEGA] interleave); g = a: [q_j | k_j | v_j]        */
  TP_W_PROJ = 4,        /* full [ad, h]             -> shard [(a/t)*d, h] (row-parallel)                      */
  TP_B_FC1 = 5,         /* full [ffn]               -> [ffn/t]                                                */
  TP_B_FC1_GATE_UP = 6, /* full [2ffn]=[bg|bu]      -> [2ffn/t] = [bg_i | bu_i]                               */
  TP_B_QKV = 7          /* full [(a+2g)d] = [bq|bk|bv] -> [(a/t + 2g/t)d] grouped like TP_W_QKV              */
} tp_wkind;

enum {
  TP_OK = 0,
  TP_E_NULL = -1,         /* a required pointer (or dims) is NULL                                  */
  TP_E_SHAPE = -2,        /* a size is non-positive or out of the supported range                 */
  TP_E_DIVISIBILITY = -3, /* s % t, ffn % t, a % t or h != a*d ([ATLAS] §1, [MEGA] divide())       */
  TP_E_DTYPE = -4,        /* unknown dtype                                                        */
  TP_E_RANK = -5,         /* rank outside [0, t) (or -1 where not allowed)                         */
  TP_E_ALIAS = -6,        /* an output buffer overlaps an input buffer                            */
  TP_E_UNSUPPORTED = -7,  /* valid but not built: activation/dtype combination, alignment, d range  */
  TP_E_HIP = -8,          /* a HIP launch failed; tp_last_hip_error() names it                      */
  TP_E_SCRATCH = -9       /* needs more scratch than the fixed no-allocation buffer holds          */
};

/* Text of a status code (static storage). */
const char* tp_status_str(int status);

/* hipError_t of the last failed launch in this thread (0 if none). */
int tp_last_hip_error(void);

/* TPSHARD_ABI_VERSION of the built library. */
int tp_abi_version(void);

/* Shard packer ([ATLAS] §2-3, [MEGA]: fc1/QKV split by output columns -- QKV by head -- and fc2/projection by
 * input rows).  Copies rank `rank`'s shard of `full` into `shard` (layouts in tp_wkind), bit for bit.
 * Uses s, b of dims not at all; needs ffn % t == 0 (FC kinds) or a % t == 0 and h == a*d (QKV/PROJ kinds).
 * full and shard must not overlap. */
int tp_shard_weights(const tp_dims* dims, int rank, tp_wkind kind, tp_dtype dtype, const void* full, void* shard,
                     hipStream_t stream);

/* MLP forward of rank `rank` ([ATLAS] §2 column->act->row; [SPLIT] two-layer forward):
 *   U_i = X A_i (+ a_i)        column GEMM, saved for the backward        [s, b, N1]
 *   Y_i = act(U_i)             element-wise, local to the shard           [s, b, ffn/t]
 *   Z_i = Y_i B_i              row GEMM: a partial sum of the block output [s, b, h]; no row bias here
 * N1 = ffn/t, or 2*ffn/t for SwiGLU (U_i = [U_gate | U_up]).  A_i [h, N1], a_i [N1] (nullable), B_i [ffn/t, h].
 * Running ranks 0..t-1 with Z_i pointing at partials + i*s*b*h and then tp_partial_reduce (g, all-reduce form)
 * or tp_reduce_scatter_dim0 (g-bar under sequence parallelism) gives the block output. */
int tp_mlp_fwd(const tp_dims* dims, int rank, tp_act act, tp_dtype dtype, const void* X, const void* A_i,
               const void* a_i, const void* B_i, void* U_i, void* Y_i, void* Z_i, hipStream_t stream);

/* MLP backward of rank `rank` ([SPLIT] backward of both layers; [ATLAS] §2 f/g):
 *   dY_i = dZ B_i^T, fused with dU_i = dY_i * act'(U_i)     -> dU_ws [s, b, N1] (caller workspace)
 *   dB_i = Y_i^T dZ                                          -> [ffn/t, h]   local weight gradient
 *   dA_i = X^T dU_i                                          -> [h, N1]      local weight gradient
 *   da_i = column sums of dU_i (nullable)                    -> [N1]
 *   dX_i = dU_i A_i^T                                        -> [s, b, h]    a partial: f sums them over ranks
 * dZ is the full upstream gradient (g is the identity in backward; after the dim-0 all-gather under SP). */
int tp_mlp_bwd(const tp_dims* dims, int rank, tp_act act, tp_dtype dtype, const void* X, const void* A_i,
               const void* B_i, const void* U_i, const void* Y_i, const void* dZ, void* dU_ws, void* dA_i,
               void* da_i, void* dB_i, void* dX_i, hipStream_t stream);

/* The MLP backward split into its two independent halves ([ATLAS] §5: the dgrad's reduction and the wgrad GEMMs
 * do not depend on each other, which is what lets the dX reduction run while the weight gradients compute):
 *   TP_BWD_DGRAD: dU_ws = (dZ B_i^T) * act'(U_i) and dX_i = dU_ws A_i^T.  Reads dZ, B_i, U_i, A_i; X, Y_i, dA_i,
 *                 da_i, dB_i are not used (may be NULL).
 *   TP_BWD_WGRAD: dB_i = Y_i^T dZ, dA_i = X^T dU_ws, da_i = column sums of dU_ws, with dU_ws as left by this rank's
 *                 TP_BWD_DGRAD call (an input here).  A_i, B_i, U_i, dX_i are not used (may be NULL).
 *   TP_BWD_ALL:   both, exactly tp_mlp_bwd.
 * The two phases of a rank, in that order, give bit-for-bit the outputs of tp_mlp_bwd (same kernels, same
 * inputs).  A caller that runs every rank's dgrad first keeps one dU_ws per rank until that rank's wgrad. */
typedef enum { TP_BWD_ALL = 0, TP_BWD_DGRAD = 1, TP_BWD_WGRAD = 2 } tp_bwd_phase;
int tp_mlp_bwd_phase(const tp_dims* dims, int rank, tp_act act, tp_dtype dtype, tp_bwd_phase phase, const void* X,
                     const void* A_i, const void* B_i, const void* U_i, const void* Y_i, const void* dZ, void* dU_ws,
                     void* dA_i, void* da_i, void* dB_i, void* dX_i, hipStream_t stream);

/* Attention forward of rank `rank` for its a/t local query heads and g/t local KV heads ([ATLAS] §3, [MEGA]: QKV
 * column-parallel by head (by query group under GQA), per-head softmax(Q K^T / sqrt d) V on the local heads,
 * output projection row-parallel; [SPCP] CP step 3: the online-softmax merge over key blocks).  n = (a/t + 2g/t)d:
 *   QKV_i = X Wqkv_i (+ bqkv_i)     [s, b, n]: per local KV group, the d columns of each of its a/g query heads,
 *                                   then its d key and d value columns (g = a: [q_j | k_j | v_j] per head)
 *   O_i   = per query head j: softmax(Q_j K_j'^T / sqrt(d), causal: key k visible to query q iff k <= q) V_j'
 *           with j' = j's KV head (its group)   [s, b, (a/t)*d], head j at columns j*d .. j*d+d-1
 *   lse_i = log sum_k exp(S[q, k]) per (b, local head, q), fp32 [b, a/t, s] (nullable)
 *   Z_i   = O_i Wo_i                [s, b, h], a partial sum (no row bias)
 * Wqkv_i [h, n] and Wo_i [(a/t)*d, h] as produced by tp_shard_weights.  bf16 path: d % 8 == 0, d <= 128.
 * fp32 path: d <= 128.  The bf16 path may use Z_i as fp32 scratch for the QKV GEMM (split-K partials when that
 * GEMM has too few output tiles to fill the GPU) before the projection writes it. */
int tp_attn_fwd(const tp_dims* dims, int rank, tp_dtype dtype, int causal, const void* X, const void* Wqkv_i,
                const void* bqkv_i, const void* Wo_i, void* QKV_i, void* O_i, float* lse_i, void* Z_i,
                hipStream_t stream);

/* Attention backward of rank `rank` for its a/t local query heads (g/t KV heads), given the upstream gradient dZ of the block output
 * ([ATLAS] §2 and §5: g's backward is the identity, so every rank receives the full dZ (gathered under SP); the
 * row-parallel projection's weight gradient and the column-parallel QKV's weight gradient stay local, the data
 * gradient dX is a partial that f sums over ranks; [SPLIT] backward of the column and row splits):
 *   dO_ws   = dZ Wo_i^T                          [s, b, (a/t)*d]    caller workspace (activation dtype)
 *   rec_ws  = per (b, local head, 64-query block) [-lse*log2(e) (64) | D (64) | padding (128)], D[q] =
 *             sum_e dO[q,e] O[q,e] (0 past the sequence)
 *                                                fp32 [b, a/t, ceil(s/64), 256], caller workspace; with g < a it
 *             also holds the per-query-head partial dK | dV of each KV head (fp32 [a/g][s*b][g/t][2d]), summed in a
 *             fixed order: size tp_attn_bwd_workspace(dims) bytes
 *   dQKV_i  = per query head dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d), dV = P^T dO with P recomputed from
 *             lse_i (P = exp(S - lse)) and dS = P * (dO V^T - D); a KV head's dK, dV sum over the query heads
 *             of its group                       [s, b, n], grouped like QKV_i
 *   dWqkv_i = X^T dQKV_i                         [h, n]            local weight gradient
 *   dbqkv_i = column sums of dQKV_i (nullable)   [n]
 *   dWo_i   = O_i^T dZ                           [(a/t)*d, h]      local weight gradient
 *   dX_i    = dQKV_i Wqkv_i^T                    [s, b, h]         a partial: f sums them over ranks
 * QKV_i, O_i and lse_i (not nullable here) are the forward's outputs for the same inputs and `causal`.  The
 * alignment and head-size rules of tp_attn_fwd apply; outputs and workspaces must not overlap the inputs.  The
 * bf16 path may use dX_i as fp32 scratch for the dO GEMM (split-K partials) before the last GEMM writes it. */
int tp_attn_bwd(const tp_dims* dims, int rank, tp_dtype dtype, int causal, const void* X, const void* Wqkv_i,
                const void* Wo_i, const void* QKV_i, const void* O_i, const float* lse_i, const void* dZ, void* dO_ws,
                float* rec_ws, void* dQKV_i, void* dWqkv_i, void* dbqkv_i, void* dWo_i, void* dX_i,
                hipStream_t stream);

/* Bytes of the rec_ws workspace tp_attn_bwd needs for dims (0 for invalid dims). */
int64_t tp_attn_bwd_workspace(const tp_dims* dims);

/* g in forward / f in backward, all-reduce form ([ATLAS] §2; [SPLIT] row-parallel merge is a sum):
 *   out[e] = sum_{i=0}^{t-1} partials[i*n + e]  (+ bias_c[e % h])
 * partials is [t][n] contiguous.  Sum in fp32 in rank order 0..t-1, the bias (nullable, [h]) added last, one
 * rounding to the output dtype (bf16: nearest, ties to even; NaN stays NaN).  Needs n % h == 0. */
int tp_partial_reduce(int64_t n, int64_t h, int t, tp_dtype dtype, const void* partials, const void* bias_c,
                      void* out, hipStream_t stream);

/* g-bar under sequence parallelism: reduce-scatter along dim 0 of [s, b, h] ([ATLAS] §1, §5; [SPCP] SP section):
 * rank r receives rows [r*s/t, (r+1)*s/t) of the sum over the t partials [t][s, b, h], same arithmetic as
 * tp_partial_reduce.  rank == -1 writes every rank's slice, out = [t][s/t, b, h].  Needs s % t == 0. */
int tp_reduce_scatter_dim0(const tp_dims* dims, int rank, tp_dtype dtype, const void* partials, const void* bias_c,
                           void* out, hipStream_t stream);

/* SP entry (forward all-gather along dim 0, [ATLAS] §1 gather along the first dim; [SPCP] SP section):
 * out [s, b, h] = concatenation of the t slices [t][s/t, b, h] in rank order, bit for bit.  Needs s % t == 0. */
int tp_gather_dim0(const tp_dims* dims, tp_dtype dtype, const void* slices, void* out, hipStream_t stream);

/* Sequence-parallel region, forward: dropout + residual add + LayerNorm on one rank's slice of the residual
 * stream.  Under sequence parallelism the per-token ops between two tensor-parallel blocks run on the rank's own
 * rows [s/t, b, h] ([ATLAS] §5 SP rows, §6; [MEGA] sequence_parallel remark; [SPCP] SP section): the block output
 * z arrives by the dim-0 reduce-scatter, and y leaves by the dim-0 all-gather into the next column GEMM.  The pages
 * name these ops without formulas; this computes the standard definitions, per row of rows = (s/t)*b rows of h:
 *   keep = (bits >= floor(p * 2^32))                    element-wise, one uint32 random word per element
 *   u    = (residual or 0) + (keep ? z / (1 - p) : 0)   rounded once to dtype; written to out if out != NULL
 *   y    = (u - mean) * rstd * gamma + beta,  mean / biased variance over the row, rstd = 1 / sqrt(var + eps)
 * with the LayerNorm reading the rounded u.  mean, rstd: fp32 [rows] (nullable; the backward needs them).
 * y may be NULL when out, mean and rstd are given: the call then writes only u and the row statistics, which is
 * what tp_ln_mlp_fwd (the LayerNorm folded into the column GEMM) reads -- out pointing into rank r's rows of the
 * gathered [s, b, h] buffer makes that buffer the gathered LayerNorm input.
 * mask (nullable): [rows, h/8] bytes, bit i of byte k = keep of column 8k + i (LSB first); the backward reads it
 * instead of the words.  p == 0 keeps every element (bits may be NULL; scale 1).  y may point into rank r's rows
 * of the gathered [s, b, h] buffer (offset r*(s/t)*b*h): the local part of the all-gather is then this write.
 * Tensors are dtype except bits, mean, rstd, mask; gamma, beta [h].  Needs 0 <= p < 1, eps >= 0, h % 8 == 0,
 * h <= 12288 and every tensor pointer except mean, rstd and mask 16-byte aligned (else TP_E_UNSUPPORTED /
 * TP_E_SHAPE).  Outputs must not overlap inputs or each other (TP_E_ALIAS). */
int tp_sp_dropout_add_ln_fwd(int64_t rows, int64_t h, tp_dtype dtype, double p, double eps, const void* z,
                             const void* residual, const uint32_t* bits, const void* gamma, const void* beta,
                             void* out, void* y, float* mean, float* rstd, uint8_t* mask, hipStream_t stream);

/* Sequence-parallel region, backward of tp_sp_dropout_add_ln_fwd on the same rank's rows.  dy is the gradient
 * of y (it arrives by the dim-0 reduce-scatter of the next block's dX, [ATLAS] §5: the backward of SP's f is a
 * reduce-scatter); dres_in (nullable = 0) is the residual stream's gradient from above.  With xh = (u - mean) *
 * rstd and g = dy * gamma:
 *   G      = dres_in + rstd * (g - mean_h(g) - xh * mean_h(g * xh))   -> dres (nullable), the gradient of residual
 *   dz     = keep ? G / (1 - p) : 0                                    -> dz (nullable), the gradient of z
 *   dgamma = sum over rows of dy * xh,  dbeta = sum over rows of dy    -> fp32 [h] each, this rank's rows only
 * u, mean, rstd and mask are the forward's out, mean, rstd and mask (mask read only when p > 0).  Under sequence
 * parallelism each rank holds part of the LayerNorm weight gradient: sum the t ranks' dgamma / dbeta (e.g.
 * tp_partial_reduce with TP_F32).  ws: fp32 scratch of tp_sp_ln_bwd_workspace(rows, h) bytes, 16-byte aligned;
 * dgamma and dbeta 16-byte aligned.  Sums over rows run in a fixed order: results are deterministic.  Same size,
 * alignment and alias rules as the forward. */
int tp_sp_dropout_add_ln_bwd(int64_t rows, int64_t h, tp_dtype dtype, double p, const void* u, const void* gamma,
                             const float* mean, const float* rstd, const void* dy, const void* dres_in,
                             const uint8_t* mask, void* dres, void* dz, float* dgamma, float* dbeta, float* ws,
                             hipStream_t stream);

/* Bytes of fp32 scratch tp_sp_dropout_add_ln_bwd needs for rows x h (one partial [dgamma | dbeta] row per
 * workgroup of the row loop); <= 0 for non-positive sizes. */
int64_t tp_sp_ln_bwd_workspace(int64_t rows, int64_t h);

/* tp_sp_dropout_add_ln_bwd for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation and kernels, bit for bit, with no ws
 * argument.  The partial rows go to a fixed 16 MiB buffer inside the library instead, one per GPU, held until the
 * process ends (looked up on a device's first call, with that device current).  Calls that need more than that,
 * tp_sp_ln_bwd_workspace(rows, h) > 16 MiB (e.g. h > 8192 with 256 or more rows), return TP_E_SCRATCH before any
 * HIP call.  The call allocates and frees nothing.  Every call on one GPU shares that GPU's buffer: calls that
 * overlap on one GPU (on different streams, or from different threads) race and must be serialised by the
 * caller.  `stream` must belong to the current device.  Other arguments, rules and errors as in
 * tp_sp_dropout_add_ln_bwd. */
int tp_sp_dropout_add_ln_bwd_noalloc(int64_t rows, int64_t h, tp_dtype dtype, double p, const void* u,
                                     const void* gamma, const float* mean, const float* rstd, const void* dy,
                                     const void* dres_in, const uint8_t* mask, void* dres, void* dz, float* dgamma,
                                     float* dbeta, hipStream_t stream);

/* Vocab-parallel cross entropy ([ATLAS] §5 table, the vocab-parallel CE row: all-reduce(max), then all-reduce(sum),
 * backward local; [MEGA] embedding remark: the column-parallel logits feed the loss directly, so only b*s scalars
 * per reduction cross ranks).  Rank r holds logits_i [rows, v_local] for vocab columns [r*v_local, (r+1)*v_local)
 * of every token row (rows = s*b).  targets: int32 [rows], global vocab ids in [0, t*v_local); a negative target
 * marks an ignored row (loss 0, zero gradient).  A target >= t*v_local is in no rank's range: combine writes NaN to
 * that row's loss and lse, so the backward's gradient row is NaN too (never a silently wrong value).
 *
 * Local pass: stats_i float4 [rows] = {m_r, s_r, tl_r, o_r} with m_r the row max of this rank's logits, s_r the sum
 * of exp(x - m_r) over them, tl_r the target's logit when the target is one of this rank's columns, else 0, and
 * o_r = 1 when it is, else 0. */
int tp_vocab_ce_fwd_local(int64_t rows, int64_t v_local, int rank, tp_dtype dtype, const void* logits_i,
                          const int32_t* targets, float* stats_i, hipStream_t stream);

/* The two all-reduces, on one GPU over the t ranks' records stats [t][rows] float4 (rank order):
 *   m = max_r m_r;  S = sum_r s_r exp(m_r - m);  lse = m + log S;  loss = lse - sum_r tl_r  (0 for ignored rows)
 * A row whose logits are all -inf gets lse = -inf and loss NaN; a counted row that no rank owns (sum_r o_r = 0)
 * gets NaN in both. 
 * loss: fp32 [rows]; lse: fp32 [rows] (nullable; the backward needs it).  stats 16-byte aligned. */
int tp_vocab_ce_combine(int64_t rows, int t, const float* stats, const int32_t* targets, float* loss, float* lse,
                        hipStream_t stream);

/* Local backward: dlogits_i[i, j] = (exp(x[i, j] - lse[i]) - [r*v_local + j == target[i]]) * dloss[i], zero rows
 * for ignored targets.  dloss fp32 [rows] (e.g. 1 / the number of counted rows for a mean loss).  logits_i and
 * dlogits_i in dtype, 16-byte aligned; v_local % 8 == 0 for both calls on logits (else TP_E_UNSUPPORTED). */
int tp_vocab_ce_bwd(int64_t rows, int64_t v_local, int rank, tp_dtype dtype, const void* logits_i,
                    const int32_t* targets, const float* lse, const float* dloss, void* dlogits_i,
                    hipStream_t stream);

/* LayerNorm folded into the column GEMM ([MEGA] the TE LayerNormColumnParallelLinear remark: the LayerNorm before
 * a column-parallel GEMM is fused with it; [ATLAS] §5, SP rows: under sequence parallelism the LayerNorm runs on
 * each rank's rows and its output is all-gathered into the GEMM).  With y = LayerNorm(u) = (u - mean) rstd gamma
 * + beta per row, y A_i = rstd (u A' - mean c) + b with A' = diag(gamma) A_i, c = the column sums of A' and
 * b = beta A_i: the GEMM reads the gathered LayerNorm input u itself and applies the row statistics in its
 * epilogue, so the LayerNorm output is never written or read.
 *
 * tp_ln_fold_weights: A_ln = bf16(gamma[k] A_i[k][j]) [h, N1] (the product of two bf16 values is exact in fp32, so
 *   this is one rounding), c_ln[j] = sum_k A_ln[k][j] and b_ln[j] = sum_k beta[k] A_i[k][j] + a_i[j] (fp32 [N1],
 *   fixed summation order).  gamma, beta [h]; A_i [h, N1] and a_i [N1] (nullable) as for tp_mlp_fwd.  Runs once
 *   per weight (and gamma / beta) update, off the step.
 * tp_ln_mlp_fwd: tp_mlp_fwd on y = LayerNorm(X) without forming y: U_i = rstd (X A_ln - mean c_ln) + b_ln
 *   (= y A_i + a_i), Y_i = act(U_i), Z_i = Y_i B_i.  X [s, b, h] is the LayerNorm input (u, gathered under SP);
 *   ln_mean, ln_rstd fp32 [s*b] its row statistics as tp_sp_dropout_add_ln_fwd writes them.  The backward is
 *   tp_mlp_bwd with X = y: the weight gradient needs y, which tp_sp_dropout_add_ln_fwd gives again from u (p = 0,
 *   z = u, no residual), bit for bit the y of the unfolded forward.
 * Both: bf16 only, h % 64 == 0 and h >= 128 (the large-tile kernel), ffn/t % 8 == 0, pointers 16-byte aligned
 * (else TP_E_UNSUPPORTED); other rules as tp_mlp_fwd. */
int tp_ln_fold_weights(const tp_dims* dims, tp_act act, tp_dtype dtype, const void* gamma, const void* beta,
                       const void* A_i, const void* a_i, void* A_ln, float* c_ln, float* b_ln, hipStream_t stream);
int tp_ln_mlp_fwd(const tp_dims* dims, int rank, tp_act act, tp_dtype dtype, const void* X, const float* ln_mean,
                  const float* ln_rstd, const void* A_ln, const float* c_ln, const float* b_ln, const void* B_i,
                  void* U_i, void* Y_i, void* Z_i, hipStream_t stream);

/* Vocab-parallel output layer ([MEGA] output-logits remark: the output (embedding) weight E [V, h] is split by
 * vocab rows, so each rank's GEMM gives its own logit columns and feeds the cross entropy above directly, with only
 * per-row scalars crossing ranks; [ATLAS] §5 table, the vocab-parallel CE row; [SPLIT] "Column Parallel" and its
 * backward).  Rank r holds E_i = E[r*v_local : (r+1)*v_local] [v_local, h], row-major (one row per vocab entry):
 *   forward:  logits_i = X E_i^T        [rows, v_local]  (rows = s*b token rows of X [rows, h])
 *   backward: dE_i     = dlogits_i^T X  [v_local, h]     local weight gradient
 *             dX_i     = dlogits_i E_i  [rows, h]        a partial: the input gradient is its sum over the t ranks
 *                                                        (tp_partial_reduce)
 * logits_i is what tp_vocab_ce_fwd_local / tp_vocab_ce_bwd read, and dlogits_i what tp_vocab_ce_bwd writes.  In the
 * backward either output may be NULL (not computed; its operand X or E_i may then be NULL too), not both.  bf16:
 * h and v_local multiples of 8, pointers 16-byte aligned (else TP_E_UNSUPPORTED).  Outputs must not overlap
 * inputs. */
int tp_vocab_logits_fwd(int64_t rows, int64_t h, int64_t v_local, tp_dtype dtype, const void* X, const void* E_i,
                        void* logits_i, hipStream_t stream);
int tp_vocab_logits_bwd(int64_t rows, int64_t h, int64_t v_local, tp_dtype dtype, const void* X, const void* E_i,
                        const void* dlogits_i, void* dX_i, void* dE_i, hipStream_t stream);

/* Launch timing, a profiling aid (not part of the block's arithmetic).  tp_timing_begin arms the calling thread:
 * every kernel launched by a later tp_* call on this thread is bracketed by hipEventRecord(starts[i], stream) and
 * hipEventRecord(stops[i], stream), for the first `capacity` launches (later ones run unrecorded).  The events are
 * created and owned by the caller (hipEventCreate).  tp_timing_end disarms and returns the number of launches
 * recorded; tp_timing_kernel(i) names the i-th (static storage; NULL if out of range).  Arming the thread again
 * restarts the log.  Returns TP_E_NULL for NULL arrays, TP_E_SHAPE for capacity <= 0. */
int tp_timing_begin(hipEvent_t* starts, hipEvent_t* stops, int capacity);
int tp_timing_end(void);
const char* tp_timing_kernel(int i);
/* Restrict the calling thread's log to launches whose kernel name starts with `prefix` (NULL: record all), so that
 * a timed region can bracket only the kernels it reports (each recorded event pair costs launch latency).  Kept
 * until changed; TP_E_SHAPE for a prefix of 64 characters or more. */
int tp_timing_filter(const char* prefix);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
