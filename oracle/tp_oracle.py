"""Oracle for the column->row tensor-parallel block: plain, slow, obviously correct NumPy in float64.

TEST INFRASTRUCTURE.  Only the tests, __graft_entry__.smoke() and the CPU-baseline leg of bench.py may import or
call anything in this package.  It shares no code with the HIP library and never imports it; the two meet only in
the seeded inputs of tp_inputs.

Pages followed (cited by title and section):
  [ATLAS]  "Tensor Parallelism (TP) 与 Sequence Parallelism (SP)", llm-infra-atlas, parallel/02_tp_sp
  [SPLIT]  111qqz.com, "tensor-parallelism-matrix-split" (the X in R^{Bx4}, W in R^{4x8}, two-GPU walk-through)
  [MEGA]   blog.vllbc.top, visual reading of Megatron-LM tensor parallelism (calculator, divisibility rules)
  [SPCP]   blog.vllbc.top, "Sequence Parallel 与 Context Parallel" (SP all-gather in / reduce-scatter out; the
           online-softmax merge of CP step 3)

What is computed: the unsharded block by its plain definition (Z = act(X A + a) B + c and its gradients; causal
multi-head attention), each rank's shard by slicing the unsharded operands ([ATLAS] §2: the sum over shards equals
the unsharded result in exact arithmetic), and the g / g-bar reductions as sums over the t partial buffers.
Activations are [s, b, h] sequence-first ([ATLAS] §1); every GEMM sees them as [s*b, h] rows in s-major order.

Readings where the pages are silent (each also listed in the design notes):
  * GeLU is the erf form; the tanh form is provided as a variant.
  * SwiGLU: the fc1 weight is [h, 2*ffn] = [gate | up]; Y = SiLU(X Ag + ag) * (X Au + au); rank i owns gate
    columns C_i and up columns C_i, packed [gate_i | up_i].
  * The row-parallel bias c is added once, after the reduction, never per partial.
  * Attention: fused QKV weight [h, 3ad] = [Wq | Wk | Wv] with head-major columns; rank r's shard groups each
    local head's columns as [q_j | k_j | v_j]; causal mask lets query q see keys k <= q; scale exactly 1/sqrt(d).
  * Partial sums are stored in the activation dtype; the bit-exact reduction adds them in fp32 in rank order
    0..t-1, adds the bias last, then rounds once to bf16 (nearest, ties to even); NaN stays NaN.

The SP-region ops (LayerNorm, dropout + residual) are the plain per-row / per-element definitions; dropout takes
its random words as an input (tp_inputs draws them), so both sides make the same keep decisions.

Vocab-parallel cross entropy follows the pages' steps (per-rank max, all-reduce(max), per-rank sum of exponentials
and target logit, all-reduce(sum)); a negative target marks an ignored row.

The attention backward (core and block) follows the chain rule through the row softmax as written out in
attention_core_backward; it is pinned by finite differences of the forward, torch's fp64 autograd, closed forms
and softmax invariants (tests/test_oracle_attention_bwd.py).

Every function here is pinned by the CPU tests (tests/test_oracle_*.py) against values the pages print, closed
forms, finite differences, brute force on tiny inputs, or an independent library routine.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

# ---------------------------------------------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bfloat16 patterns (uint16): a bf16 value is the fp32 value whose top 16 bits are the pattern."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 patterns: nearest, ties to even; NaN maps to a quiet NaN of the same sign.

    The 16 discarded bits decide the rounding: above half rounds up, below half truncates, exactly half rounds to
    the even kept pattern.  Overflow past the largest finite bf16 becomes infinity (carry into the exponent)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    kept = u >> np.uint64(16)
    low = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    round_up = (low > half) | ((low == half) & ((kept & np.uint64(1)) == np.uint64(1)))
    out = kept + round_up.astype(np.uint64)
    is_nan = ((u & np.uint64(0x7F800000)) == np.uint64(0x7F800000)) & ((u & np.uint64(0x007FFFFF)) != 0)
    out = np.where(is_nan, kept | np.uint64(0x0040), out)
    return out.astype(np.uint16)


def stored(x: np.ndarray, dtype: str) -> np.ndarray:
    """The value a device keeps when it stores x in `dtype`: fp32 rounding of x, then (bf16) one more rounding to
    bfloat16 nearest-even -- the storage precision of an intermediate the ABI hands back (e.g. QKV_i)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f64(f32_to_bf16_bits(x32))
    return x32.astype(np.float64)


def _keep(x: np.ndarray, store: Optional[str]) -> np.ndarray:
    """x as the block stores it between two steps: unchanged for store=None (the exact chain), else stored(x)."""
    return x if store is None else stored(x, store)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form (uint16 bf16 patterns or float32) to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------------------------------
# Element-wise activations and their derivatives ([ATLAS] §2: the nonlinearity is element-wise, so it runs on
# each column shard locally; [SPLIT] two-layer section uses ReLU)
# ---------------------------------------------------------------------------------------------------------------

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)
_TANH_C = math.sqrt(2.0 / math.pi)


def gelu(x):
    """GeLU(x) = x * Phi(x) with Phi the standard normal CDF = (1 + erf(x / sqrt 2)) / 2."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / _SQRT2))


def gelu_grad(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x), phi the standard normal density."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + _erf(x / _SQRT2)) + x * _INV_SQRT_2PI * np.exp(-0.5 * x * x)


def gelu_tanh(x):
    """The tanh approximation of GeLU: x/2 * (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(_TANH_C * (x + 0.044715 * x ** 3)))


def gelu_tanh_grad(x):
    x = np.asarray(x, dtype=np.float64)
    u = _TANH_C * (x + 0.044715 * x ** 3)
    th = np.tanh(u)
    du = _TANH_C * (1.0 + 3.0 * 0.044715 * x * x)
    return 0.5 * (1.0 + th) + 0.5 * x * (1.0 - th * th) * du


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def silu_grad(x):
    sg = sigmoid(x)
    return sg * (1.0 + np.asarray(x, dtype=np.float64) * (1.0 - sg))


def relu(x):
    return np.maximum(np.asarray(x, dtype=np.float64), 0.0)


def relu_grad(x):
    return (np.asarray(x, dtype=np.float64) > 0.0).astype(np.float64)


ACTS = {
    "gelu": (gelu, gelu_grad),
    "gelu_tanh": (gelu_tanh, gelu_tanh_grad),
    "relu": (relu, relu_grad),
}


# ---------------------------------------------------------------------------------------------------------------
# One linear layer Y = X W split two ways across t devices ([SPLIT] "Column Parallel", "Row Parallel" and the
# backward section; math layout W [in, out])
# ---------------------------------------------------------------------------------------------------------------


def _col_ranges(n: int, t: int) -> List[slice]:
    if n % t != 0:
        raise ValueError(f"{n} is not divisible by t={t}")
    w = n // t
    return [slice(i * w, (i + 1) * w) for i in range(t)]


def column_parallel_linear(X: np.ndarray, W: np.ndarray, t: int) -> List[np.ndarray]:
    """Device i holds the output columns C_i of W and computes Y_i = X W[:, C_i]; the full Y is their concatenation."""
    return [X @ W[:, c] for c in _col_ranges(W.shape[1], t)]


def row_parallel_linear(X: np.ndarray, W: np.ndarray, t: int) -> List[np.ndarray]:
    """Device i holds input rows R_i of W and the matching input columns of X; it returns the partial X_i W_i, all
    of full output shape, whose sum is X W."""
    return [X[:, r] @ W[r, :] for r in _col_ranges(W.shape[0], t)]


def column_parallel_input_grad(dY_shards: Sequence[np.ndarray], W: np.ndarray, t: int) -> np.ndarray:
    """X feeds every column shard, so by the multivariate chain rule dX is the sum over shards of dY_i W_i^T."""
    total = None
    for dYi, c in zip(dY_shards, _col_ranges(W.shape[1], t)):
        g = dYi @ W[:, c].T
        total = g if total is None else total + g
    return total


def row_parallel_input_grads(dY: np.ndarray, W: np.ndarray, t: int) -> List[np.ndarray]:
    """Each X_i is a distinct variable used by one shard only: dX_i = dY W_i^T, no sum; dX is their concatenation."""
    return [dY @ W[r, :].T for r in _col_ranges(W.shape[0], t)]


def column_parallel_weight_grads(X: np.ndarray, dY_shards: Sequence[np.ndarray]) -> List[np.ndarray]:
    """dW_i = X^T dY_i uses only what device i holds: no communication."""
    return [X.T @ g for g in dY_shards]


# ---------------------------------------------------------------------------------------------------------------
# Dim-0 split / gather / reductions ([ATLAS] §1 split/gather/reduce-scatter along the first dim and the
# divisibility assertion; §2 f/g; [SPCP] SP: all-gather in, reduce-scatter out)
# ---------------------------------------------------------------------------------------------------------------


def split_dim0(x: np.ndarray, t: int, rank: int) -> np.ndarray:
    """Rank r's contiguous slice of the sequence dim: rows [r*s/t, (r+1)*s/t).  s must be divisible by t."""
    s = x.shape[0]
    if s % t != 0:
        raise ValueError(f"sequence length {s} is not divisible by t={t}")
    loc = s // t
    return x[rank * loc:(rank + 1) * loc]


def gather_dim0(slices: Sequence[np.ndarray]) -> np.ndarray:
    """All-gather along dim 0: concatenation of the ranks' slices in rank order."""
    return np.concatenate(list(slices), axis=0)


def allreduce_sum(partials: Sequence[np.ndarray], bias: Optional[np.ndarray] = None) -> np.ndarray:
    """g in forward (and f in backward): the element-wise sum of all ranks' partials (exact, fp64); the row bias,
    if any, is added once."""
    acc = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        acc = acc + np.asarray(p, dtype=np.float64)
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float64)
    return acc


def reduce_scatter_dim0(partials: Sequence[np.ndarray], t: int, rank: int,
                        bias: Optional[np.ndarray] = None) -> np.ndarray:
    """g-bar under sequence parallelism: rank r keeps its dim-0 slice of the sum over ranks."""
    return split_dim0(allreduce_sum(partials, bias), t, rank)


def reduce_f32_rank_order(partials_f32: Sequence[np.ndarray], bias_f32: Optional[np.ndarray] = None) -> np.ndarray:
    """The reduction as a device computes it: acc = p_0, then acc = fp32(acc + p_i) for i = 1..t-1 in rank order,
    then acc = fp32(acc + bias); every add rounds to nearest-even fp32 (numpy float32 addition)."""
    acc = np.array(partials_f32[0], dtype=np.float32, copy=True)
    for p in partials_f32[1:]:
        acc = (acc + np.asarray(p, dtype=np.float32)).astype(np.float32)
    if bias_f32 is not None:
        acc = (acc + np.asarray(bias_f32, dtype=np.float32)).astype(np.float32)
    return acc


def reduce_storage(partials: np.ndarray, dtype: str, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Bit-exact expected output of the on-device reduction, in storage form.

    partials: [t, ...] in storage form (uint16 bf16 patterns or float32); bias: [h] broadcast over the last dim.
    bf16: fp32 rank-order sum, bias last, one rounding to bf16.  f32: the fp32 rank-order sum itself."""
    if dtype == "bf16":
        p32 = [bf16_bits_to_f64(p).astype(np.float32) for p in partials]
        b32 = None if bias is None else bf16_bits_to_f64(bias).astype(np.float32)
        return f32_to_bf16_bits(reduce_f32_rank_order(p32, b32))
    p32 = [np.asarray(p, dtype=np.float32) for p in partials]
    b32 = None if bias is None else np.asarray(bias, dtype=np.float32)
    return reduce_f32_rank_order(p32, b32)


# ---------------------------------------------------------------------------------------------------------------
# Shard layout ([ATLAS] §2-3 and [MEGA]: fc1 column-sharded, fc2 row-sharded, QKV column-sharded by head, output
# projection row-sharded; [MEGA] divide() and the heads % t assertion)
# ---------------------------------------------------------------------------------------------------------------

W_FC1, W_FC1_GATE_UP, W_FC2, W_QKV, W_PROJ, B_FC1, B_FC1_GATE_UP, B_QKV = range(8)


def _need_div(n: int, t: int, what: str):
    if n % t != 0:
        raise ValueError(f"{what}={n} is not divisible by t={t}")


def local_head_ids(a: int, t: int, rank: int) -> List[int]:
    _need_div(a, t, "heads")
    hl = a // t
    return list(range(rank * hl, (rank + 1) * hl))


def qkv_shard_columns(a: int, d: int, t: int, rank: int, g: Optional[int] = None) -> np.ndarray:
    """Full-QKV column index of every column of rank r's grouped shard.  Full layout [Wq | Wk | Wv]: a*d query
    columns (head j at j*d .. j*d+d-1), then g*d key and g*d value columns (KV head, i.e. query group, j likewise).
    g = None means g = a (multi-head attention).  Query head j belongs to group j // (a/g).  Rank r owns groups
    r*g/t .. (r+1)*g/t - 1; per local group in order: the d columns of each of its a/g query heads, then its d key
    columns, then its d value columns -- the interleave [q1 q2 k1 v1 | q3 q4 k2 v2 | ...] of [MEGA]'s QKV remark,
    which for g = a is [q_j | k_j | v_j] per head."""
    g = a if g is None else g
    _need_div(a, g, "a (query heads) by g (KV heads)")
    _need_div(g, t, "g (KV heads)")
    G = a // g
    gl = g // t
    cols = []
    for grp in range(rank * gl, (rank + 1) * gl):
        for slot in range(G):
            base = (grp * G + slot) * d
            cols.extend(range(base, base + d))
        for base in (a * d + grp * d, a * d + g * d + grp * d):
            cols.extend(range(base, base + d))
    return np.asarray(cols, dtype=np.int64)


def shard_weight(kind: int, full: np.ndarray, t: int, rank: int, ffn: int = 0, a: int = 0, d: int = 0,
                 g: Optional[int] = None):
    """One rank's shard of a full weight or bias (any dtype; pure index selection)."""
    if kind == W_FC1:
        _need_div(full.shape[1], t, "ffn")
        w = full.shape[1] // t
        return full[:, rank * w:(rank + 1) * w].copy()
    if kind == B_FC1:
        _need_div(full.shape[0], t, "ffn")
        w = full.shape[0] // t
        return full[rank * w:(rank + 1) * w].copy()
    if kind in (W_FC1_GATE_UP, B_FC1_GATE_UP):
        f = full.shape[-1] // 2
        _need_div(f, t, "ffn")
        w = f // t
        idx = np.concatenate([np.arange(rank * w, (rank + 1) * w), f + np.arange(rank * w, (rank + 1) * w)])
        return np.take(full, idx, axis=-1).copy()
    if kind == W_FC2:
        _need_div(full.shape[0], t, "ffn")
        w = full.shape[0] // t
        return full[rank * w:(rank + 1) * w, :].copy()
    if kind in (W_QKV, B_QKV):
        return np.take(full, qkv_shard_columns(a, d, t, rank, g), axis=-1).copy()
    if kind == W_PROJ:
        hl = len(local_head_ids(a, t, rank))
        return full[rank * hl * d:(rank + 1) * hl * d, :].copy()
    raise ValueError(f"unknown weight kind {kind}")


# ---------------------------------------------------------------------------------------------------------------
# MLP block Z = act(X A + a) B + c and its backward ([ATLAS] §2; [SPLIT] two-layer MLP forward and backward;
# [MEGA] first layer GeLU(XA), second layer YB)
# ---------------------------------------------------------------------------------------------------------------


def _act_fwd(U: np.ndarray, act: str) -> np.ndarray:
    if act == "swiglu":
        f = U.shape[1] // 2
        return silu(U[:, :f]) * U[:, f:]
    return ACTS[act][0](U)


def _act_bwd(U: np.ndarray, dY: np.ndarray, act: str) -> np.ndarray:
    """Gradient with respect to the pre-activation U given dY (the element-wise local step of the backward)."""
    if act == "swiglu":
        f = U.shape[1] // 2
        g, u = U[:, :f], U[:, f:]
        return np.concatenate([dY * u * silu_grad(g), dY * silu(g)], axis=1)
    return dY * ACTS[act][1](U)


def mlp_forward(X: np.ndarray, A: np.ndarray, B: np.ndarray, act: str = "gelu",
                a_bias: Optional[np.ndarray] = None, c_bias: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Unsharded block.  X [M, h] (M = s*b rows, s-major), A [h, ffn] (SwiGLU: [h, 2ffn] = [gate|up]), B [ffn, h].
    Returns U = X A + a (pre-activation), Y = act(U), Z = Y B + c."""
    U = X @ A
    if a_bias is not None:
        U = U + a_bias
    Y = _act_fwd(U, act)
    Z = Y @ B
    if c_bias is not None:
        Z = Z + c_bias
    return {"U": U, "Y": Y, "Z": Z}


def mlp_backward(X: np.ndarray, A: np.ndarray, B: np.ndarray, U: np.ndarray, Y: np.ndarray, dZ: np.ndarray,
                 act: str = "gelu") -> Dict[str, np.ndarray]:
    """Gradients of the unsharded block for upstream gradient dZ:
    dY = dZ B^T, dB = Y^T dZ, dc = column sums of dZ, dU = dY * act'(U), dA = X^T dU, da = column sums of dU,
    dX = dU A^T."""
    dY = dZ @ B.T
    dB = Y.T @ dZ
    dc = dZ.sum(axis=0)
    dU = _act_bwd(U, dY, act)
    dA = X.T @ dU
    da = dU.sum(axis=0)
    dX = dU @ A.T
    return {"dY": dY, "dB": dB, "dc": dc, "dU": dU, "dA": dA, "da": da, "dX": dX}


def mlp_shard_columns(ffn: int, t: int, rank: int, act: str) -> np.ndarray:
    """Columns of the full fc1 output (U) that rank r owns, in its packed order."""
    _need_div(ffn, t, "ffn")
    w = ffn // t
    own = np.arange(rank * w, (rank + 1) * w)
    if act == "swiglu":
        return np.concatenate([own, ffn + own])
    return own


def mlp_shard_forward(X: np.ndarray, A: np.ndarray, B: np.ndarray, t: int, rank: int, act: str = "gelu",
                      a_bias: Optional[np.ndarray] = None, store: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Rank r's part of the forward, by slicing the unsharded operands: U_i = X A[:, C_i] + a[C_i], Y_i = act(U_i),
    Z_i = Y_i B[R_i, :] is a partial sum of full shape (no row bias).

    store = None is the exact chain.  store = "bf16" follows the block's data flow with 16-bit activations ([MEGA]
    calculator and [ATLAS] §5 size every activation at 2 bytes): Y_i is stored before the row GEMM reads it, and
    U_i is kept stored for the backward.  Each returned entry is the exact value of the step that produces it from
    its (stored) inputs, before that step's own rounding."""
    ffn = B.shape[0]
    cols = mlp_shard_columns(ffn, t, rank, act)
    w = ffn // t
    Ui = X @ A[:, cols]
    if a_bias is not None:
        Ui = Ui + a_bias[cols]
    Yi = _act_fwd(Ui, act)
    Zi = _keep(Yi, store) @ B[rank * w:(rank + 1) * w, :]
    return {"U": Ui, "Y": Yi, "Z": Zi}


def mlp_shard_backward(X: np.ndarray, A: np.ndarray, B: np.ndarray, dZ: np.ndarray, t: int, rank: int,
                       act: str = "gelu", a_bias: Optional[np.ndarray] = None,
                       store: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Rank r's part of the backward ([SPLIT] backward section): row layer dY_i = dZ B_i^T (no sum) and
    dB_i = Y_i^T dZ; local act' step; column layer dA_i = X^T dU_i (local) and the partial dX_i = dU_i A_i^T, whose
    sum over ranks is dX.  store as in mlp_shard_forward: the saved U_i and Y_i are the stored ones, and dU_i is
    stored before the two GEMMs (and the column sum) that read it."""
    ffn = B.shape[0]
    cols = mlp_shard_columns(ffn, t, rank, act)
    w = ffn // t
    fw = mlp_shard_forward(X, A, B, t, rank, act, a_bias)
    Bi = B[rank * w:(rank + 1) * w, :]
    dYi = dZ @ Bi.T
    dBi = _keep(fw["Y"], store).T @ dZ
    dUi = _act_bwd(_keep(fw["U"], store), dYi, act)
    dUs = _keep(dUi, store)
    dAi = X.T @ dUs
    dai = dUs.sum(axis=0)
    dXi = dUs @ A[:, cols].T
    return {"dY": dYi, "dB": dBi, "dU": dUi, "dA": dAi, "da": dai, "dX": dXi}


def mlp_shard_rows(X_rows: np.ndarray, dZ_rows: np.ndarray, A: np.ndarray, B: np.ndarray, t: int, rank: int,
                   act: str = "gelu", a_bias: Optional[np.ndarray] = None,
                   store: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Rank r's per-token results for a subset of token rows.  Every row of U_i, Y_i, Z_i, dU_i and dX_i depends
    only on the same row of X (and of dZ), so computing them for sampled rows is exact.  store as in
    mlp_shard_backward."""
    ffn = B.shape[0]
    cols = mlp_shard_columns(ffn, t, rank, act)
    w = ffn // t
    Bi = B[rank * w:(rank + 1) * w, :]
    Ai = A[:, cols]
    U = X_rows @ Ai
    if a_bias is not None:
        U = U + a_bias[cols]
    Y = _act_fwd(U, act)
    Z = _keep(Y, store) @ Bi
    dY = dZ_rows @ Bi.T
    dU = _act_bwd(_keep(U, store), dY, act)
    dX = _keep(dU, store) @ Ai.T
    return {"U": U, "Y": Y, "Z": Z, "dU": dU, "dX": dX}


def mlp_shard_weight_grad_cols(X: np.ndarray, dZ: np.ndarray, A: np.ndarray, B: np.ndarray, t: int, rank: int,
                               j_cols: Sequence[int], act: str = "gelu",
                               a_bias: Optional[np.ndarray] = None,
                               store: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Rank r's weight gradients restricted to shard columns j of the GeLU/ReLU output (for SwiGLU: j indexes the
    f/t output columns and both the gate column j and the up column f/t + j of dA_i are returned).
    dB_i[j, :] = Y_i[:, j]^T dZ and dA_i[:, j] = X^T dU_i[:, j] each need only column j of the activations, over
    all token rows, so sampling columns is exact.  store as in mlp_shard_backward."""
    ffn = B.shape[0]
    w = ffn // t
    j = np.asarray(j_cols, dtype=np.int64)
    Bj = B[rank * w + j, :]                      # rows of B_i for the sampled columns
    full_cols = mlp_shard_columns(ffn, t, rank, act)
    if act == "swiglu":
        sel = np.concatenate([j, w + j])          # gate j and up j within the packed shard
    else:
        sel = j
    cols = full_cols[sel]
    U = X @ A[:, cols]
    if a_bias is not None:
        U = U + a_bias[cols]
    Y = _act_fwd(U, act)                          # [M, len(j)]
    dY = dZ @ Bj.T
    dU = _keep(_act_bwd(_keep(U, store), dY, act), store)  # [M, len(sel)]
    return {"dB_rows": _keep(Y, store).T @ dZ, "dA_cols": X.T @ dU, "da_cols": dU.sum(axis=0), "sel": sel}


# ---------------------------------------------------------------------------------------------------------------
# Attention block ([ATLAS] §3; [MEGA]: QKV column-parallel by head, per-head softmax(Q K^T / sqrt d) V locally,
# output projection row-parallel, one reduction at the exit)
# ---------------------------------------------------------------------------------------------------------------


def attention_core(Q: np.ndarray, K: np.ndarray, V: np.ndarray, causal: bool = True):
    """One head of one sequence: Q, K, V [s, d].  S = Q K^T / sqrt(d) with S[q, k] = -inf for k > q when causal;
    P = row softmax of S; O = P V.  Also returns lse[q] = log sum_k exp(S[q, k]) over the visible keys."""
    s, d = Q.shape
    S = (Q @ K.T) / math.sqrt(d)
    if causal:
        mask = np.triu(np.ones((s, K.shape[0]), dtype=bool), k=1)
        S = np.where(mask, -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    den = E.sum(axis=1, keepdims=True)
    O = (E / den) @ V
    lse = (m + np.log(den))[:, 0]
    return O, lse


def _kv_cols(a: int, d: int, g: int, j: int):
    """Key and value column ranges of query head j in the full [Wq | Wk | Wv] layout (group j // (a/g))."""
    grp = j // (a // g)
    return slice(a * d + grp * d, a * d + (grp + 1) * d), slice(a * d + (g + grp) * d, a * d + (g + grp + 1) * d)


def shard_head_columns(G: int, d: int, jj: int):
    """Query, key and value column ranges of local query head jj in a grouped shard ([MEGA] interleave)."""
    base = (jj // G) * (G + 2) * d
    q0 = base + (jj % G) * d
    return slice(q0, q0 + d), slice(base + G * d, base + (G + 1) * d), slice(base + (G + 1) * d, base + (G + 2) * d)


def attention_forward(X: np.ndarray, Wqkv: np.ndarray, Wo: np.ndarray, s: int, b: int, a: int, d: int,
                      causal: bool = True, bqkv: Optional[np.ndarray] = None,
                      c_bias: Optional[np.ndarray] = None, g: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Unsharded attention block.  X [M = s*b, h] rows s-major; Wqkv [h, (a + 2g)d] = [Wq|Wk|Wv] (g KV heads,
    g = None for g = a); Wo [ad, h].  Query head j attends with key / value head j // (a/g) (grouped-query
    attention; [MEGA] QKV remark).  Returns QKV, O [M, ad] (head j at columns j*d..), lse [b, a, s],
    Z = O Wo + c."""
    g = a if g is None else g
    QKV = X @ Wqkv
    if bqkv is not None:
        QKV = QKV + bqkv
    ad = a * d
    O = np.zeros((s * b, ad))
    lse = np.zeros((b, a, s))
    for bi in range(b):
        rows = np.arange(s) * b + bi
        for j in range(a):
            ck, cv = _kv_cols(a, d, g, j)
            q = QKV[rows, j * d:(j + 1) * d]
            k = QKV[rows, ck]
            v = QKV[rows, cv]
            o, l = attention_core(q, k, v, causal)
            O[rows, j * d:(j + 1) * d] = o
            lse[bi, j, :] = l
    Z = O @ Wo
    if c_bias is not None:
        Z = Z + c_bias
    return {"QKV": QKV, "O": O, "lse": lse, "Z": Z}


def attention_shard_forward(X: np.ndarray, Wqkv: np.ndarray, Wo: np.ndarray, s: int, b: int, a: int, d: int,
                            t: int, rank: int, causal: bool = True,
                            bqkv: Optional[np.ndarray] = None, g: Optional[int] = None,
                            store: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Rank r's part: QKV_i in the grouped column order of qkv_shard_columns for its local groups, O_i = its query
    heads' outputs (head-major), lse_i [b, a/t, s], and the partial Z_i = O_i Wo[rows of its heads] (no row
    bias).  store = "bf16": QKV_i is stored before the attention reads it and O_i before the projection reads it
    (16-bit activations, as in mlp_shard_forward); each entry is the exact value of its step from stored inputs."""
    g = a if g is None else g
    G = a // g
    cols = qkv_shard_columns(a, d, t, rank, g)
    QKVi = X @ Wqkv[:, cols]
    if bqkv is not None:
        QKVi = QKVi + bqkv[cols]
    QKVk = _keep(QKVi, store)
    heads = local_head_ids(a, t, rank)
    hl = len(heads)
    Oi = np.zeros((s * b, hl * d))
    lsei = np.zeros((b, hl, s))
    for bi in range(b):
        rows = np.arange(s) * b + bi
        for jj in range(hl):
            cq, ck, cv = shard_head_columns(G, d, jj)
            o, l = attention_core(QKVk[rows, cq], QKVk[rows, ck], QKVk[rows, cv], causal)
            Oi[rows, jj * d:(jj + 1) * d] = o
            lsei[bi, jj, :] = l
    Zi = _keep(Oi, store) @ Wo[rank * hl * d:(rank + 1) * hl * d, :]
    return {"QKV": QKVi, "O": Oi, "lse": lsei, "Z": Zi}


def attention_rows(QKV_i: np.ndarray, s: int, b: int, hl: int, d: int, q_rows: Sequence[int],
                   causal: bool = True, G: int = 1) -> Dict[str, np.ndarray]:
    """Attention outputs for selected token rows only (row index = s_idx*b + b_idx), from a rank's grouped QKV_i
    (G query heads per KV head).  Each output row needs just its own query and the keys/values of its sequence,
    so sampling rows is exact."""
    q_rows = np.asarray(q_rows, dtype=np.int64)
    O = np.zeros((len(q_rows), hl * d))
    lse = np.zeros((len(q_rows), hl))
    for n, r in enumerate(q_rows):
        si, bi = divmod(int(r), b)
        nk = si + 1 if causal else s
        krows = np.arange(nk) * b + bi
        for jj in range(hl):
            cq, ck, cv = shard_head_columns(G, d, jj)
            q = QKV_i[r, cq]
            k = QKV_i[krows, ck]
            v = QKV_i[krows, cv]
            sc = (k @ q) / math.sqrt(d)
            m = sc.max()
            e = np.exp(sc - m)
            O[n, jj * d:(jj + 1) * d] = (e / e.sum()) @ v
            lse[n, jj] = m + math.log(e.sum())
    return {"O": O, "lse": lse}


def attention_core_backward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, causal: bool = True):
    """Gradients of one head's O = softmax(Q K^T / sqrt(d), causal) V for the upstream gradient dO, by the chain rule
    written out: dV = P^T dO; dP = dO V^T; the row softmax's Jacobian gives dS = P * (dP - rowsum(P * dP)); then
    S = Q K^T / sqrt(d) gives dQ = dS K / sqrt(d) and dK = dS^T Q / sqrt(d).  Masked entries have P = 0 and so no
    gradient.  Returns dQ, dK, dV (each [s, d])."""
    s, d = Q.shape
    S = (Q @ K.T) / math.sqrt(d)
    if causal:
        S = np.where(np.triu(np.ones((s, K.shape[0]), dtype=bool), k=1), -np.inf, S)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    P = E / E.sum(axis=1, keepdims=True)
    dV = P.T @ dO
    dP = dO @ V.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dQ = dS @ K / math.sqrt(d)
    dK = dS.T @ Q / math.sqrt(d)
    return dQ, dK, dV


def attention_backward(X: np.ndarray, Wqkv: np.ndarray, Wo: np.ndarray, dZ: np.ndarray, s: int, b: int, a: int,
                       d: int, causal: bool = True, bqkv: Optional[np.ndarray] = None,
                       g: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Gradients of the unsharded attention block Z = O Wo + c for the upstream dZ [M, h]: dO = dZ Wo^T,
    dWo = O^T dZ, dc = column sums of dZ; per (sequence, query head) the core gradients into dQKV ([Wq|Wk|Wv]
    column order), a KV head's dK and dV summing over the query heads of its group; dWqkv = X^T dQKV,
    dbqkv = column sums of dQKV, dX = dQKV Wqkv^T."""
    g = a if g is None else g
    fw = attention_forward(X, Wqkv, Wo, s, b, a, d, causal, bqkv, g=g)
    QKV, O = fw["QKV"], fw["O"]
    dO = dZ @ Wo.T
    dQKV = np.zeros_like(QKV)
    for bi in range(b):
        rows = np.arange(s) * b + bi
        for j in range(a):
            cq = slice(j * d, (j + 1) * d)
            ck, cv = _kv_cols(a, d, g, j)
            gq, gk, gv = attention_core_backward(QKV[rows, cq], QKV[rows, ck], QKV[rows, cv], dO[rows, cq], causal)
            dQKV[rows, cq] = gq
            dQKV[rows, ck] += gk
            dQKV[rows, cv] += gv
    return {"dO": dO, "dWo": O.T @ dZ, "dc": dZ.sum(axis=0), "dQKV": dQKV, "dWqkv": X.T @ dQKV,
            "dbqkv": dQKV.sum(axis=0), "dX": dQKV @ Wqkv.T, "O": O, "QKV": QKV, "lse": fw["lse"]}


def attention_shard_backward(X: np.ndarray, Wqkv: np.ndarray, Wo: np.ndarray, dZ: np.ndarray, s: int, b: int,
                             a: int, d: int, t: int, rank: int, causal: bool = True,
                             bqkv: Optional[np.ndarray] = None, g: Optional[int] = None,
                             store: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Rank r's part of the attention backward: its heads' dO_i = dZ Wo_i^T (Wo_i = the rows of its heads), the
    weight gradients dWo_i = O_i^T dZ, dQKV_i in the grouped [q_j k_j v_j] order, dWqkv_i = X^T dQKV_i,
    dbqkv_i, and the partial dX_i = dQKV_i Wqkv_i^T (the f reduction sums these over ranks).  store = "bf16": the
    forward's QKV_i and O_i are the stored ones (attention_shard_forward), dO_i is stored before the core
    backward reads it and dQKV_i before the two GEMMs (and the column sum) that read it."""
    g = a if g is None else g
    G = a // g
    fw = attention_shard_forward(X, Wqkv, Wo, s, b, a, d, t, rank, causal, bqkv, g=g, store=store)
    QKVi, Oi = _keep(fw["QKV"], store), _keep(fw["O"], store)
    hl = a // t
    Wo_i = Wo[rank * hl * d:(rank + 1) * hl * d, :]
    Wqkv_i = Wqkv[:, qkv_shard_columns(a, d, t, rank, g)]
    dOi = dZ @ Wo_i.T
    dOk = _keep(dOi, store)
    dQKVi = np.zeros_like(QKVi)
    for bi in range(b):
        rows = np.arange(s) * b + bi
        for jj in range(hl):
            cq, ck, cv = shard_head_columns(G, d, jj)
            gq, gk, gv = attention_core_backward(QKVi[rows, cq], QKVi[rows, ck], QKVi[rows, cv],
                                                 dOk[rows, jj * d:(jj + 1) * d], causal)
            dQKVi[rows, cq] = gq
            dQKVi[rows, ck] += gk
            dQKVi[rows, cv] += gv
    dQk = _keep(dQKVi, store)
    return {"dO": dOi, "dWo": Oi.T @ dZ, "dQKV": dQKVi, "dWqkv": X.T @ dQk, "dbqkv": dQk.sum(axis=0),
            "dX": dQk @ Wqkv_i.T, "O": fw["O"], "QKV": fw["QKV"], "lse": fw["lse"], "Z": fw["Z"]}


# ---------------------------------------------------------------------------------------------------------------
# Sequence-parallel region ([ATLAS] §5 "SP: g -> RS" / "SP: f -> AG" rows and §6; [MEGA] sequence_parallel note;
# [SPCP] "SP: all-gather in, reduce-scatter out": LayerNorm, dropout and the residual add are per-token / per-element
# and run on each rank's [s/t, b, h] slice between the reduce-scatter of one block and the all-gather of the next)
# ---------------------------------------------------------------------------------------------------------------


def layernorm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float):
    """Per row of x [rows, h]: mean, biased variance, y = (x - mean) / sqrt(var + eps) * gamma + beta.
    Returns y, mean [rows], rstd [rows] = 1 / sqrt(var + eps)."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=1)
    var = ((x - mean[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    return (x - mean[:, None]) * rstd[:, None] * gamma[None, :] + beta[None, :], mean, rstd


def layernorm_backward(x: np.ndarray, gamma: np.ndarray, dy: np.ndarray, eps: float):
    """Gradients of layernorm for the upstream dy: with xh = (x - mean) rstd and g = dy * gamma,
    dx = rstd (g - mean_h(g) - xh mean_h(g xh)); dgamma = sum over rows of dy xh; dbeta = sum over rows of dy."""
    x = np.asarray(x, dtype=np.float64)
    _, mean, rstd = layernorm(x, np.ones(x.shape[1]), np.zeros(x.shape[1]), eps)
    xh = (x - mean[:, None]) * rstd[:, None]
    g = dy * gamma[None, :]
    dx = rstd[:, None] * (g - g.mean(axis=1, keepdims=True) - xh * (g * xh).mean(axis=1, keepdims=True))
    return dx, (dy * xh).sum(axis=0), dy.sum(axis=0)


def ln_fold(gamma: np.ndarray, beta: np.ndarray, A: np.ndarray, a: Optional[np.ndarray] = None,
            store: Optional[str] = None):
    """The LayerNorm folded into the following column GEMM ([MEGA] remark on TE's LayerNormColumnParallelLinear,
    the LayerNorm fused with the column-parallel linear after it).  With y = (u - mean) rstd gamma + beta per row,
    y A + a = rstd (u A' - mean c) + b where A' = diag(gamma) A, c = the column sums of A' and b = beta A + a.
    store="bf16": A' is kept in bf16 (the product of two bf16 values is exact in fp32, so one rounding) and c sums
    the kept values, so the identity stays exact for the stored A'.  Returns A', c, b."""
    Af = np.asarray(gamma, dtype=np.float64)[:, None] * np.asarray(A, dtype=np.float64)
    Af = _keep(Af, store)
    b = np.asarray(beta, dtype=np.float64) @ np.asarray(A, dtype=np.float64)
    if a is not None:
        b = b + np.asarray(a, dtype=np.float64)
    return Af, Af.sum(axis=0), b


def ln_folded_linear(u: np.ndarray, mean: np.ndarray, rstd: np.ndarray, A_fold: np.ndarray, c: np.ndarray,
                     b: np.ndarray) -> np.ndarray:
    """rstd (u A' - mean c) + b per row: the column GEMM of the LayerNorm output computed from its input."""
    u = np.asarray(u, dtype=np.float64)
    return np.asarray(rstd, dtype=np.float64)[:, None] * (u @ A_fold - np.outer(mean, c)) + b


def dropout_keep(bits: np.ndarray, p: float) -> np.ndarray:
    """Keep decision from 32-bit random words: keep iff bits >= floor(p * 2^32), so P(keep) = 1 - p to 2^-32."""
    return np.asarray(bits, dtype=np.uint64) >= np.uint64(math.floor(p * 2.0 ** 32))


def dropout_add(z: np.ndarray, residual: np.ndarray, bits: np.ndarray, p: float) -> np.ndarray:
    """out = residual + keep * z / (1 - p) (inverted dropout on the block output, then the residual add)."""
    keep = dropout_keep(bits, p)
    return np.asarray(residual, dtype=np.float64) + np.where(keep, np.asarray(z, dtype=np.float64) / (1.0 - p), 0.0)


def dropout_add_backward(dout: np.ndarray, bits: np.ndarray, p: float):
    """Gradients of dropout_add: dz = keep * dout / (1 - p); dresidual = dout."""
    keep = dropout_keep(bits, p)
    dout = np.asarray(dout, dtype=np.float64)
    return np.where(keep, dout / (1.0 - p), 0.0), dout


# ---------------------------------------------------------------------------------------------------------------
# Vocab-parallel cross entropy ([ATLAS] §5 table: the vocab-parallel CE row, all-reduce(max) then all-reduce(sum),
# backward local; [MEGA] embedding / logits remark: the column-parallel logits feed the loss directly, so only b*s
# scalars per reduction cross ranks).  Targets are global vocab ids; a negative target marks an ignored row (loss 0,
# no gradient).
# ---------------------------------------------------------------------------------------------------------------


def cross_entropy(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Unsharded per-row loss: log(sum_j exp(logits[i, j])) - logits[i, targets[i]]; 0 where targets[i] < 0.

    Rows the definition leaves undefined give NaN, so they cannot pass for a loss: a target at or beyond the vocab
    size (no such logit), and a row whose logits are all -inf (log 0 - (-inf))."""
    x = np.asarray(logits, dtype=np.float64)
    tg = np.asarray(targets, dtype=np.int64)
    m = x.max(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = np.where(np.isneginf(m), -np.inf, m + np.log(np.exp(x - m[:, None]).sum(axis=1)))
        keep = tg >= 0
        inside = keep & (tg < x.shape[1])
        loss = np.zeros(x.shape[0])
        loss[keep] = np.nan
        loss[inside] = lse[inside] - x[np.nonzero(inside)[0], tg[inside]]
    return loss


def cross_entropy_backward(logits: np.ndarray, targets: np.ndarray, dloss: np.ndarray) -> np.ndarray:
    """Gradient of sum_i dloss[i] * loss[i]: (softmax(logits[i]) - onehot(targets[i])) * dloss[i]; 0 rows when
    ignored."""
    x = np.asarray(logits, dtype=np.float64)
    tg = np.asarray(targets, dtype=np.int64)
    e = np.exp(x - x.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    keep = tg >= 0
    rows = np.nonzero(keep)[0]
    p[rows, tg[keep]] -= 1.0
    p *= np.asarray(dloss, dtype=np.float64)[:, None]
    p[~keep] = 0.0
    return p


def vocab_parallel_cross_entropy(logit_shards: Sequence[np.ndarray], targets: np.ndarray):
    """The pages' sharded steps over t ranks, rank r holding vocab columns [r*v, (r+1)*v) of the logits:
    1. each rank's row max, then all-reduce(max) -> m;
    2. each rank's sum of exp(logits - m) and its target logit (0 when the target is not in its range), then
       all-reduce(sum) of both -> S, target logit;
    3. loss = log S + m - target logit (0 for ignored rows).  Returns loss and lse = m + log S per row.
    A target that no rank's range holds gives NaN for both loss and lse (the backward then gives NaN too); a row
    whose logits are all -inf gives lse = -inf and loss NaN, as in cross_entropy."""
    v = logit_shards[0].shape[1]
    tg = np.asarray(targets, dtype=np.int64)
    xs = [np.asarray(x, dtype=np.float64) for x in logit_shards]
    m = np.max(np.stack([x.max(axis=1) for x in xs]), axis=0)                       # all-reduce(max)
    sums, tls, owned = [], [], np.zeros(len(tg), dtype=bool)
    with np.errstate(invalid="ignore", divide="ignore"):
        for r, x in enumerate(xs):
            sums.append(np.where(np.isneginf(m), 0.0, np.exp(x - m[:, None]).sum(axis=1)))
            local = tg - r * v
            mine = (tg >= 0) & (local >= 0) & (local < v)
            owned |= mine
            tl = np.zeros(x.shape[0])
            tl[mine] = x[np.nonzero(mine)[0], local[mine]]
            tls.append(tl)
        S = np.sum(np.stack(sums), axis=0)                                           # all-reduce(sum)
        tl = np.sum(np.stack(tls), axis=0)
        lse = np.where(np.isneginf(m), -np.inf, m + np.log(S))
        lse = np.where((tg >= 0) & ~owned, np.nan, lse)
        loss = np.where(tg >= 0, lse - tl, 0.0)
    return loss, lse


def vocab_parallel_logits(X: np.ndarray, E: np.ndarray, t: int, rank: int) -> np.ndarray:
    """Rank r's logits of the vocab-sharded output layer ([MEGA] output-logits remark; [ATLAS] §5 vocab-parallel
    row): the output weight E [V, h] (one row per vocab entry, the embedding table's layout) is split by vocab rows,
    rank r holding E_r = E[r*V/t : (r+1)*V/t]; its logits are X E_r^T [rows, V/t], the columns
    [r*V/t, (r+1)*V/t) of the full X E^T."""
    V = E.shape[0]
    _need_div(V, t, "vocab")
    v = V // t
    return np.asarray(X, dtype=np.float64) @ np.asarray(E[rank * v:(rank + 1) * v], dtype=np.float64).T


def vocab_parallel_logits_backward(X: np.ndarray, E: np.ndarray, dlogits_r: np.ndarray, t: int, rank: int):
    """Gradients of rank r's logits X E_r^T for the upstream gradient dlogits_r [rows, V/t]: the local weight
    gradient dE_r = dlogits_r^T X [V/t, h], and the partial input gradient dX_r = dlogits_r E_r [rows, h], whose sum
    over the t ranks is the input gradient (the backward of a column-parallel layer, [SPLIT] "Column Parallel"
    backward)."""
    V = E.shape[0]
    _need_div(V, t, "vocab")
    v = V // t
    d = np.asarray(dlogits_r, dtype=np.float64)
    Er = np.asarray(E[rank * v:(rank + 1) * v], dtype=np.float64)
    return {"dX": d @ Er, "dE": d.T @ np.asarray(X, dtype=np.float64)}


def vocab_parallel_cross_entropy_backward(logits_r: np.ndarray, targets: np.ndarray, rank: int, lse: np.ndarray,
                                          dloss: np.ndarray) -> np.ndarray:
    """Rank-local backward: (exp(logits_r - lse) - [global column == target]) * dloss per row; 0 when ignored."""
    x = np.asarray(logits_r, dtype=np.float64)
    v = x.shape[1]
    tg = np.asarray(targets, dtype=np.int64)
    g = np.exp(x - np.asarray(lse, dtype=np.float64)[:, None])
    local = tg - rank * v
    mine = (tg >= 0) & (local >= 0) & (local < v)
    g[np.nonzero(mine)[0], local[mine]] -= 1.0
    g *= np.asarray(dloss, dtype=np.float64)[:, None]
    g[tg < 0] = 0.0
    return g


# ---------------------------------------------------------------------------------------------------------------
# Accounting ([MEGA] calculator: per-rank linear parameters (2hf + 4h^2)/t with MHA attention, all-reduce payload
# b*s*h elements per call, four calls per layer, ring traffic 8 b s h (t-1)/t elements per card; [ATLAS] §6)
# ---------------------------------------------------------------------------------------------------------------


def linear_params_per_rank(h: int, f: int, t: int) -> int:
    """Linear-layer weights one rank holds per layer: fc1 h*f + fc2 f*h + QKV 3h^2 + projection h^2, over t."""
    total = h * f + f * h + 3 * h * h + h * h
    if total % t != 0:
        raise ValueError("parameter count not divisible by t")
    return total // t


def allreduce_payload_elems(b: int, s: int, h: int) -> int:
    """One g (or f) all-reduce moves the whole activation [s, b, h], independent of t."""
    return b * s * h


def allreduce_calls_per_layer() -> int:
    """Attention and MLP each reduce once in forward (g) and once in backward (f)."""
    return 4


def ring_elems_per_card_per_layer(b: int, s: int, h: int, t: int) -> float:
    """A ring all-reduce moves 2 N (t-1)/t elements per card; four calls per layer."""
    return allreduce_calls_per_layer() * 2.0 * allreduce_payload_elems(b, s, h) * (t - 1) / t


# ---------------------------------------------------------------------------------------------------------------
# Error measures used by the parity tests
# ---------------------------------------------------------------------------------------------------------------


def rel_frobenius(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((got - ref).ravel()) / (den if den > 0 else 1.0))
