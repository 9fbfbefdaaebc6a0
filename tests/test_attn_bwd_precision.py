"""Why the bf16 attention backward feeds P, dS, P*dP to the matrix cores as bf16 hi + lo pairs, and takes D from
its own pass over the keys: a CPU emulation of those kernels' precision choices against the oracle, under the same
element bound the GPU parity tests apply (max(3e-2 RMS, 2^-7 |ref|), tests/parity_utils.py).

The backward of one head follows the chain rule written out in "visual reading of Megatron-LM tensor parallelism"
(attention split by heads; each head's softmax backward is local) and the online-softmax statistics of "Sequence
Parallel 与 Context Parallel" (P recomputed from the forward's log-sum-exp).  The kernels:
  * dK/dV pass: dV = P^T dO, dK = dS^T Q / sqrt(d), with dS = P (dP - D), dP = dO V^T;
  * dQ pass, which runs first and does not know D: dQ = (A - D B) / sqrt(d) with A = sum_k (P dP) K, B = sum_k P K,
    D = sum_k P dP (one walk over the keys gathers all three).
Everything is fp32 on the GPU except the matrix-core operands, which are bf16.  The emulation keeps fp64 for the
fp32 steps (fp32 accumulation adds about 2^-24 relative, far below the bf16 effects studied here) and rounds to bf16
exactly where the kernels do: the stored inputs (Q, K, V, dO), each matrix operand, and the outputs (once).  An
operand is either one bf16 value, or a pair hi = bf16(x), lo = bf16(x - hi) whose two products sum to x within
about 2^-17 of it.

Inputs: the 22B-class attention shape (h = 6144, 64 heads of 96, s = 4096, t = 8, causal) from tp_inputs, rank 0's
QKV_i = X Wqkv_i and dO = dZ Wo_i^T rounded to bf16 as the block stores them, heads 0 and 3.  The reference is
the oracle's core backward on those same stored inputs.  Findings, each asserted below:
  * with the pairs, every output sits at its own bf16 rounding (about 0.015 of the unit), half the bound;
  * each single-bf16 operand alone pushes its output past the bound: P in dV (about 0.040), dS in dK (0.033),
    P dP in A (0.061), P in B (0.055) -- so all four pairs are needed;
  * D taken as the row sum of dO * O with the stored bf16 O (the usual shortcut, which would let dQ use dS
    directly) is past the bound even with exact dS (dQ 0.036, dK 0.038).
"""
import math

import numpy as np
import pytest

import oracle as O
import tp_inputs as TI
from parity_utils import BF16_MAX_ABS_UNIT, max_err_unit_scale

HEADS = (0, 3)


def bf(x):
    return O.stored(x, "bf16")


def pair(x):
    """hi + lo as the kernels form them from an fp32 value (the sum of the two bf16 operands' products)."""
    x32 = np.asarray(x, dtype=np.float32).astype(np.float64)
    hi = bf(x32)
    return hi + bf(x32 - hi)


@pytest.fixture(scope="module")
def emulated():
    w = TI.ATTN_22B
    inp = TI.attn_inputs(w, seed=0)
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], "bf16").reshape(w.M, w.h)
    Wqkv, Wo = O.as_f64(inp["Wqkv"], "bf16"), O.as_f64(inp["Wo"], "bf16")
    hl, d, r = w.a // w.t, w.d, 0
    QKV = bf(X @ Wqkv[:, O.qkv_shard_columns(w.a, d, w.t, r)])
    dO = bf(dZ @ Wo[r * hl * d:(r + 1) * hl * d].T)
    sc = 1.0 / math.sqrt(d)
    refs = {n: [] for n in "QKV"}
    out = {}
    for jj in HEADS:
        base = jj * 3 * d
        Q, K, V = (QKV[:, base + n * d: base + (n + 1) * d] for n in range(3))
        G = dO[:, jj * d:(jj + 1) * d]
        for n, ref in zip("QKV", O.attention_core_backward(Q, K, V, G, True)):
            refs[n].append(ref)
        s = Q.shape[0]
        S = (Q @ K.T) * sc
        S[np.triu(np.ones((s, s), dtype=bool), k=1)] = -np.inf
        m = S.max(axis=1, keepdims=True)
        lse = m + np.log(np.exp(S - m).sum(axis=1, keepdims=True))
        P = np.exp(S - lse)                       # from the forward's log-sum-exp, as the kernels recompute it
        dP = G @ V.T
        D = (P * dP).sum(axis=1, keepdims=True)   # exact: the dQ pass sums P dP in fp32
        dS = P * (dP - D)
        Ob = bf(P @ V)                            # the forward's stored output
        D_o = (G * Ob).sum(axis=1, keepdims=True)
        forms = {
            ("V", "pairs"): pair(P).T @ G,
            ("V", "single P"): bf(P).T @ G,
            ("K", "pairs"): pair(dS).T @ Q * sc,
            ("K", "single dS"): bf(dS).T @ Q * sc,
            ("Q", "pairs"): (pair(P * dP) @ K - D * (pair(P) @ K)) * sc,
            ("Q", "single P dP in A"): (bf(P * dP) @ K - D * (pair(P) @ K)) * sc,
            ("Q", "single P in B"): (pair(P * dP) @ K - D * (bf(P) @ K)) * sc,
            ("Q", "D from stored O"): (P * (dP - D_o)) @ K * sc,
            ("K", "D from stored O"): (P * (dP - D_o)).T @ Q * sc,
        }
        for key, val in forms.items():
            out.setdefault(key, []).append(bf(val))
    return {key: max_err_unit_scale(np.concatenate(v, axis=1), np.concatenate(refs[key[0]], axis=1))
            for key, v in out.items()}


def test_pairs_stay_at_the_output_rounding(emulated):
    for n in "QKV":
        assert emulated[(n, "pairs")] <= 0.6 * BF16_MAX_ABS_UNIT, (n, emulated[(n, "pairs")])


@pytest.mark.parametrize("key", [("V", "single P"), ("K", "single dS"), ("Q", "single P dP in A"),
                                 ("Q", "single P in B")])
def test_each_single_bf16_operand_breaks_the_bound(emulated, key):
    assert emulated[key] > BF16_MAX_ABS_UNIT, (key, emulated[key])


def test_d_from_the_stored_output_breaks_the_bound(emulated):
    assert emulated[("Q", "D from stored O")] > BF16_MAX_ABS_UNIT
    assert emulated[("K", "D from stored O")] > BF16_MAX_ABS_UNIT
