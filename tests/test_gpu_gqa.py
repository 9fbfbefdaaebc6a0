"""Grouped-query attention (g KV heads, a/g query heads each) through the C ABI, against the fp64 oracle.

* the QKV shard packer with g < a: bit for bit against the oracle's slicing (the pages' per-group interleave);
* forward and backward of every rank at small ragged shapes (s = 100: a partial 64-row tile), group sizes 2 to 4,
  one or two local groups, t up to 8 (split-K GEMMs), every head-dim bucket, causal and not, bf16 and fp32, with a QKV bias: O_i, lse_i, Z_i
  and dQKV_i (a KV head's dK / dV summed over its group's query heads), dWqkv_i, dbqkv_i, dWo_i, dX_i;
* the Llama-70B-sized shape for one rank (h = 8192, 64 query heads and 8 KV heads of 128, t = 8, s = 4096: one
  group of 8 query heads per rank): sampled output rows, QKV_i in full, the group's dK and dV in full, two heads'
  dQ in full, sampled rows of dX_i and both weight gradients in full.

Tolerances as in the multi-head tests: fp32 relative Frobenius 1e-5; bf16 relative Frobenius 1e-2 against the
exact chain and the unit-scale element bound against the oracle fed the intermediates the library stored.
"""
import numpy as np
import pytest
import torch

import oracle as O
import tp_inputs as TI
from parity_utils import check_close, dev, empty, f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_block_columnparallel_amd as pkg

    return pkg.load()


def run_rank(L, w, inp, r, dtype, with_bias, causal, backward=True):
    s, b, h, a, d, t, g = w.s, w.b, w.h, w.a, w.d, w.t, w.g
    hl, n = a // t, (a // t + 2 * (g // t)) * d
    M = s * b
    dims = L.make_dims(s=s, b=b, h=h, a=a, d=d, t=t, g=g)
    Wq, Wo = empty((h, n), dtype), empty((hl * d, h), dtype)
    L.tp_shard_weights(dims, r, "qkv", dev(inp["Wqkv"], dtype), Wq)
    L.tp_shard_weights(dims, r, "proj", dev(inp["Wo"], dtype), Wo)
    bq = None
    if with_bias:
        bq = empty((n,), dtype)
        L.tp_shard_weights(dims, r, "b_qkv", dev(inp["bqkv"], dtype), bq)
    X, dZ = dev(inp["X"], dtype), dev(inp["dZ"], dtype)
    QKV, Oo, Z = empty((M, n), dtype), empty((M, hl * d), dtype), empty((M, h), dtype)
    lse = torch.empty((b, hl, s), dtype=torch.float32, device="cuda")
    L.tp_attn_fwd(dims, r, causal, X, Wq, bq, Wo, QKV, Oo, lse, Z)
    out = dict(Wq=Wq, bq=bq, QKV=QKV, O=Oo, lse=lse, Z=Z)
    if backward:
        nqb = (s + 63) // 64
        dO = empty((M, hl * d), dtype)
        rec = torch.empty(L.tp_attn_bwd_workspace(dims) // 4, dtype=torch.float32, device="cuda")
        assert rec.numel() == b * hl * nqb * 256 + (s * b * (g // t) * 2 * d * (a // g) if g < a else 0)
        dQKV, dWq, dWo, dX = empty((M, n), dtype), empty((h, n), dtype), empty((hl * d, h), dtype), empty((M, h), dtype)
        dbq = empty((n,), dtype) if with_bias else None
        L.tp_attn_bwd(dims, r, causal, X, Wq, Wo, QKV, Oo, lse, dZ, dO, rec, dQKV, dWq, dbq, dWo, dX)
        out.update(dO=dO, dQKV=dQKV, dWqkv=dWq, dbqkv=dbq, dWo=dWo, dX=dX)
    torch.cuda.synchronize()
    return out


def core_grads_stored(QKVs, dOs, s, b, hl, G, d, causal):
    """dQKV_i from the stored QKV_i and dO by the oracle's per-head core backward, dK / dV summed per group."""
    dQKV = np.zeros_like(QKVs)
    for bi in range(b):
        rows = np.arange(s) * b + bi
        for jj in range(hl):
            cq, ck, cv = O.shard_head_columns(G, d, jj)
            gq, gk, gv = O.attention_core_backward(QKVs[rows, cq], QKVs[rows, ck], QKVs[rows, cv],
                                                   dOs[rows, jj * d:(jj + 1) * d], causal)
            dQKV[rows, cq] = gq
            dQKV[rows, ck] += gk
            dQKV[rows, cv] += gv
    return dQKV


def test_qkv_packer_with_groups(L):
    h, a, g, d, t = 64, 8, 4, 8, 2
    say("GQA QKV packer a=8 g=4 d=8 t=2 (weight and bias), bf16 and fp32")
    for dtype in ("bf16", "f32"):
        full = TI.tensor(3, 1, (h, (a + 2 * g) * d), 1.0, dtype)
        bias = TI.tensor(3, 4, ((a + 2 * g) * d,), 1.0, dtype)
        dims = L.make_dims(h=h, a=a, d=d, t=t, g=g)
        n = (a // t + 2 * g // t) * d
        for r in range(t):
            sh, sb = empty((h, n), dtype), empty((n,), dtype)
            L.tp_shard_weights(dims, r, "qkv", dev(full, dtype), sh)
            L.tp_shard_weights(dims, r, "b_qkv", dev(bias, dtype), sb)
            torch.cuda.synchronize()
            cols = O.qkv_shard_columns(a, d, t, r, g)
            assert np.array_equal(f64(sh), O.as_f64(full, dtype)[:, cols])
            assert np.array_equal(f64(sb), O.as_f64(bias, dtype)[cols])


CASES = [  # a, g, d, t, dtype, causal
    (8, 2, 32, 2, "bf16", True),     # 4 query heads per group, one group per rank
    (6, 3, 64, 3, "bf16", True),     # 2 per group, t = 3
    (8, 4, 96, 2, "bf16", False),    # 2 per group, two groups per rank
    (4, 2, 128, 2, "bf16", True),
    (8, 2, 40, 2, "bf16", True),     # d = 40 in the 64 bucket
    (16, 8, 32, 8, "bf16", True),    # t = 8: the QKV and dO GEMMs fill one tile, so K is split over workgroups
    (8, 8, 64, 8, "bf16", False),    # g = a (plain multi-head), t = 8: split-K dO GEMM
    (4, 2, 16, 2, "f32", True),
    (6, 2, 8, 2, "f32", False),
]


@pytest.mark.parametrize("a,g,d,t,dtype,causal", CASES)
def test_gqa_small_ragged(L, a, g, d, t, dtype, causal):
    w = TI.Workload("gqa_small", "attn", s=100, b=2, h=a * d, a=a, d=d, t=t, g=g, causal=causal, dtype=dtype)
    say(f"GQA fwd+bwd s=100 b=2 a={a} g={g} d={d} t={t} causal={causal} {dtype}")
    inp = TI.attn_inputs(w, with_bias=True, seed=a + g + d)
    X = O.as_f64(inp["X"], dtype).reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], dtype).reshape(w.M, w.h)
    Wqkv, Wo, bq = O.as_f64(inp["Wqkv"], dtype), O.as_f64(inp["Wo"], dtype), O.as_f64(inp["bqkv"], dtype)
    hl, G = a // t, a // g
    for r in range(t):
        got = run_rank(L, w, inp, r, dtype, True, causal)
        fw = O.attention_shard_forward(X, Wqkv, Wo, w.s, w.b, a, d, t, r, causal, bq, g=g)
        ref = O.attention_shard_backward(X, Wqkv, Wo, dZ, w.s, w.b, a, d, t, r, causal, bq, g=g)
        if dtype == "f32":
            for k in ("QKV", "O", "Z"):
                check_close(f64(got[k]), fw[k], dtype, k)
            check_close(f64(got["lse"]), fw["lse"], dtype, "lse")
            for k in ("dO", "dQKV", "dWqkv", "dbqkv", "dWo", "dX"):
                check_close(f64(got[k]), ref[k], dtype, k)
            continue
        for k in ("O", "Z", "dO", "dQKV", "dWqkv", "dbqkv", "dWo", "dX"):
            want = fw[k] if k in ("O", "Z") else ref[k]
            rf = O.rel_frobenius(f64(got[k]), want)
            assert rf <= 1e-2, f"rank {r} {k}: rel Frobenius {rf:.3e}"
        QKVs, Os, dOs = f64(got["QKV"]), f64(got["O"]), f64(got["dO"])
        # forward element bound: the oracle's attention on the stored QKV_i
        rows = np.arange(w.M)
        check_close(Os, O.attention_rows(QKVs, w.s, w.b, hl, d, rows, causal, G=G)["O"], dtype, "O", row_unit=True)
        Wo_i = Wo[r * hl * d:(r + 1) * hl * d, :]
        Wq_i = Wqkv[:, O.qkv_shard_columns(a, d, t, r, g)]
        qc = O.qkv_shard_columns(a, d, t, r, g)
        check_close(QKVs, X @ Wq_i + bq[qc], dtype, "QKV")
        check_close(dOs, dZ @ Wo_i.T, dtype, "dO")
        check_close(f64(got["dQKV"]), core_grads_stored(QKVs, dOs, w.s, w.b, hl, G, d, causal), dtype, "dQKV")
        dQs = f64(got["dQKV"])
        check_close(f64(got["dWqkv"]), X.T @ dQs, dtype, "dWqkv")
        check_close(f64(got["dbqkv"]), dQs.sum(axis=0), dtype, "dbqkv")
        check_close(f64(got["dWo"]), Os.T @ dZ, dtype, "dWo")
        check_close(f64(got["dX"]), dQs @ Wq_i.T, dtype, "dX")


def test_gqa_llama70b_shape_one_rank(L):
    w = TI.ATTN_GQA_70B
    r = 3
    say("GQA h=8192 a=64 g=8 d=128 s=4096 t=8 rank 3 (one group of 8 query heads)")
    inp = TI.attn_inputs(w, seed=0)
    got = run_rank(L, w, inp, r, "bf16", False, True)
    hl, d, G = w.a // w.t, w.d, w.a // w.g
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], "bf16").reshape(w.M, w.h)
    Wqkv, Wo = O.as_f64(inp["Wqkv"], "bf16"), O.as_f64(inp["Wo"], "bf16")
    cols_i = O.qkv_shard_columns(w.a, d, w.t, r, w.g)
    Wq_i, Wo_i = Wqkv[:, cols_i], Wo[r * hl * d:(r + 1) * hl * d, :]
    QKVs, Os, dOs, dQs = f64(got["QKV"]), f64(got["O"]), f64(got["dO"]), f64(got["dQKV"])
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(w.M, size=48, replace=False))
    rows[0], rows[-1] = 0, w.M - 1
    check_close(QKVs[rows], X[rows] @ Wq_i, "bf16", "QKV rows")
    check_close(Os[rows], O.attention_rows(QKVs, w.s, w.b, hl, d, rows, True, G=G)["O"], "bf16", "O rows",
                row_unit=True)
    check_close(dOs[rows], dZ[rows] @ Wo_i.T, "bf16", "dO rows")
    # the group's dK and dV in full (sum over its 8 query heads), two heads' dQ in full
    dK = np.zeros((w.M, d))
    dV = np.zeros((w.M, d))
    for jj in range(hl):
        cq, ck, cv = O.shard_head_columns(G, d, jj)
        gq, gk, gv = O.attention_core_backward(QKVs[:, cq], QKVs[:, ck], QKVs[:, cv], dOs[:, jj * d:(jj + 1) * d], True)
        dK += gk
        dV += gv
        if jj in (0, hl - 1):
            check_close(dQs[:, cq], gq, "bf16", f"dQ head {jj}")
    _, ck, cv = O.shard_head_columns(G, d, 0)
    check_close(dQs[:, ck], dK, "bf16", "dK (group)")
    check_close(dQs[:, cv], dV, "bf16", "dV (group)")
    check_close(f64(got["dX"])[rows], dQs[rows] @ Wq_i.T, "bf16", "dX rows")
    # the GEMMs that split K over workgroups (the QKV GEMM in full, the weight-gradient pair's tail tiles) in full
    check_close(QKVs, X @ Wq_i, "bf16", "QKV")
    check_close(f64(got["dWqkv"]), X.T @ dQs, "bf16", "dWqkv")
    check_close(f64(got["dWo"]), Os.T @ dZ, "bf16", "dWo")
