"""GPU parity of the per-rank attention backward (tp_attn_bwd) against the fp64 oracle, through the C ABI.

* small shapes with ragged 64-row tiles (s = 100), every supported head-dim bucket, causal and not, fp32 and bf16,
  with a QKV bias: dQKV_i, dWqkv_i, dbqkv_i, dWo_i and dX_i of every rank against the oracle's shard backward on
  the same stored inputs;
* the 22B-width workload at full size for one rank (s = 4096, 8 local heads of 96, causal): the core gradients of
  two heads in full against the oracle's core backward fed the QKV_i and dO the library stored (bf16), sampled
  rows of dX_i and the weight gradients in full against the oracle on the library's stored dQKV_i.

The bf16 path stores QKV_i, O_i and dO in bf16 and feeds P and dS to the matrix cores in bf16, so the exact fp64
chain from X differs from it by storage rounding; as in the forward tests, the relative Frobenius bound is taken
against the exact chain and the element bound against the oracle fed the stored intermediates.
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


def run_rank(L, w, inp, r, dtype, with_bias, causal):
    s, b, h, a, d, t = w.s, w.b, w.h, w.a, w.d, w.t
    hl = a // t
    M = s * b
    dims = L.make_dims(s=s, b=b, h=h, a=a, d=d, t=t)
    Wq, Wo = empty((h, 3 * hl * d), dtype), empty((hl * d, h), dtype)
    L.tp_shard_weights(dims, r, "qkv", dev(inp["Wqkv"], dtype), Wq)
    L.tp_shard_weights(dims, r, "proj", dev(inp["Wo"], dtype), Wo)
    bq = None
    if with_bias:
        bq = empty((3 * hl * d,), dtype)
        L.tp_shard_weights(dims, r, "b_qkv", dev(inp["bqkv"], dtype), bq)
    X, dZ = dev(inp["X"], dtype), dev(inp["dZ"], dtype)
    QKV, Oo, Z = empty((M, 3 * hl * d), dtype), empty((M, hl * d), dtype), empty((M, h), dtype)
    lse = torch.empty((b, hl, s), dtype=torch.float32, device="cuda")
    L.tp_attn_fwd(dims, r, causal, X, Wq, bq, Wo, QKV, Oo, lse, Z)
    nqb = (s + 63) // 64
    dO = empty((M, hl * d), dtype)
    rec = torch.empty((b, hl, nqb, 256), dtype=torch.float32, device="cuda")
    dQKV, dWq, dWo, dX = empty((M, 3 * hl * d), dtype), empty((h, 3 * hl * d), dtype), empty((hl * d, h), dtype), \
        empty((M, h), dtype)
    dbq = empty((3 * hl * d,), dtype) if with_bias else None
    L.tp_attn_bwd(dims, r, causal, X, Wq, Wo, QKV, Oo, lse, dZ, dO, rec, dQKV, dWq, dbq, dWo, dX)
    torch.cuda.synchronize()
    return dict(QKV=QKV, O=Oo, lse=lse, dO=dO, dQKV=dQKV, dWqkv=dWq, dbqkv=dbq, dWo=dWo, dX=dX, rec=rec)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 40])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_backward_small_ragged(L, dtype, d, causal):
    a, t = 4, 2
    w = TI.Workload("attn_small", "attn", s=100, b=2, h=a * d, a=a, d=d, t=t, causal=causal, dtype=dtype)
    say(f"attention backward s=100 b=2 a=4 d={d} t=2 causal={causal} {dtype}")
    inp = TI.attn_inputs(w, with_bias=True, seed=d + 1)
    X = O.as_f64(inp["X"], dtype).reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], dtype).reshape(w.M, w.h)
    Wqkv, Wo, bq = O.as_f64(inp["Wqkv"], dtype), O.as_f64(inp["Wo"], dtype), O.as_f64(inp["bqkv"], dtype)
    hl = a // t
    for r in range(t):
        got = run_rank(L, w, inp, r, dtype, True, causal)
        ref = O.attention_shard_backward(X, Wqkv, Wo, dZ, w.s, w.b, a, d, t, r, causal, bq)
        if dtype == "f32":
            for k in ("dO", "dQKV", "dWqkv", "dbqkv", "dWo", "dX"):
                check_close(f64(got[k]), ref[k], dtype, k)
            continue
        # exact chain: relative Frobenius
        for k in ("dO", "dQKV", "dWqkv", "dbqkv", "dWo", "dX"):
            rf = O.rel_frobenius(f64(got[k]), ref[k])
            assert rf <= 1e-2, f"{k}: rel Frobenius {rf:.3e}"
        # element bounds against the oracle fed the stored intermediates (QKV_i, O_i, dO in bf16)
        QKVs, Os, dOs = f64(got["QKV"]), f64(got["O"]), f64(got["dO"])
        Wo_i = Wo[r * hl * d:(r + 1) * hl * d, :]
        Wq_i = Wqkv[:, O.qkv_shard_columns(a, d, t, r)]
        check_close(f64(got["dO"]), dZ @ Wo_i.T, dtype, "dO")
        dQKV = np.zeros_like(QKVs)
        for bi in range(w.b):
            rows = np.arange(w.s) * w.b + bi
            for jj in range(hl):
                base = jj * 3 * d
                g = O.attention_core_backward(QKVs[rows, base:base + d], QKVs[rows, base + d:base + 2 * d],
                                              QKVs[rows, base + 2 * d:base + 3 * d], dOs[rows, jj * d:(jj + 1) * d],
                                              causal)
                for n, gg in enumerate(g):
                    dQKV[rows, base + n * d:base + (n + 1) * d] = gg
        check_close(f64(got["dQKV"]), dQKV, dtype, "dQKV")
        dQs = f64(got["dQKV"])
        check_close(f64(got["dWqkv"]), X.T @ dQs, dtype, "dWqkv")
        check_close(f64(got["dbqkv"]), dQs.sum(axis=0), dtype, "dbqkv")
        check_close(f64(got["dWo"]), Os.T @ dZ, dtype, "dWo")
        check_close(f64(got["dX"]), dQs @ Wq_i.T, dtype, "dX")


def test_attention_backward_full_size_one_rank_sampled(L):
    w = TI.ATTN_22B
    r = 5
    say("attention backward h=6144 a=64 d=96 s=4096 t=8 rank 5 (two heads in full, sampled rows, full weight gradients)")
    inp = TI.attn_inputs(w, seed=0)
    got = run_rank(L, w, inp, r, "bf16", False, True)
    hl, d = w.a // w.t, w.d
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], "bf16").reshape(w.M, w.h)
    Wqkv, Wo = O.as_f64(inp["Wqkv"], "bf16"), O.as_f64(inp["Wo"], "bf16")
    Wo_i = Wo[r * hl * d:(r + 1) * hl * d, :]
    Wq_i = Wqkv[:, O.qkv_shard_columns(w.a, d, w.t, r)]
    QKVs, Os, dOs, dQs = f64(got["QKV"]), f64(got["O"]), f64(got["dO"]), f64(got["dQKV"])
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(w.M, size=64, replace=False))
    rows[0], rows[-1] = 0, w.M - 1
    check_close(dOs[rows], dZ[rows] @ Wo_i.T, "bf16", "dO rows")
    for jj in (0, hl - 1):  # two heads in full (b = 1: every row is one sequence position)
        base = jj * 3 * d
        g = O.attention_core_backward(QKVs[:, base:base + d], QKVs[:, base + d:base + 2 * d],
                                      QKVs[:, base + 2 * d:base + 3 * d], dOs[:, jj * d:(jj + 1) * d], True)
        for n, name in enumerate(("dQ", "dK", "dV")):
            check_close(dQs[:, base + n * d:base + (n + 1) * d], g[n], "bf16", f"{name} head {jj}")
    check_close(f64(got["dX"])[rows], dQs[rows] @ Wq_i.T, "bf16", "dX rows")
    # the weight gradients in full (the pair's tail tiles split K over workgroups)
    check_close(f64(got["dWqkv"]), X.T @ dQs, "bf16", "dWqkv")
    check_close(f64(got["dWo"]), Os.T @ dZ, "bf16", "dWo")


def test_attention_backward_ragged_pair_tail(L):
    """A shape whose weight-gradient pair has ragged tiles and overruns one round of 256 tiles (dWo 800 x 6400 and
    dWqkv 6400 x 2400: 350 tiles, a tail of 94 split over two K ranges): both weight gradients in full."""
    w = TI.Workload("attn_ragged_tail", "attn", s=4096, b=1, h=6400, a=80, d=80, t=8, causal=True, dtype="bf16")
    r = 3
    say("attention backward h=6400 a=80 d=80 s=4096 t=8 rank 3 (ragged weight-gradient tiles, split tail)")
    inp = TI.attn_inputs(w, seed=3)
    got = run_rank(L, w, inp, r, "bf16", False, True)
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], "bf16").reshape(w.M, w.h)
    Os, dQs = f64(got["O"]), f64(got["dQKV"])
    check_close(f64(got["dWqkv"]), X.T @ dQs, "bf16", "dWqkv")
    check_close(f64(got["dWo"]), Os.T @ dZ, "bf16", "dWo")
