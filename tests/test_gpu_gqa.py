"""Grouped-query attention (g KV heads, a/g query heads each) through the C ABI, against the fp64 oracle.

* the QKV shard packer with g < a: bit for bit against the oracle's slicing (the pages' per-group interleave);
* forward and backward of every rank at small ragged shapes (s = 100: a partial 64-row tile), group sizes 2 to 4,
  one or two local groups, t up to 8 (split-K GEMMs), every head-dim bucket, causal and not, bf16 and fp32, with a QKV bias: O_i, lse_i, Z_i
  and dQKV_i (a KV head's dK / dV summed over its group's query heads), dWqkv_i, dbqkv_i, dWo_i, dX_i;
* the Llama-70B-sized shape for one rank (h = 8192, 64 query heads and 8 KV heads of 128, t = 8, s = 4096: one
  group of 8 query heads per rank): sampled output rows, QKV_i in full, the group's dK and dV in full, two heads'
  dQ in full, sampled rows of dX_i and both weight gradients in full.

Tolerances as in the multi-head tests: fp32 relative Frobenius 1e-5; bf16 relative Frobenius 1e-2 against the
exact fp64 chain from X and the unit-scale element bound against the oracle's chain along the block's bf16 data
flow (QKV_i, O_i, dO and dQKV_i rounded where the block stores them).  Every expected value is the oracle's.  For
the element check the backward reads the oracle's stored forward outputs; the library's own forward into its
backward is checked against the exact chain too.
"""
import numpy as np
import pytest
import torch

import oracle as O
import tp_inputs as TI
from parity_utils import check_close, dev, empty, f64, say, storage

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_block_columnparallel_amd as pkg

    return pkg.load()


def oracle_saved(st, dtype):
    """The forward outputs the backward reads (QKV_i, O_i, lse_i) from the oracle's bf16 data-flow forward, in
    storage form (so that the backward's element check compares like with like; as in the multi-head tests)."""
    return {"QKV": storage(st["QKV"], dtype), "O": storage(st["O"], dtype), "lse": st["lse"].astype(np.float32)}


def run_rank(L, w, inp, r, dtype, with_bias, causal, backward=True, saved=None):
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
        Qb, Ob, lb = QKV, Oo, lse
        if saved is not None:
            Qb, Ob = dev(saved["QKV"], dtype), dev(saved["O"], dtype)
            lb = torch.from_numpy(np.ascontiguousarray(saved["lse"], dtype=np.float32)).cuda()
        L.tp_attn_bwd(dims, r, causal, X, Wq, Wo, Qb, Ob, lb, dZ, dO, rec, dQKV, dWq, dbq, dWo, dX)
        out.update(dO=dO, dQKV=dQKV, dWqkv=dWq, dbqkv=dbq, dWo=dWo, dX=dX)
    torch.cuda.synchronize()
    return out


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
    store = None if dtype == "f32" else "bf16"
    for r in range(t):
        ref = O.attention_shard_backward(X, Wqkv, Wo, dZ, w.s, w.b, a, d, t, r, causal, bq, g=g)
        rst = O.attention_shard_backward(X, Wqkv, Wo, dZ, w.s, w.b, a, d, t, r, causal, bq, g=g, store=store)
        # forward outputs from the library's forward; the backward from the oracle's stored forward outputs
        got = run_rank(L, w, inp, r, dtype, True, causal, saved=oracle_saved(rst, dtype))
        for k in ("QKV", "O", "Z", "lse", "dO", "dQKV", "dWqkv", "dbqkv", "dWo", "dX"):
            # attention rows average different numbers of value rows: their unit is the row's RMS
            check_close(f64(got[k]).reshape(ref[k].shape), ref[k], dtype, f"rank {r} {k}",
                        row_unit=k in ("O", "Z"), elem_ref=rst[k])
        # the library's own forward into its backward
        nat = run_rank(L, w, inp, r, dtype, True, causal)
        for k in ("dQKV", "dWqkv", "dWo", "dX"):
            if dtype == "f32":
                check_close(f64(nat[k]), ref[k], dtype, f"rank {r} {k} (own forward)")
            else:
                rf = O.rel_frobenius(f64(nat[k]), ref[k])
                assert rf <= 1e-2, f"rank {r} {k} (own forward): rel Frobenius {rf:.3e}"


def test_gqa_llama70b_shape_one_rank(L):
    w = TI.ATTN_GQA_70B
    r = 3
    say("GQA h=8192 a=64 g=8 d=128 s=4096 t=8 rank 3 (one group of 8 query heads)")
    inp = TI.attn_inputs(w, seed=0)
    hl, d, G = w.a // w.t, w.d, w.a // w.g
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], "bf16").reshape(w.M, w.h)
    Wqkv, Wo = O.as_f64(inp["Wqkv"], "bf16"), O.as_f64(inp["Wo"], "bf16")
    say("GQA rank 3: oracle, exact chain and bf16 data flow")
    ref = O.attention_shard_backward(X, Wqkv, Wo, dZ, w.s, w.b, w.a, d, w.t, r, True, g=w.g)
    rst = O.attention_shard_backward(X, Wqkv, Wo, dZ, w.s, w.b, w.a, d, w.t, r, True, g=w.g, store="bf16")
    say("GQA rank 3: library forward into backward, then backward from the oracle's forward")
    nat = run_rank(L, w, inp, r, "bf16", False, True)
    for k in ("dQKV", "dWqkv", "dWo", "dX"):
        rf = O.rel_frobenius(f64(nat[k]), ref[k])
        assert rf <= 1e-2, f"{k} (own forward): rel Frobenius {rf:.3e}"
    got = run_rank(L, w, inp, r, "bf16", False, True, saved=oracle_saved(rst, "bf16"))
    QKVs, Os, dQs = f64(got["QKV"]), f64(got["O"]), f64(got["dQKV"])
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(w.M, size=48, replace=False))
    rows[0], rows[-1] = 0, w.M - 1
    # the QKV GEMM splits K over workgroups: in full
    check_close(QKVs, ref["QKV"], "bf16", "QKV", elem_ref=rst["QKV"])
    check_close(Os[rows], ref["O"][rows], "bf16", "O rows", row_unit=True, elem_ref=rst["O"][rows])
    check_close(f64(got["Z"])[rows], ref["Z"][rows], "bf16", "Z rows", row_unit=True, elem_ref=rst["Z"][rows])
    check_close(f64(got["dO"])[rows], ref["dO"][rows], "bf16", "dO rows", elem_ref=rst["dO"][rows])
    # the group's dK and dV in full (sums over its 8 query heads), two heads' dQ in full
    for jj in (0, hl - 1):
        cq, _, _ = O.shard_head_columns(G, d, jj)
        check_close(dQs[:, cq], ref["dQKV"][:, cq], "bf16", f"dQ head {jj}", elem_ref=rst["dQKV"][:, cq])
    _, ck, cv = O.shard_head_columns(G, d, 0)
    check_close(dQs[:, ck], ref["dQKV"][:, ck], "bf16", "dK (group)", elem_ref=rst["dQKV"][:, ck])
    check_close(dQs[:, cv], ref["dQKV"][:, cv], "bf16", "dV (group)", elem_ref=rst["dQKV"][:, cv])
    check_close(f64(got["dX"])[rows], ref["dX"][rows], "bf16", "dX rows", elem_ref=rst["dX"][rows])
    # the weight-gradient pair's tail tiles split K over workgroups: both in full
    check_close(f64(got["dWqkv"]), ref["dWqkv"], "bf16", "dWqkv", elem_ref=rst["dWqkv"])
    check_close(f64(got["dWo"]), ref["dWo"], "bf16", "dWo", elem_ref=rst["dWo"])
