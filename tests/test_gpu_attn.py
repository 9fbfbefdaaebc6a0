"""GPU parity of the per-rank attention block (tp_attn_fwd) against the fp64 oracle, through the C ABI: small
shapes with ragged sequence tiles for every supported head-dim bucket, causal and not, fp32 and bf16; and the
22B-width workload at full size for one rank with sampled query rows (exact: a query row needs only its own
query and its sequence's keys and values).

bf16 outputs meet relative Frobenius 1e-2 against the exact fp64 chain and the unit-scale element bound against
the oracle's chain with QKV_i and O_i rounded to bf16 where the block stores them (store="bf16")."""
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
    QKV, Oo, Z = empty((M, 3 * hl * d), dtype), empty((M, hl * d), dtype), empty((M, h), dtype)
    lse = torch.empty((b, hl, s), dtype=torch.float32, device="cuda")
    L.tp_attn_fwd(dims, r, causal, dev(inp["X"], dtype), Wq, bq, Wo, QKV, Oo, lse, Z)
    torch.cuda.synchronize()
    return dict(QKV=QKV, O=Oo, lse=lse, Z=Z)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 40])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_small_ragged(L, dtype, d, causal):
    a, t = 4, 2
    w = TI.Workload("attn_small", "attn", s=100, b=2, h=a * d, a=a, d=d, t=t, causal=causal, dtype=dtype)
    say(f"attention s=100 b=2 a=4 d={d} t=2 causal={causal} {dtype}")
    inp = TI.attn_inputs(w, with_bias=True, seed=d)
    X = O.as_f64(inp["X"], dtype).reshape(w.M, w.h)
    Wqkv, Wo, bq = O.as_f64(inp["Wqkv"], dtype), O.as_f64(inp["Wo"], dtype), O.as_f64(inp["bqkv"], dtype)
    for r in range(t):
        got = run_rank(L, w, inp, r, dtype, True, causal)
        ref = O.attention_shard_forward(X, Wqkv, Wo, w.s, w.b, a, d, t, r, causal, bq)
        rst = ref if dtype == "f32" else O.attention_shard_forward(X, Wqkv, Wo, w.s, w.b, a, d, t, r, causal, bq,
                                                                   store="bf16")
        check_close(f64(got["QKV"]), ref["QKV"], dtype, "QKV", elem_ref=rst["QKV"])
        check_close(f64(got["O"]), ref["O"], dtype, "O", row_unit=True, elem_ref=rst["O"])
        check_close(f64(got["Z"]), ref["Z"], dtype, "Z", row_unit=True, elem_ref=rst["Z"])
        lse = got["lse"].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(lse - ref["lse"])) < (1e-4 if dtype == "f32" else 2e-2)



@pytest.mark.parametrize("d", [40, 96, 128])
def test_attention_causal_long_ragged(L, d):
    # s = 1100: 18 query tiles of up to 18 key blocks each, the last tile ragged (12 queries, a 12-key last block)
    a, t, s = 4, 2, 1100
    w = TI.Workload("attn_long", "attn", s=s, b=2, h=a * d, a=a, d=d, t=t, causal=True, dtype="bf16")
    say(f"attention s={s} b=2 a=4 d={d} t=2 causal bf16")
    inp = TI.attn_inputs(w, with_bias=True, seed=200 + d)
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    Wqkv, Wo, bq = O.as_f64(inp["Wqkv"], "bf16"), O.as_f64(inp["Wo"], "bf16"), O.as_f64(inp["bqkv"], "bf16")
    r = 1
    got = run_rank(L, w, inp, r, "bf16", True, True)
    ref = O.attention_shard_forward(X, Wqkv, Wo, w.s, w.b, a, d, t, r, True, bq)
    rst = O.attention_shard_forward(X, Wqkv, Wo, w.s, w.b, a, d, t, r, True, bq, store="bf16")
    check_close(f64(got["O"]), ref["O"], "bf16", "O", row_unit=True, elem_ref=rst["O"])
    check_close(f64(got["Z"]), ref["Z"], "bf16", "Z", row_unit=True, elem_ref=rst["Z"])
    lse = got["lse"].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(lse - ref["lse"])) < 2e-2
    assert np.max(np.abs(lse - rst["lse"])) < 2e-3

@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_short_sequence_masked_key_half(L, d, causal):
    # s < 32: the forward splits each 64-key block between two waves of the same queries, and here the upper half
    # (keys 32..63) holds no key at all, so that half's running max stays -inf up to the merge
    a, t, s = 4, 2, 20
    w = TI.Workload("attn_short", "attn", s=s, b=3, h=a * d, a=a, d=d, t=t, causal=causal, dtype="bf16")
    say(f"attention s={s} b=3 a=4 d={d} t=2 causal={causal} bf16")
    inp = TI.attn_inputs(w, with_bias=False, seed=100 + d)
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    Wqkv, Wo = O.as_f64(inp["Wqkv"], "bf16"), O.as_f64(inp["Wo"], "bf16")
    for r in range(t):
        got = run_rank(L, w, inp, r, "bf16", False, causal)
        ref = O.attention_shard_forward(X, Wqkv, Wo, w.s, w.b, a, d, t, r, causal, None)
        rst = O.attention_shard_forward(X, Wqkv, Wo, w.s, w.b, a, d, t, r, causal, None, store="bf16")
        assert torch.isfinite(got["O"].float()).all() and torch.isfinite(got["lse"]).all()
        check_close(f64(got["O"]), ref["O"], "bf16", "O", row_unit=True, elem_ref=rst["O"])
        check_close(f64(got["Z"]), ref["Z"], "bf16", "Z", row_unit=True, elem_ref=rst["Z"])
        lse = got["lse"].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(lse - ref["lse"])) < 2e-2


def test_attention_full_size_one_rank_sampled(L):
    w = TI.ATTN_22B
    r = 3
    say("attention h=6144 a=64 d=96 s=4096 t=8 rank 3 (sampled query rows)")
    inp = TI.attn_inputs(w, seed=0)
    got = run_rank(L, w, inp, r, "bf16", False, True)
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    Wqkv, Wo = O.as_f64(inp["Wqkv"], "bf16"), O.as_f64(inp["Wo"], "bf16")
    cols = O.qkv_shard_columns(w.a, w.d, w.t, r)
    QKV = X @ Wqkv[:, cols]  # every token's q, k, v of the local heads (the keys need all rows)
    check_close(f64(got["QKV"]), QKV, "bf16", "QKV")
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(w.M, size=96, replace=False))
    rows[0], rows[-1] = 0, w.M - 1
    hl = w.a // w.t
    ref = O.attention_rows(QKV, w.s, w.b, hl, w.d, rows, True)
    Wo_i = Wo[r * hl * w.d:(r + 1) * hl * w.d, :]
    got_o, got_z = f64(got["O"])[rows], f64(got["Z"])[rows]
    # against the exact block: relative Frobenius error
    assert O.rel_frobenius(got_o, ref["O"]) <= 1e-2
    assert O.rel_frobenius(got_z, ref["O"] @ Wo_i) <= 1e-2
    # the attention step consumes QKV_i as the ABI stores it (bf16): against the oracle's own exact QKV rounded to
    # that storage, every bf16 bound holds; the rounding of Q and K alone moves a 4096-key softmax by ~0.4%
    ref_st = O.attention_rows(O.stored(QKV, "bf16"), w.s, w.b, hl, w.d, rows, True)
    check_close(got_o, ref_st["O"], "bf16", "O vs stored QKV", row_unit=True)
    check_close(got_z, O.stored(ref_st["O"], "bf16") @ Wo_i, "bf16", "Z vs stored O", row_unit=True)
    lse = got["lse"].cpu().numpy()[0][:, rows].T.astype(np.float64)  # [rows, hl]
    assert np.max(np.abs(lse - ref["lse"])) < 2e-2
    assert np.max(np.abs(lse - ref_st["lse"])) < 2e-3


def test_attention_split_k_qkv_192_column_tiles_sampled(L):
    # t = 16 at h = 4096, d = 128: the rank's QKV GEMM is 4096 x 768 x 4096, whose 256-column tiles (48) leave most
    # CUs idle, and Z_i lends room for two K runs; 64 tiles of 192 columns split in two finish sooner, so the QKV GEMM
    # takes the split 192-column kernel with the bias applied by the partial sum
    w = TI.Workload("attn_t16", "attn", s=4096, b=1, h=4096, a=32, d=128, t=16, causal=True, dtype="bf16")
    r = 11
    say("attention h=4096 a=32 d=128 s=4096 t=16 rank 11 (split-K 192-column QKV; sampled query rows)")
    inp = TI.attn_inputs(w, with_bias=True, seed=5)
    with L.LaunchTimer(16, only="gemm_bf16") as lt:
        got = run_rank(L, w, inp, r, "bf16", True, True)
    assert "gemm_bf16_big192_splitk_KM" in lt.names, lt.names
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    Wqkv, bq = O.as_f64(inp["Wqkv"], "bf16"), O.as_f64(inp["bqkv"], "bf16")
    cols = O.qkv_shard_columns(w.a, w.d, w.t, r)
    QKV = X @ Wqkv[:, cols] + bq[cols]
    check_close(f64(got["QKV"]), QKV, "bf16", "QKV")
    rng = np.random.default_rng(13)
    rows = np.sort(rng.choice(w.M, size=64, replace=False))
    rows[0], rows[-1] = 0, w.M - 1
    ref_st = O.attention_rows(O.stored(QKV, "bf16"), w.s, w.b, w.a // w.t, w.d, rows, True)
    check_close(f64(got["O"])[rows], ref_st["O"], "bf16", "O vs stored QKV", row_unit=True)
