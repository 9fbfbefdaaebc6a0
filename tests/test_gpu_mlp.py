"""GPU parity of the MLP block (tp_mlp_fwd / tp_mlp_bwd and the rank loop with the on-device reduction) against
the fp64 oracle, through the C ABI.

* tiny fp32 workload: every rank's outputs and the reduced block output, element by element;
* bf16 at sizes that span several tiles with ragged tails in every dimension, each activation, with biases;
* bf16 at the full workload sizes, one rank, in the launch configuration the bench times: token rows sampled for
  U, Y, Z, dU, dX (exact: a row depends only on its own inputs) and output columns sampled for dA, dB, da.

bf16 outputs meet relative Frobenius 1e-2 against the exact fp64 chain, and the unit-scale element bound against
the oracle's same chain along the block's bf16 data flow (U_i, Y_i and dU_i rounded to bf16 where the block
stores them; store="bf16").  The backward reads the oracle's stored U_i and Y_i (see oracle_saved); the forward's
own outputs are checked on their own, and the whole-block tests run the library's forward into its backward.
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


def _shard_host(full, kind, t, r, **kw):
    return O.shard_weight(kind, full, t, r, **kw)


def oracle_saved(w, inp, r, dtype, with_bias):
    """The forward activations the backward reads (U_i, Y_i), computed by the oracle and stored as the block stores
    them.  Feeding these to tp_mlp_bwd, rather than the library's own forward outputs, lets the backward's element
    check compare like with like: where U_i sits on a rounding boundary, the library's fp32-accumulated U_i and the
    oracle's exact one may round to neighbouring bf16 values, and act' can magnify one such step past the bound."""
    X = O.as_f64(inp["X"], dtype).reshape(w.M, w.h)
    A, B = O.as_f64(inp["A"], dtype), O.as_f64(inp["B"], dtype)
    a = O.as_f64(inp["a"], dtype) if with_bias else None
    fw = O.mlp_shard_forward(X, A, B, w.t, r, w.act, a)
    return {"U": storage(fw["U"], dtype), "Y": storage(fw["Y"], dtype)}


def run_rank(L, w, inp, r, dtype, with_bias, saved=None):
    """Pack rank r's shards with the library, run fwd + bwd, return device outputs.  saved: the U_i, Y_i (storage
    form) the backward reads instead of the forward's outputs."""
    s, b, h, t, f = w.s, w.b, w.h, w.t, w.f_l
    n1 = w.n1
    M = s * b
    dims = L.make_dims(s=s, b=b, h=h, ffn=w.ffn, t=t)
    X = dev(inp["X"], dtype)
    dZ = dev(inp["dZ"], dtype)
    A_full, B_full = dev(inp["A"], dtype), dev(inp["B"], dtype)
    wk = "fc1_gate_up" if w.act == "swiglu" else "fc1"
    Ai, Bi = empty((h, n1), dtype), empty((f, h), dtype)
    L.tp_shard_weights(dims, r, wk, A_full, Ai)
    L.tp_shard_weights(dims, r, "fc2", B_full, Bi)
    ai = None
    if with_bias:
        ai = empty((n1,), dtype)
        L.tp_shard_weights(dims, r, "b_fc1_gate_up" if w.act == "swiglu" else "b_fc1", dev(inp["a"], dtype), ai)
    U, Y, Z = empty((M, n1), dtype), empty((M, f), dtype), empty((M, h), dtype)
    L.tp_mlp_fwd(dims, r, w.act, X, Ai, ai, Bi, U, Y, Z)
    dU, dA, dB, dX = empty((M, n1), dtype), empty((h, n1), dtype), empty((f, h), dtype), empty((M, h), dtype)
    da = empty((n1,), dtype) if with_bias else None
    Ub, Yb = (U, Y) if saved is None else (dev(saved["U"], dtype), dev(saved["Y"], dtype))
    L.tp_mlp_bwd(dims, r, w.act, X, Ai, Bi, Ub, Yb, dZ, dU, dA, da, dB, dX)
    torch.cuda.synchronize()
    return dict(U=U, Y=Y, Z=Z, dU=dU, dA=dA, da=da, dB=dB, dX=dX)


def oracle_full_rank(w, inp, r, dtype, with_bias, store=None):
    X = O.as_f64(inp["X"], dtype).reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], dtype).reshape(w.M, w.h)
    A, B = O.as_f64(inp["A"], dtype), O.as_f64(inp["B"], dtype)
    a = O.as_f64(inp["a"], dtype) if with_bias else None
    fw = O.mlp_shard_forward(X, A, B, w.t, r, w.act, a, store=store)
    bw = O.mlp_shard_backward(X, A, B, dZ, w.t, r, w.act, a, store=store)
    return fw, bw


def check_rank_full(w, got, ex, st, dtype, with_bias):
    """ex = (forward, backward) of the exact chain, st = the same along the bf16 data flow (or None for fp32)."""
    fw, bw = ex
    sfw, sbw = st if st is not None else ex
    for k in ("U", "Y", "Z"):
        check_close(f64(got[k]), fw[k], dtype, k, elem_ref=sfw[k])
    for k in ("dU", "dA", "dB", "dX"):
        check_close(f64(got[k]), bw[k], dtype, k, elem_ref=sbw[k])
    if with_bias:
        check_close(f64(got["da"]), bw["da"], dtype, "da", elem_ref=sbw["da"])


@pytest.mark.parametrize("with_bias", [True, False])
def test_tiny_fp32_every_rank_and_reduced_block(L, with_bias):
    w = TI.TINY
    say(f"tiny fp32 MLP t={w.t} bias={with_bias}")
    inp = TI.mlp_inputs(w, with_bias=with_bias)
    for r in range(w.t):
        got = run_rank(L, w, inp, r, "f32", with_bias)
        check_rank_full(w, got, oracle_full_rank(w, inp, r, "f32", with_bias), None, "f32", with_bias)
    # the whole block through the rank loop and the on-device g / f reductions
    from attention_block_columnparallel_amd.block import MlpBlock

    blk = MlpBlock(w.s, w.b, w.h, w.ffn, w.t, w.act, dev(inp["A"], "f32"), dev(inp["B"], "f32"),
                   dev(inp["a"], "f32") if with_bias else None, dev(inp["c"], "f32") if with_bias else None)
    X = dev(inp["X"], "f32")
    Z = blk.forward(X)
    dX = blk.backward(X, dev(inp["dZ"], "f32"))
    Xo = O.as_f64(inp["X"], "f32").reshape(w.M, w.h)
    full = O.mlp_forward(Xo, O.as_f64(inp["A"], "f32"), O.as_f64(inp["B"], "f32"), w.act,
                         O.as_f64(inp["a"], "f32") if with_bias else None,
                         O.as_f64(inp["c"], "f32") if with_bias else None)
    bwd = O.mlp_backward(Xo, O.as_f64(inp["A"], "f32"), O.as_f64(inp["B"], "f32"), full["U"], full["Y"],
                         O.as_f64(inp["dZ"], "f32").reshape(w.M, w.h), w.act)
    check_close(f64(Z), full["Z"], "f32", "Z block")
    check_close(f64(dX), bwd["dX"], "f32", "dX block")


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "relu", "swiglu"])
def test_bf16_multi_tile_ragged(L, act):
    # M = 37*3 = 111 rows, h = 200, f/t = 264: every dimension ragged against every tile size
    w = TI.Workload("ragged", "mlp", s=37, b=3, h=200, ffn=528, t=2, act=act, dtype="bf16")
    say(f"bf16 MLP ragged M=111 h=200 f_l=264 act={act}")
    inp = TI.mlp_inputs(w, with_bias=True, seed=3)
    for r in range(w.t):
        got = run_rank(L, w, inp, r, "bf16", True, saved=oracle_saved(w, inp, r, "bf16", True))
        check_rank_full(w, got, oracle_full_rank(w, inp, r, "bf16", True),
                        oracle_full_rank(w, inp, r, "bf16", True, store="bf16"), "bf16", True)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_fp32_small_multi_tile(L, act):
    w = TI.Workload("agree", "mlp", s=64, b=2, h=128, ffn=512, t=4, act=act, dtype="f32")
    say(f"fp32 MLP small act={act}")
    inp = TI.mlp_inputs(w, with_bias=True, seed=4)
    got = run_rank(L, w, inp, 1, "f32", True)
    check_rank_full(w, got, oracle_full_rank(w, inp, 1, "f32", True), None, "f32", True)


def _sampled_check(L, w, r, nrows=192, ncols=24, with_bias=False, seed=0):
    inp = TI.mlp_inputs(w, with_bias=with_bias, seed=seed)
    got = run_rank(L, w, inp, r, "bf16", with_bias, saved=oracle_saved(w, inp, r, "bf16", with_bias))
    rng = np.random.default_rng(100 + r)
    rows = np.sort(rng.choice(w.M, size=min(nrows, w.M), replace=False))
    rows[0], rows[-1] = 0, w.M - 1  # first and last rows always checked
    X = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], "bf16").reshape(w.M, w.h)
    A, B = O.as_f64(inp["A"], "bf16"), O.as_f64(inp["B"], "bf16")
    a = O.as_f64(inp["a"], "bf16") if with_bias else None
    ref = O.mlp_shard_rows(X[rows], dZ[rows], A, B, w.t, r, w.act, a)
    rst = O.mlp_shard_rows(X[rows], dZ[rows], A, B, w.t, r, w.act, a, store="bf16")
    for k in ("U", "Y", "Z", "dU", "dX"):
        check_close(f64(got[k])[rows], ref[k], "bf16", k, elem_ref=rst[k])
    js = np.sort(rng.choice(w.f_l, size=min(ncols, w.f_l), replace=False))
    js[0], js[-1] = 0, w.f_l - 1
    wc = O.mlp_shard_weight_grad_cols(X, dZ, A, B, w.t, r, js, w.act, a)
    ws = O.mlp_shard_weight_grad_cols(X, dZ, A, B, w.t, r, js, w.act, a, store="bf16")
    check_close(f64(got["dB"])[js], wc["dB_rows"], "bf16", "dB", elem_ref=ws["dB_rows"])
    check_close(f64(got["dA"])[:, wc["sel"]], wc["dA_cols"], "bf16", "dA", elem_ref=ws["dA_cols"])
    if with_bias:
        check_close(f64(got["da"])[wc["sel"]], wc["da_cols"], "bf16", "da", elem_ref=ws["da_cols"])


def test_bf16_large_ragged_k_sampled(L):
    # large enough that 256x256 tiles are chosen, ragged in M, N and K (K % 32 != 0: the general-K kernel)
    w = TI.Workload("large_ragged", "mlp", s=2043, b=8, h=1000, ffn=2 * 2040, t=2, act="gelu", dtype="bf16")
    say("bf16 MLP large ragged M=16344 h=1000 f_l=2040 (sampled)")
    _sampled_check(L, w, 1, with_bias=True, seed=7)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_bf16_large_ragged_mn_sampled(L, act):
    # ragged M = 16352 and N in {1056, 2080, 2 x 2080}; K in {1056, 2080} is not a multiple of 64, so these GEMMs take
    # the register-staged kernel (SwiGLU's dX, K = 4160, the large-tile one)
    w = TI.Workload("large_ragged_mn", "mlp", s=2044, b=8, h=1056, ffn=2 * 2080, t=2, act=act, dtype="bf16")
    say(f"bf16 MLP large ragged M=16352 h=1056 f_l=2080 act={act} (sampled)")
    _sampled_check(L, w, 0, with_bias=True, seed=8)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_bf16_large_tile_kernels_ragged_sampled(L, act):
    # every K a multiple of 64 (h = 3136, f_l = 2112, M = 16320) and enough tiles for the pair (over 3/4 of the
    # CUs), so every GEMM of the rank takes the large-tile kernel -- the 8-wave column, row and dY GEMMs, the 4-wave
    # dX GEMM and weight-gradient pair -- while M, h and f_l are not multiples of 256: ragged last row and column
    # tiles in every one of them
    w = TI.Workload("large_tile_ragged", "mlp", s=2040, b=8, h=3136, ffn=2 * 2112, t=2, act=act, dtype="bf16")
    say(f"bf16 MLP large-tile kernels ragged M=16320 h=3136 f_l=2112 act={act} (sampled)")
    with L.LaunchTimer(256, only="gemm_bf16") as lt:
        _sampled_check(L, w, 1, with_bias=True, seed=11)
    fwd_epi, bwd_epi = ("swiglu_fwd", "swiglu_bwd") if act == "swiglu" else ("bias_act", "act_bwd")
    # each GEMM on the large-tile kernel, at 256 or (where fewer rounds of CUs pay) 192 columns per tile
    for role in (f"KM_{fwd_epi}", "KM_store", f"KK_{bwd_epi}", "KK_store", "pair_MM_store"):
        assert {f"gemm_bf16_big_{role}", f"gemm_bf16_big192_{role}"} & set(lt.names), (role, lt.names)


@pytest.mark.parametrize("act", ["gelu", "relu"])
def test_bf16_192_column_tiles_ragged_sampled(L, act):
    # h = 1216 and f_l = 704 (multiples of 64, not of 192) at M = 16320: 192-column tiles take one or two rounds of
    # CUs fewer than 256-column ones, so the column, row, dY and dX GEMMs take them, each with a ragged last column
    # tile (and a ragged last row tile)
    w = TI.Workload("n192_ragged", "mlp", s=2040, b=8, h=1216, ffn=2 * 704, t=2, act=act, dtype="bf16")
    say(f"bf16 MLP 192-column tiles ragged M=16320 h=1216 f_l=704 act={act} (sampled)")
    with L.LaunchTimer(256, only="gemm_bf16") as lt:
        _sampled_check(L, w, 1, with_bias=True, seed=12)
    want = {"gemm_bf16_big192_KM_bias_act", "gemm_bf16_big192_KM_store", "gemm_bf16_big192_KK_act_bwd",
            "gemm_bf16_big192_KK_store"}
    assert want <= set(lt.names), (want - set(lt.names), lt.names)


@pytest.mark.parametrize("name,rank", [("mlp_h3072_ffn12288_t8_b8_s1024", 5),
                                       ("mlp_h4096_ffn16384_t8_b8_s2048", 2),
                                       ("sp_swiglu_h8192_ffn28672_t8_s4096", 7)])
def test_bf16_full_size_one_rank_sampled(L, name, rank):
    w = TI.WORKLOADS[name]
    say(f"bf16 MLP full size {name} rank {rank} (sampled rows / columns)")
    _sampled_check(L, w, rank, nrows=128, ncols=16)


def test_bf16_block_end_to_end_with_sp(L):
    # all t ranks, g as all-reduce and as dim-0 reduce-scatter, f on dX; row bias c added once
    w = TI.Workload("e2e", "mlp", s=48, b=2, h=136, ffn=4 * 152, t=4, act="gelu", dtype="bf16")
    say("bf16 MLP block end to end t=4 (AR and SP forms)")
    inp = TI.mlp_inputs(w, with_bias=True, seed=11)
    from attention_block_columnparallel_amd.block import MlpBlock

    blk = MlpBlock(w.s, w.b, w.h, w.ffn, w.t, w.act, dev(inp["A"], "bf16"), dev(inp["B"], "bf16"),
                   dev(inp["a"], "bf16"), dev(inp["c"], "bf16"))
    # SP entry: the input arrives as t dim-0 slices and is gathered on the device
    Xfull = inp["X"]
    slices = np.stack([O.split_dim0(Xfull, w.t, r) for r in range(w.t)])
    X = empty((w.s, w.b, w.h), "bf16")
    L.tp_gather_dim0(blk.dims, dev(slices, "bf16"), X)
    blk.forward_ranks(X)
    Z_ar = blk.reduce_forward(sp=False).clone()
    Z_rs = blk.reduce_forward(sp=True, out=empty((w.t, w.s // w.t, w.b, w.h), "bf16"))
    dX = blk.backward(X, dev(inp["dZ"], "bf16"))
    Xo = O.as_f64(Xfull, "bf16").reshape(w.M, w.h)
    A, B = O.as_f64(inp["A"], "bf16"), O.as_f64(inp["B"], "bf16")
    a, c = O.as_f64(inp["a"], "bf16"), O.as_f64(inp["c"], "bf16")
    full = O.mlp_forward(Xo, A, B, w.act, a, c)
    bwd = O.mlp_backward(Xo, A, B, full["U"], full["Y"], O.as_f64(inp["dZ"], "bf16").reshape(w.M, w.h), w.act)
    check_close(f64(Z_ar), full["Z"], "bf16", "Z (all-reduce)")
    assert torch.equal(Z_rs.reshape(-1).view(torch.int16), Z_ar.reshape(-1).view(torch.int16))
    check_close(f64(dX), bwd["dX"], "bf16", "dX")
    for r in range(w.t):
        check_close(f64(blk.dA[r]), bwd["dA"][:, O.mlp_shard_columns(w.ffn, w.t, r, w.act)], "bf16", "dA")


def test_deterministic_bits(L):
    w = TI.Workload("det", "mlp", s=64, b=4, h=264, ffn=2 * 320, t=2, act="gelu", dtype="bf16")
    say("bf16 MLP run twice, identical bits")
    inp = TI.mlp_inputs(w, with_bias=True, seed=2)
    g1 = run_rank(L, w, inp, 0, "bf16", True)
    g2 = run_rank(L, w, inp, 0, "bf16", True)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k].view(torch.int16), g2[k].view(torch.int16)), k
