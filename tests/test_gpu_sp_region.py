"""Sequence-parallel region (dropout + residual add + LayerNorm on one rank's [s/t, b, h] rows) against the
oracle, through the C ABI.

* forward: the keep mask bit for bit (the decision compares integers on both sides), u = residual + dropout(z),
  y = LayerNorm(u), mean and rstd, at small ragged sizes (row lengths that leave a partial chunk of threads, the
  512-thread row shape, the largest supported h) and both dtypes;
* backward: dres / dz, and the LayerNorm weight gradients, from oracle-made saved statistics and mask;
* the sequence-parallel round trip at the full SP SwiGLU workload shape (s=4096, b=1, h=8192, t=8): every rank's
  forward writes its LayerNorm output straight into its rows of the gathered [s, b, h] buffer, every rank's
  backward gives its part of dgamma / dbeta, and the t parts summed by tp_partial_reduce (fp32) equal the
  unsharded oracle's gradients.

Tolerances: fp32 outputs relative Frobenius <= 1e-5; bf16 outputs 1e-2 / 3e-2 (unit scale).  dgamma / dbeta are
fp32 sums of exactly represented products in both dtypes, so they take the fp32 bound.  The oracle runs on the
same input bits (fp64); the bf16 kernels normalise the stored (rounded) u, whose rounding sits well inside the
bf16 bound.
"""
import numpy as np
import pytest
import torch

import oracle as O
import tp_inputs as TI
from parity_utils import check_close, dev, empty, f64, say

pytestmark = pytest.mark.gpu

EPS = 1e-5


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_block_columnparallel_amd as pkg

    return pkg.load()


def val(x, dtype):
    return O.bf16_bits_to_f64(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def packed_keep(bits, p):
    """The documented mask layout: bit i of byte k of a row = keep of column 8k + i."""
    return np.packbits(O.dropout_keep(bits, p), axis=1, bitorder="little")


def run_fwd(L, inp, rows, h, p, dtype, with_res=True, y=None):
    z, res = dev(inp["z"], dtype), dev(inp["residual"], dtype) if with_res else None
    bits = torch.from_numpy(inp["bits"].view(np.int32)).cuda()
    gam, bet = dev(inp["gamma"], dtype), dev(inp["beta"], dtype)
    out, y = empty((rows, h), dtype), (empty((rows, h), dtype) if y is None else y)
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    mask = torch.empty((rows, h // 8), dtype=torch.uint8, device="cuda")
    L.tp_sp_dropout_add_ln_fwd(rows, h, p, EPS, z, res, bits, gam, bet, out, y, mean, rstd, mask, dtype=dtype)
    return out, y, mean, rstd, mask


def oracle_fwd(inp, p, dtype, with_res=True):
    z = val(inp["z"], dtype)
    res = val(inp["residual"], dtype) if with_res else np.zeros_like(z)
    u = O.dropout_add(z, res, inp["bits"], p)
    y, mean, rstd = O.layernorm(u, val(inp["gamma"], dtype), val(inp["beta"], dtype), EPS)
    return u, y, mean, rstd


FWD_CASES = [  # rows, h, p, dtype, residual
    (1, 8, 0.1, "bf16", True),
    (3, 24, 0.0, "bf16", True),
    (37, 264, 0.1, "bf16", False),
    (5, 2056, 0.5, "bf16", True),     # 257 chunks: a second, nearly empty chunk per thread
    (7, 6144, 0.1, "bf16", True),     # 3 chunks per thread, 256 threads
    (3, 8200, 0.1, "bf16", True),     # 512-thread rows with a partial third chunk
    (2, 12288, 0.25, "bf16", True),   # largest supported row
    (9, 264, 0.1, "f32", True),
    (4, 4096, 0.0, "f32", False),
    (3, 8192, 0.3, "f32", True),
]


@pytest.mark.parametrize("rows,h,p,dtype,with_res", FWD_CASES)
def test_fwd_matches_oracle(L, rows, h, p, dtype, with_res):
    say(f"sp fwd rows={rows} h={h} p={p} {dtype} residual={with_res}")
    inp = TI.sp_region_inputs(rows, h, dtype, seed=rows + h)
    out, y, mean, rstd, mask = run_fwd(L, inp, rows, h, p, dtype, with_res)
    torch.cuda.synchronize()
    u_ref, y_ref, mean_ref, rstd_ref = oracle_fwd(inp, p, dtype, with_res)
    assert np.array_equal(mask.cpu().numpy(), packed_keep(inp["bits"], p))
    check_close(f64(out), u_ref, dtype, "u")
    check_close(f64(y), y_ref, dtype, "y")
    check_close(f64(mean), mean_ref, dtype, "mean")
    check_close(f64(rstd), rstd_ref, dtype, "rstd")


BWD_CASES = [  # rows, h, p, dtype, dres_in present
    (1, 8, 0.1, "bf16", True),
    (3, 24, 0.0, "bf16", False),
    (37, 264, 0.1, "bf16", True),
    (300, 1032, 0.2, "bf16", True),   # more rows than workgroups: each strides over two rows
    (5, 6144, 0.1, "bf16", False),
    (3, 8200, 0.5, "bf16", True),
    (2, 12288, 0.1, "bf16", True),
    (9, 264, 0.1, "f32", True),
    (261, 4096, 0.0, "f32", True),
    (3, 8192, 0.3, "f32", False),
]


@pytest.mark.parametrize("rows,h,p,dtype,with_dres", BWD_CASES)
def test_bwd_matches_oracle(L, rows, h, p, dtype, with_dres):
    say(f"sp bwd rows={rows} h={h} p={p} {dtype} dres_in={with_dres}")
    inp = TI.sp_region_inputs(rows, h, dtype, seed=7 * rows + h)
    u = val(inp["x"], dtype)  # the saved LayerNorm input
    gam = val(inp["gamma"], dtype)
    _, mean, rstd = O.layernorm(u, gam, np.zeros(h), EPS)
    dy = val(inp["dy"], dtype)
    dres_in = val(inp["residual"], dtype) if with_dres else np.zeros_like(u)
    dx, dg_ref, db_ref = O.layernorm_backward(u, gam, dy, EPS)
    G = dx + dres_in
    dz_ref, dres_ref = O.dropout_add_backward(G, inp["bits"], p)

    mask = torch.from_numpy(packed_keep(inp["bits"], p)).cuda()
    mean_t = torch.from_numpy(mean.astype(np.float32)).cuda()
    rstd_t = torch.from_numpy(rstd.astype(np.float32)).cuda()
    dres, dz = empty((rows, h), dtype), empty((rows, h), dtype)
    dgamma = torch.empty(h, dtype=torch.float32, device="cuda")
    dbeta = torch.empty(h, dtype=torch.float32, device="cuda")
    ws = torch.empty(L.tp_sp_ln_bwd_workspace(rows, h) // 4, dtype=torch.float32, device="cuda")
    L.tp_sp_dropout_add_ln_bwd(rows, h, p, dev(inp["x"], dtype), dev(inp["gamma"], dtype), mean_t, rstd_t,
                               dev(inp["dy"], dtype), dev(inp["residual"], dtype) if with_dres else None, mask,
                               dres, dz, dgamma, dbeta, ws, dtype=dtype)
    torch.cuda.synchronize()
    check_close(f64(dres), dres_ref, dtype, "dres")
    check_close(f64(dz), dz_ref, dtype, "dz")
    check_close(f64(dgamma), dg_ref, "f32", "dgamma")
    check_close(f64(dbeta), db_ref, "f32", "dbeta")
    # dropped elements carry exactly zero gradient into z
    keep = O.dropout_keep(inp["bits"], p)
    assert np.all(f64(dz)[~keep] == 0.0)


def test_optional_outputs_may_be_null(L):
    rows, h, p = 6, 512, 0.1
    inp = TI.sp_region_inputs(rows, h, "bf16", seed=3)
    z, bits = dev(inp["z"], "bf16"), torch.from_numpy(inp["bits"].view(np.int32)).cuda()
    gam, bet = dev(inp["gamma"], "bf16"), dev(inp["beta"], "bf16")
    y = empty((rows, h), "bf16")
    L.tp_sp_dropout_add_ln_fwd(rows, h, p, EPS, z, None, bits, gam, bet, None, y, None, None, None, dtype="bf16")
    torch.cuda.synchronize()
    _, y_ref, _, _ = oracle_fwd(inp, p, "bf16", with_res=False)
    check_close(f64(y), y_ref, "bf16", "y")


def test_sp_round_trip_full_shape(L):
    """SP SwiGLU workload: s=4096, b=1, h=8192, t=8 -> 512 rows of 8192 per rank."""
    s, b, h, t, p = 4096, 1, 8192, 8, 0.1
    rows = s // t * b
    inp = TI.sp_region_inputs(s * b, h, "bf16", seed=11)
    say(f"sp round trip s={s} b={b} h={h} t={t} p={p}")
    z, res = dev(inp["z"], "bf16"), dev(inp["residual"], "bf16")
    bits = torch.from_numpy(inp["bits"].view(np.int32)).cuda()
    gam, bet = dev(inp["gamma"], "bf16"), dev(inp["beta"], "bf16")
    dy = dev(inp["dy"], "bf16")
    Yg = torch.full((s * b, h), float("nan"), dtype=torch.bfloat16, device="cuda")  # the gathered buffer
    U = empty((s * b, h), "bf16")
    mean = torch.empty(s * b, dtype=torch.float32, device="cuda")
    rstd = torch.empty(s * b, dtype=torch.float32, device="cuda")
    mask = torch.empty((s * b, h // 8), dtype=torch.uint8, device="cuda")
    dres, dz = empty((s * b, h), "bf16"), empty((s * b, h), "bf16")
    parts = torch.empty((2 * t, h), dtype=torch.float32, device="cuda")  # [dgamma_0..t-1 | dbeta_0..t-1]
    ws = torch.empty(L.tp_sp_ln_bwd_workspace(rows, h) // 4, dtype=torch.float32, device="cuda")
    for r in range(t):
        sl = slice(r * rows, (r + 1) * rows)
        L.tp_sp_dropout_add_ln_fwd(rows, h, p, EPS, z[sl], res[sl], bits[sl], gam, bet, U[sl], Yg[sl], mean[sl],
                                   rstd[sl], mask[sl], dtype="bf16")
    for r in range(t):
        sl = slice(r * rows, (r + 1) * rows)
        L.tp_sp_dropout_add_ln_bwd(rows, h, p, U[sl], gam, mean[sl], rstd[sl], dy[sl], None, mask[sl], dres[sl],
                                   dz[sl], parts[r], parts[t + r], ws, dtype="bf16")
    dgamma = torch.empty(h, dtype=torch.float32, device="cuda")
    dbeta = torch.empty(h, dtype=torch.float32, device="cuda")
    L.tp_partial_reduce(h, h, t, parts[:t], None, dgamma, dtype="f32")
    L.tp_partial_reduce(h, h, t, parts[t:], None, dbeta, dtype="f32")
    torch.cuda.synchronize()

    u_ref, y_ref, mean_ref, rstd_ref = oracle_fwd(inp, p, "bf16")
    assert np.array_equal(mask.cpu().numpy(), packed_keep(inp["bits"], p))
    check_close(f64(U), u_ref, "bf16", "u")
    check_close(f64(Yg), y_ref, "bf16", "gathered y")  # every row written (the NaN fill would fail)
    check_close(f64(mean), mean_ref, "bf16", "mean")
    check_close(f64(rstd), rstd_ref, "bf16", "rstd")
    dx, dg_ref, db_ref = O.layernorm_backward(u_ref, val(inp["gamma"], "bf16"), val(inp["dy"], "bf16"), EPS)
    dz_ref, dres_ref = O.dropout_add_backward(dx, inp["bits"], p)
    check_close(f64(dres), dres_ref, "bf16", "dres")
    check_close(f64(dz), dz_ref, "bf16", "dz")
    # the backward ran on the rounded u, the oracle on the exact one: bf16 bound for the summed weight gradients
    rf_g, _ = check_close(f64(dgamma), dg_ref, "bf16", "dgamma (sum over ranks)")
    rf_b, _ = check_close(f64(dbeta), db_ref, "f32", "dbeta (sum over ranks)")
    say(f"round trip: dgamma rel {rf_g:.2e}, dbeta rel {rf_b:.2e}")
