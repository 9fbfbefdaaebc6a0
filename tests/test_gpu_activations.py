"""The fused activation epilogues against the exact functions, through the C ABI.

With identity weights the column GEMM reproduces its input exactly (each output is x * 1 plus exact zeros, in fp32
accumulation), so the forward's Y is act(x) on a chosen grid of x, and with dZ = 1 and B = I the backward's dU is
act'(x).  The reference values are the oracle's GeLU / GeLU' / sigmoid (fp64, pinned against math.erf and finite
differences in the oracle tests).

* fp32 path: GeLU and GeLU' within the error bound of the rational erfc approximation the kernels use
  (Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26: |error| <= 1.5e-7 on erf) plus fp32
  evaluation rounding; SwiGLU forward and backward within a few fp32 roundings of the sigmoid.
* bf16 path, small (register-staged kernel) and large (large-tile kernel): within one bf16 ulp of the exact value.
"""
import numpy as np
import pytest
import torch

import oracle as O
from parity_utils import f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_block_columnparallel_amd as pkg

    return pkg.load()


def _grid(n, lo=-12.0, hi=12.0):
    x = np.linspace(lo, hi, n - 8).astype(np.float32)
    special = np.array([0.0, -0.0, 1e-30, -1e-30, 40.0, -40.0, 1.0, -1.0], dtype=np.float32)
    return np.concatenate([special, x])


def _run(L, act, x, h, dtype):
    """Forward and backward of one t = 1 block with identity weights on inputs x [M * h]."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    M = x.size // h
    n1 = 2 * h if act == "swiglu" else h
    Xh = torch.from_numpy(x.reshape(M, h)).to(tdt)
    X = Xh.cuda()
    eye = torch.eye(h, dtype=tdt, device="cuda")
    A = torch.cat([eye, eye], dim=1).contiguous() if act == "swiglu" else eye
    B = eye.clone()
    dims = L.make_dims(s=M, b=1, h=h, ffn=h, t=1)
    U = torch.empty((M, n1), dtype=tdt, device="cuda")
    Y = torch.empty((M, h), dtype=tdt, device="cuda")
    Z = torch.empty((M, h), dtype=tdt, device="cuda")
    L.tp_mlp_fwd(dims, 0, act, X, A, None, B, U, Y, Z)
    dZ = torch.ones((M, h), dtype=tdt, device="cuda")
    dU = torch.empty((M, n1), dtype=tdt, device="cuda")
    dA = torch.empty((h, n1), dtype=tdt, device="cuda")
    dB = torch.empty((h, h), dtype=tdt, device="cuda")
    dX = torch.empty((M, h), dtype=tdt, device="cuda")
    L.tp_mlp_bwd(dims, 0, act, X, A, B, U, Y, dZ, dU, dA, None, dB, dX)
    torch.cuda.synchronize()
    xin = f64(Xh).reshape(-1)  # the input as the host rounded it (the device holds the same bits)
    # the exactness the test rests on: the identity GEMM returns its input
    u = f64(U)
    assert np.array_equal(u[:, :h].reshape(-1), xin)
    if act == "swiglu":
        assert np.array_equal(u[:, h:].reshape(-1), xin)
    return xin, f64(Y).reshape(-1), f64(dU)


def _bf16_ulp(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_activations_fp32_within_approximation_bound(L, act):
    h = 64
    x = _grid(1024 * h)
    xin, y, du = _run(L, act, x, h, "f32")
    ax = np.maximum(1.0, np.abs(xin))
    if act == "gelu":
        err_y = np.abs(y - O.gelu(xin))
        err_d = np.abs(du.reshape(-1) - O.gelu_grad(xin))
        say(f"gelu fp32: max |Y - gelu| / max(1,|x|) = {np.max(err_y / ax):.2e}, "
            f"max |dU - gelu'| / max(1,|x|) = {np.max(err_d / ax):.2e}")
        # 0.5 |x| * 1.5e-7 from the approximation, the rest fp32 evaluation
        assert np.all(err_y <= 5e-7 * ax)
        assert np.all(err_d <= 1e-6 * ax)
    else:
        sg = O.sigmoid(xin)
        ref_y = xin * sg * xin
        tol = (1e-6 + 2e-7 * np.abs(xin))
        err_y = np.abs(y - ref_y)
        assert np.all(err_y <= tol * np.abs(ref_y) + 1e-37), np.max(err_y / (np.abs(ref_y) + 1e-37))
        dg, du_ = du[:, :h].reshape(-1), du[:, h:].reshape(-1)
        ref_dg = xin * sg * (1.0 + xin * (1.0 - sg))  # dY * u * silu'(g) with dY = 1, u = g = x
        ref_du = xin * sg                               # dY * silu(g)
        scale_g = np.abs(xin) * sg * (1.0 + np.abs(xin) * (1.0 - sg))
        assert np.all(np.abs(dg - ref_dg) <= 2 * tol * scale_g + 1e-37)
        assert np.all(np.abs(du_ - ref_du) <= tol * np.abs(ref_du) + 1e-37)
        say(f"swiglu fp32: max rel err Y {np.max(err_y / (np.abs(ref_y) + 1e-30)):.2e}")


@pytest.mark.parametrize("rows", [1024, 65536], ids=["register_staged", "large_tile"])
def test_gelu_bf16_within_one_ulp(L, rows):
    h = 64 if rows == 1024 else 256
    x = _grid(rows * h, -8.0, 8.0)
    xin, y, du = _run(L, "gelu", x, h, "bf16")
    ref_y, ref_d = O.gelu(xin), O.gelu_grad(xin)
    ey = np.abs(y - ref_y) / (_bf16_ulp(ref_y) + 1e-6 * np.maximum(1.0, np.abs(xin)))
    ed = np.abs(du.reshape(-1) - ref_d) / (_bf16_ulp(ref_d) + 1e-6 * np.maximum(1.0, np.abs(xin)))
    say(f"gelu bf16 rows={rows}: max error in bf16 ulps Y {ey.max():.2f}, dU {ed.max():.2f}")
    assert ey.max() <= 1.0 and ed.max() <= 1.0
