"""Pins of the oracle's bf16 data-flow chains (store="bf16"), CPU only.

The block keeps its activations in 16 bits between steps ([MEGA] calculator and [ATLAS] §5 size them at 2 bytes),
at the points the C ABI names as stored buffers: U_i, Y_i and dU_i of the MLP; QKV_i, O_i, dO and dQKV_i of the
attention block.  These tests work out one-element cases by hand -- math.erf for GeLU, torch's own bf16 conversion
for the rounding (not the oracle's converter) -- so a rounding put at the wrong step, missing, or applied to the
step's output instead of the next step's input fails here.  store=None must leave the exact chain untouched.
"""
import math

import numpy as np
import torch

import oracle as O


def bf(v: float) -> float:
    """bf16 round-to-nearest-even of v through torch's CPU conversion (fp64 -> fp32 -> bf16)."""
    return float(torch.tensor(v, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64))


def gelu(u: float) -> float:
    return 0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0)))


def gelu_d(u: float) -> float:
    return 0.5 * (1.0 + math.erf(u / math.sqrt(2.0))) + u * math.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def test_store_none_is_the_exact_chain():
    rng = np.random.default_rng(0)
    X, A, B, dZ = rng.normal(size=(6, 4)), rng.normal(size=(4, 8)), rng.normal(size=(8, 4)), rng.normal(size=(6, 4))
    for r in range(2):
        a = O.mlp_shard_backward(X, A, B, dZ, 2, r, "gelu")
        b = O.mlp_shard_backward(X, A, B, dZ, 2, r, "gelu", store=None)
        for k in a:
            assert np.array_equal(a[k], b[k])
    Wq, Wo = rng.normal(size=(4, 12)), rng.normal(size=(4, 4))
    a = O.attention_shard_backward(X, Wq, Wo, dZ, 3, 2, 2, 2, 2, 1, True)
    b = O.attention_shard_backward(X, Wq, Wo, dZ, 3, 2, 2, 2, 2, 1, True, store=None)
    for k in a:
        assert np.array_equal(a[k], b[k])


def test_mlp_one_element_by_hand():
    # s = b = h = 1, ffn = 1, t = 1, GeLU: every quantity is a scalar and none of them is a bf16 value
    x, a, b, dz = 1.0, 0.7123456789, -1.3579246801, 0.4142135623
    X, A, B, dZ = np.array([[x]]), np.array([[a]]), np.array([[b]]), np.array([[dz]])
    fw = O.mlp_shard_forward(X, A, B, 1, 0, "gelu", store="bf16")
    bw = O.mlp_shard_backward(X, A, B, dZ, 1, 0, "gelu", store="bf16")
    u = x * a
    assert fw["U"][0, 0] == u and fw["Y"][0, 0] == gelu(u)           # pre-rounding values of their steps
    assert abs(fw["Z"][0, 0] - bf(gelu(u)) * b) < 1e-15                # the row GEMM reads the stored Y
    dy = dz * b
    du = dy * gelu_d(bf(u))                                            # act' reads the stored U
    assert abs(bw["dY"][0, 0] - dy) < 1e-15
    assert abs(bw["dU"][0, 0] - du) < 1e-15
    assert abs(bw["dB"][0, 0] - bf(gelu(u)) * dz) < 1e-15             # wgrad reads the stored Y
    assert abs(bw["dA"][0, 0] - x * bf(du)) < 1e-15                    # both GEMMs read the stored dU
    assert abs(bw["dX"][0, 0] - bf(du) * a) < 1e-15
    assert abs(bw["da"][0] - bf(du)) < 1e-15
    # and the storage is visible: each differs from the exact chain
    ex = O.mlp_shard_backward(X, A, B, dZ, 1, 0, "gelu")
    for k in ("dU", "dA", "dB", "dX"):
        assert bw[k][0, 0] != ex[k][0, 0], k
    # sampled helpers follow the same flow
    rows = O.mlp_shard_rows(X, dZ, A, B, 1, 0, "gelu", store="bf16")
    for k in ("U", "Y", "Z", "dU", "dX"):
        assert abs(rows[k][0, 0] - {**fw, **bw}[k][0, 0]) < 1e-15, k
    cols = O.mlp_shard_weight_grad_cols(X, dZ, A, B, 1, 0, [0], "gelu", store="bf16")
    assert abs(cols["dB_rows"][0, 0] - bw["dB"][0, 0]) < 1e-15
    assert abs(cols["dA_cols"][0, 0] - bw["dA"][0, 0]) < 1e-15


def test_attention_single_key_by_hand():
    # s = 1, b = 1, one head of d = 2, t = 1: the only key is the query's own, P = 1, so O = V, dV = dO, dQ = dK = 0
    rng = np.random.default_rng(7)
    d, h = 2, 2
    X = rng.normal(size=(1, h))
    Wqkv = rng.normal(size=(h, 3 * d))
    Wo = rng.normal(size=(d, h))
    dZ = rng.normal(size=(1, h))
    r = O.attention_shard_backward(X, Wqkv, Wo, dZ, 1, 1, 1, d, 1, 0, True, store="bf16")
    qkv = X[0] @ Wqkv
    v = qkv[2 * d:]
    v_s = np.array([bf(e) for e in v])
    assert np.allclose(r["QKV"][0], qkv, rtol=0, atol=1e-15)
    assert np.allclose(r["O"][0], v_s, rtol=0, atol=1e-15)            # attention reads the stored V
    z = np.array([bf(e) for e in v_s]) @ Wo                            # the projection reads the stored O
    assert np.allclose(r["Z"][0], z, rtol=0, atol=1e-14)
    do = dZ[0] @ Wo.T
    assert np.allclose(r["dO"][0], do, rtol=0, atol=1e-15)
    dqkv = np.concatenate([np.zeros(2 * d), [bf(e) for e in do]])     # dV = stored dO; dQ = dK = 0
    assert np.allclose(r["dQKV"][0], dqkv, rtol=0, atol=1e-15)
    dqkv_s = np.array([bf(e) for e in dqkv])                           # the GEMMs read the stored dQKV
    assert np.allclose(r["dWqkv"], np.outer(X[0], dqkv_s), rtol=0, atol=1e-14)
    assert np.allclose(r["dX"][0], dqkv_s @ Wqkv.T, rtol=0, atol=1e-14)
    assert np.allclose(r["dbqkv"], dqkv_s, rtol=0, atol=1e-15)
    assert np.allclose(r["dWo"], np.outer(v_s, dZ[0]), rtol=0, atol=1e-14)  # dWo reads the stored O
    ex = O.attention_shard_backward(X, Wqkv, Wo, dZ, 1, 1, 1, d, 1, 0, True)
    assert not np.array_equal(ex["dX"], r["dX"])
