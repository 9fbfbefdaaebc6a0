"""Pins of the oracle's attention backward (CPU, fp64) against things other than its own formulas.

* central finite differences of the oracle's forward (the core and the whole block with biases and weights);
* torch's fp64 autograd of scaled_dot_product_attention (an independent library routine);
* closed forms: one key (dV = dO, dQ = dK = 0) and Q = 0 (uniform causal weights);
* invariants of the softmax Jacobian: shifting every key by one vector changes each score row by a constant, so
  no gradient changes; and the key gradients sum to zero over the keys.  Both fail if the row-sum term of the
  softmax derivative is dropped;
* the shards of the block backward sum (dX) or slice (weights, dQKV) to the unsharded gradients ("Tensor
  Parallelism (TP) 与 Sequence Parallelism (SP)" §2 and §5: the f operator's backward is the sum over ranks;
  the weight gradients stay local).
"""
import math

import numpy as np
import pytest

import oracle as O



def _rng(seed):
    return np.random.default_rng(seed)


def _fd(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("causal", [True, False])
def test_core_backward_by_finite_differences(causal):
    r = _rng(1)
    s, d = 5, 3
    Q, K, V, G = (r.standard_normal((s, d)) for _ in range(4))

    def loss():
        return float((O.attention_core(Q, K, V, causal)[0] * G).sum())

    dQ, dK, dV = O.attention_core_backward(Q, K, V, G, causal)
    for name, x, g in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        fd = _fd(loss, x)
        assert np.allclose(g, fd, rtol=1e-6, atol=1e-8), name


@pytest.mark.parametrize("causal", [True, False])
def test_core_backward_against_torch_autograd(causal):
    torch = pytest.importorskip("torch")
    r = _rng(2)
    s, d = 7, 4
    Q, K, V, G = (r.standard_normal((s, d)) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], is_causal=causal)[0]
    out.backward(torch.tensor(G, dtype=torch.float64))
    dQ, dK, dV = O.attention_core_backward(Q, K, V, G, causal)
    assert np.allclose(dQ, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dK, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dV, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_core_backward_closed_forms():
    r = _rng(3)
    # a single key: P = 1, O = V, so dV = dO and nothing reaches Q or K
    Q, K, V, G = (r.standard_normal((1, 4)) for _ in range(4))
    dQ, dK, dV = O.attention_core_backward(Q, K, V, G, True)
    assert np.allclose(dV, G) and np.allclose(dQ, 0) and np.allclose(dK, 0)
    # Q = 0, causal: P[q, k] = 1 / (q + 1) for k <= q, so dV[k] = sum_{q >= k} dO[q] / (q + 1)
    s, d = 6, 3
    K, V, G = (r.standard_normal((s, d)) for _ in range(3))
    _, _, dV = O.attention_core_backward(np.zeros((s, d)), K, V, G, True)
    want = np.array([sum(G[q] / (q + 1) for q in range(k, s)) for k in range(s)])
    assert np.allclose(dV, want)


@pytest.mark.parametrize("causal", [True, False])
def test_core_backward_softmax_invariants(causal):
    r = _rng(4)
    s, d = 6, 4
    Q, K, V, G = (r.standard_normal((s, d)) for _ in range(4))
    base = O.attention_core_backward(Q, K, V, G, causal)
    shifted = O.attention_core_backward(Q, K + r.standard_normal(d)[None, :], V, G, causal)
    for a, b in zip(base, shifted):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-12)
    assert np.allclose(base[1].sum(axis=0), 0.0, atol=1e-12)


def _block_inputs(seed, s=3, b=2, a=2, d=2):
    r = _rng(seed)
    h = a * d
    X = r.standard_normal((s * b, h))
    Wqkv = r.standard_normal((h, 3 * a * d)) * 0.5
    Wo = r.standard_normal((a * d, h)) * 0.5
    bqkv = r.standard_normal(3 * a * d) * 0.1
    dZ = r.standard_normal((s * b, h))
    return X, Wqkv, Wo, bqkv, dZ


def test_block_backward_by_finite_differences():
    s, b, a, d = 3, 2, 2, 2
    X, Wqkv, Wo, bqkv, dZ = _block_inputs(5, s, b, a, d)

    def loss():
        return float((O.attention_forward(X, Wqkv, Wo, s, b, a, d, True, bqkv)["Z"] * dZ).sum())

    g = O.attention_backward(X, Wqkv, Wo, dZ, s, b, a, d, True, bqkv)
    for name, x, want in (("X", X, g["dX"]), ("Wqkv", Wqkv, g["dWqkv"]), ("Wo", Wo, g["dWo"]),
                          ("bqkv", bqkv, g["dbqkv"])):
        fd = _fd(loss, x)
        assert np.allclose(want, fd, rtol=1e-6, atol=1e-8), name


def test_shard_backward_sums_and_slices_to_unsharded():
    s, b, a, d, t = 4, 2, 4, 2, 2
    X, Wqkv, Wo, bqkv, dZ = _block_inputs(6, s, b, a, d)
    full = O.attention_backward(X, Wqkv, Wo, dZ, s, b, a, d, True, bqkv)
    dX = np.zeros_like(full["dX"])
    hl = a // t
    for r in range(t):
        sh = O.attention_shard_backward(X, Wqkv, Wo, dZ, s, b, a, d, t, r, True, bqkv)
        cols = O.qkv_shard_columns(a, d, t, r)
        rows = slice(r * hl * d, (r + 1) * hl * d)
        assert np.allclose(sh["dQKV"], full["dQKV"][:, cols], rtol=1e-12, atol=1e-12)
        assert np.allclose(sh["dWqkv"], full["dWqkv"][:, cols], rtol=1e-12, atol=1e-12)
        assert np.allclose(sh["dbqkv"], full["dbqkv"][cols], rtol=1e-12, atol=1e-12)
        assert np.allclose(sh["dWo"], full["dWo"][rows], rtol=1e-12, atol=1e-12)
        assert np.allclose(sh["dO"], full["dO"][:, rows], rtol=1e-12, atol=1e-12)
        dX += sh["dX"]
    assert np.allclose(dX, full["dX"], rtol=1e-12, atol=1e-12)
