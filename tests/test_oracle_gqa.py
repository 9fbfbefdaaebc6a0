"""Pins of the oracle's grouped-query attention (g KV heads shared by a/g query heads each), forward and backward.

* layout: the shard columns of index-valued weights decode to the interleave the Megatron-LM visual reading prints
  for the fused QKV weight under GQA, [q1 q2 k1 v1 | q3 q4 k2 v2 | ...], one group after another by rank;
* torch's fp64 scaled_dot_product_attention with enable_gqa (an independent library routine), outputs and
  autograd gradients;
* reduction to multi-head attention: repeating each KV head's weight columns for the query heads of its group
  gives an MHA block with the same output, and the GQA key / value weight gradients are the sums of the repeated
  heads' MHA gradients (fails if a group's dK / dV were overwritten instead of summed);
* finite differences of the block; the shards sum (dX) or slice (dQKV, weights) to the unsharded gradients.
"""
import numpy as np
import pytest

import oracle as O


def test_shard_columns_decode_to_the_pages_interleave():
    a, g, d, t = 4, 2, 1, 1
    full = np.arange((a + 2 * g) * d)  # [q1 q2 q3 q4 | k1 k2 | v1 v2] as column ids 0..7
    cols = O.qkv_shard_columns(a, d, t, 0, g)
    assert list(full[cols]) == [0, 1, 4, 6, 2, 3, 5, 7]  # q1 q2 k1 v1 | q3 q4 k2 v2
    # t = 2: each rank owns one group, d = 2 keeps each head's columns contiguous
    d = 2
    assert list(O.qkv_shard_columns(a, d, 2, 1, g)) == [4, 5, 6, 7, 10, 11, 14, 15]
    # g = a is the multi-head layout [q_j | k_j | v_j]
    assert list(O.qkv_shard_columns(2, 1, 1, 0, 2)) == list(O.qkv_shard_columns(2, 1, 1, 0)) == [0, 2, 4, 1, 3, 5]
    with pytest.raises(ValueError):
        O.qkv_shard_columns(4, 1, 4, 0, 2)  # fewer KV heads than ranks: a rank would not own a whole group


def _block(seed, s=5, b=2, a=4, g=2, d=3):
    r = np.random.default_rng(seed)
    h = 6
    X = r.standard_normal((s * b, h))
    Wqkv = r.standard_normal((h, (a + 2 * g) * d)) * 0.5
    Wo = r.standard_normal((a * d, h)) * 0.5
    bqkv = r.standard_normal((a + 2 * g) * d) * 0.1
    dZ = r.standard_normal((s * b, h))
    return X, Wqkv, Wo, bqkv, dZ


@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_sdpa_gqa(causal):
    torch = pytest.importorskip("torch")
    s, b, a, g, d = 6, 2, 4, 2, 3
    X, Wqkv, Wo, bqkv, dZ = _block(1, s, b, a, g, d)
    fw = O.attention_forward(X, Wqkv, Wo, s, b, a, d, causal, bqkv, g=g)
    QKV = fw["QKV"]

    def heads(cols, n):  # [M = s*b, n*d] -> [b, n, s, d]
        return torch.tensor(QKV[:, cols].reshape(s, b, n, d).transpose(1, 2, 0, 3).copy(), requires_grad=True)

    q = heads(slice(0, a * d), a)
    k = heads(slice(a * d, (a + g) * d), g)
    v = heads(slice((a + g) * d, (a + 2 * g) * d), g)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=True)
    o_ref = out.detach().numpy().transpose(2, 0, 1, 3).reshape(s * b, a * d)
    assert np.allclose(fw["O"], o_ref, rtol=1e-12, atol=1e-12)
    dO = dZ @ Wo.T
    out.backward(torch.tensor(dO.reshape(s, b, a, d).transpose(1, 2, 0, 3).copy()))
    bw = O.attention_backward(X, Wqkv, Wo, dZ, s, b, a, d, causal, bqkv, g=g)

    def flat(tg, n):
        return tg.grad.numpy().transpose(2, 0, 1, 3).reshape(s * b, n * d)

    assert np.allclose(bw["dQKV"][:, :a * d], flat(q, a), rtol=1e-10, atol=1e-12)
    assert np.allclose(bw["dQKV"][:, a * d:(a + g) * d], flat(k, g), rtol=1e-10, atol=1e-12)
    assert np.allclose(bw["dQKV"][:, (a + g) * d:], flat(v, g), rtol=1e-10, atol=1e-12)


def test_reduces_to_mha_with_repeated_kv_heads():
    s, b, a, g, d = 5, 2, 6, 2, 2
    G = a // g
    X, Wqkv, Wo, bqkv, dZ = _block(2, s, b, a, g, d)
    # MHA weight: query columns as they are, key / value head j = the group's head j // G
    rep = [j // G for j in range(a)]
    kcols = np.concatenate([np.arange(a * d + r * d, a * d + (r + 1) * d) for r in rep])
    vcols = np.concatenate([np.arange((a + g) * d + r * d, (a + g) * d + (r + 1) * d) for r in rep])
    mcols = np.concatenate([np.arange(a * d), kcols, vcols])
    W_mha, b_mha = Wqkv[:, mcols], bqkv[mcols]
    gq = O.attention_forward(X, Wqkv, Wo, s, b, a, d, True, bqkv, g=g)
    mh = O.attention_forward(X, W_mha, Wo, s, b, a, d, True, b_mha)
    assert np.allclose(gq["Z"], mh["Z"], rtol=1e-12, atol=1e-12)
    gb = O.attention_backward(X, Wqkv, Wo, dZ, s, b, a, d, True, bqkv, g=g)
    mb = O.attention_backward(X, W_mha, Wo, dZ, s, b, a, d, True, b_mha)
    assert np.allclose(gb["dX"], mb["dX"], rtol=1e-12, atol=1e-12)
    want = np.zeros_like(gb["dWqkv"])
    np.add.at(want.T, mcols, mb["dWqkv"].T)  # repeated columns' gradients add up in the shared column
    assert np.allclose(gb["dWqkv"], want, rtol=1e-12, atol=1e-12)


def test_block_backward_by_finite_differences():
    s, b, a, g, d = 4, 1, 4, 2, 2
    X, Wqkv, Wo, bqkv, dZ = _block(3, s, b, a, g, d)

    def loss():
        return float((O.attention_forward(X, Wqkv, Wo, s, b, a, d, True, bqkv, g=g)["Z"] * dZ).sum())

    bw = O.attention_backward(X, Wqkv, Wo, dZ, s, b, a, d, True, bqkv, g=g)
    for name, x, want in (("X", X, bw["dX"]), ("Wqkv", Wqkv, bw["dWqkv"]), ("bqkv", bqkv, bw["dbqkv"])):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + 1e-6
            fp = loss()
            x[i] = old - 1e-6
            fm = loss()
            x[i] = old
            fd[i] = (fp - fm) / 2e-6
        assert np.allclose(want, fd, rtol=1e-6, atol=1e-8), name


def test_shards_sum_and_slice_to_unsharded():
    s, b, a, g, d, t = 4, 2, 8, 4, 2, 2
    X, Wqkv, Wo, bqkv, dZ = _block(4, s, b, a, g, d)
    full = O.attention_backward(X, Wqkv, Wo, dZ, s, b, a, d, True, bqkv, g=g)
    fz = O.attention_forward(X, Wqkv, Wo, s, b, a, d, True, bqkv, g=g)
    dX = np.zeros_like(full["dX"])
    Z = np.zeros_like(fz["Z"])
    for r in range(t):
        sh = O.attention_shard_backward(X, Wqkv, Wo, dZ, s, b, a, d, t, r, True, bqkv, g=g)
        fw = O.attention_shard_forward(X, Wqkv, Wo, s, b, a, d, t, r, True, bqkv, g=g)
        cols = O.qkv_shard_columns(a, d, t, r, g)
        assert np.allclose(sh["dQKV"], full["dQKV"][:, cols], rtol=1e-12, atol=1e-12)
        assert np.allclose(sh["dWqkv"], full["dWqkv"][:, cols], rtol=1e-12, atol=1e-12)
        dX += sh["dX"]
        Z += fw["Z"]
    assert np.allclose(dX, full["dX"], rtol=1e-12, atol=1e-12)
    assert np.allclose(Z, fz["Z"], rtol=1e-12, atol=1e-12)
