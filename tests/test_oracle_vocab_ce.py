"""Pins of the oracle's cross entropy and its vocab-parallel form ("Tensor Parallelism (TP) 与 Sequence
Parallelism (SP)" §5, the vocab-parallel CE row: all-reduce(max), all-reduce(sum), local backward).

* the unsharded loss and gradient against torch's fp64 cross_entropy and autograd (an independent library
  routine; a negative target -100 is torch's default ignored index);
* closed forms: equal logits give log V; a target logit far above the rest gives a loss near 0;
* shifting a row by a constant changes nothing; gradient rows sum to 0 and match finite differences;
* the sharded steps equal the unsharded loss for t = 1, 2, 4, with targets in every shard, and stay finite for
  logits of magnitude 1e4 (a plain exp would overflow);
* undefined rows (a target past the vocab, a row of -inf logits) give NaN;
* the vocab-sharded logits X E_r^T against a triple loop, and their backward (dX_r summed over ranks, dE_r
  stacked) against central differences of the whole output-layer loss.
"""
import numpy as np
import pytest

import oracle as O


def _case(seed, rows=9, V=24, scale=3.0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((rows, V)) * scale
    tg = r.integers(0, V, rows)
    tg[2] = -100
    return x, tg


def test_against_torch_fp64():
    torch = pytest.importorskip("torch")
    x, tg = _case(1)
    dl = np.random.default_rng(2).standard_normal(x.shape[0])
    tx = torch.tensor(x, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(tx, torch.tensor(tg), reduction="none")
    (loss * torch.tensor(dl)).sum().backward()
    assert np.allclose(O.cross_entropy(x, tg), loss.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(O.cross_entropy_backward(x, tg, dl), tx.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_closed_forms_and_invariance():
    V = 50
    x = np.full((3, V), 2.5)
    assert np.allclose(O.cross_entropy(x, np.array([0, 7, 49])), np.log(V))
    y = np.zeros((1, V))
    y[0, 3] = 60.0
    assert O.cross_entropy(y, np.array([3]))[0] < 1e-20
    x, tg = _case(3)
    shift = np.random.default_rng(4).standard_normal(x.shape[0])[:, None] * 10
    assert np.allclose(O.cross_entropy(x + shift, tg), O.cross_entropy(x, tg))


def test_backward_finite_differences_and_row_sums():
    x, tg = _case(5, rows=4, V=7)
    dl = np.random.default_rng(6).standard_normal(4)
    g = O.cross_entropy_backward(x, tg, dl)
    fd = np.zeros_like(x)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += 1e-6
            xm[i, j] -= 1e-6
            fd[i, j] = ((O.cross_entropy(xp, tg) - O.cross_entropy(xm, tg)) * dl).sum() / 2e-6
    assert np.allclose(g, fd, rtol=1e-6, atol=1e-8)
    assert np.allclose(g.sum(axis=1), 0.0, atol=1e-12)


@pytest.mark.parametrize("t", [1, 2, 4])
def test_vocab_parallel_equals_unsharded(t):
    x, tg = _case(7, rows=12, V=32)
    tg[:4] = [0, 31, 8 * 1 + 3, 16]  # targets in the first, last and middle shards
    tg[5] = -100
    shards = [x[:, r * 32 // t:(r + 1) * 32 // t] for r in range(t)]
    loss, lse = O.vocab_parallel_cross_entropy(shards, tg)
    assert np.allclose(loss, O.cross_entropy(x, tg), rtol=1e-12, atol=1e-12)
    m = x.max(axis=1)
    assert np.allclose(lse, m + np.log(np.exp(x - m[:, None]).sum(axis=1)))
    dl = np.random.default_rng(8).standard_normal(12)
    g = np.concatenate([O.vocab_parallel_cross_entropy_backward(shards[r], tg, r, lse, dl) for r in range(t)], axis=1)
    assert np.allclose(g, O.cross_entropy_backward(x, tg, dl), rtol=1e-12, atol=1e-12)
    assert loss[5] == 0.0 and np.all(g[5] == 0.0)


def test_large_logits_stay_finite():
    x, tg = _case(9, rows=5, V=16, scale=1e4)
    loss, lse = O.vocab_parallel_cross_entropy([x[:, :8], x[:, 8:]], tg)
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(lse))
    assert np.allclose(loss, O.cross_entropy(x, tg))


@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")
def test_undefined_rows_are_nan_not_a_number_that_passes():
    """A target past the vocab (no such logit) and a row of -inf logits have no defined loss: both give NaN, in the
    unsharded definition and in the sharded steps; ignored rows stay 0; the other rows are unaffected."""
    x, tg = _case(11, rows=6, V=16)
    x[2, :] = -np.inf            # every logit of row 2 is -inf
    tg[[0, 2, 3, 5]] = [0, 3, 9, 15]
    tg[1] = 16                   # past the vocab: no rank of t = 2 (8 columns each) owns it
    tg[4] = -100                 # ignored
    loss = O.cross_entropy(x, tg)
    assert np.isnan(loss[1]) and np.isnan(loss[2]) and loss[4] == 0.0
    ok = [0, 3, 5]
    m = x[ok].max(axis=1)
    ref = m + np.log(np.exp(x[ok] - m[:, None]).sum(axis=1)) - x[ok, tg[ok]]
    assert np.allclose(loss[ok], ref, rtol=1e-14)
    lv, lse = O.vocab_parallel_cross_entropy([x[:, :8], x[:, 8:]], tg)
    assert np.isnan(lv[1]) and np.isnan(lse[1])          # the backward's exp(x - lse) turns NaN too
    assert np.isnan(lv[2]) and np.isneginf(lse[2])
    assert lv[4] == 0.0 and np.allclose(lv[ok], loss[ok], rtol=1e-12)
    g = O.vocab_parallel_cross_entropy_backward(x[:, :8], tg, 0, lse, np.ones(6))
    assert np.all(np.isnan(g[1])) and np.all(g[4] == 0.0)


def test_vocab_parallel_logits_brute_force_and_concat():
    """Rank r's logits are columns [r V/t, (r+1) V/t) of X E^T: against a triple loop on a tiny case, and the t
    shards concatenated give the unsharded logits."""
    rng = np.random.default_rng(21)
    rows, h, V, t = 3, 5, 8, 2
    X, E = rng.standard_normal((rows, h)), rng.standard_normal((V, h))
    full = np.zeros((rows, V))
    for i in range(rows):
        for j in range(V):
            for k in range(h):
                full[i, j] += X[i, k] * E[j, k]
    shards = [O.vocab_parallel_logits(X, E, t, r) for r in range(t)]
    assert np.allclose(np.concatenate(shards, axis=1), full, rtol=1e-14, atol=1e-14)
    assert np.allclose(shards[1], full[:, 4:], rtol=1e-14, atol=1e-14)
    with pytest.raises(ValueError):
        O.vocab_parallel_logits(X, E[:7], 2, 0)


def test_vocab_parallel_logits_backward_by_finite_differences():
    """The loss sum_i dloss_i CE(X E^T)_i: its gradients by central differences equal the sum over ranks of dX_r
    and the stacked dE_r, with dlogits the cross entropy's own backward (the whole output-layer chain)."""
    rng = np.random.default_rng(22)
    rows, h, V, t = 4, 6, 12, 3
    X, E = rng.standard_normal((rows, h)), rng.standard_normal((V, h)) * 0.5
    tg = rng.integers(0, V, rows)
    tg[1] = -100
    dl = rng.standard_normal(rows)

    def loss(Xv, Ev):
        return float((O.cross_entropy(Xv @ Ev.T, tg) * dl).sum())

    shards = [O.vocab_parallel_logits(X, E, t, r) for r in range(t)]
    _, lse = O.vocab_parallel_cross_entropy(shards, tg)
    dX = np.zeros_like(X)
    dE = []
    for r in range(t):
        g = O.vocab_parallel_cross_entropy_backward(shards[r], tg, r, lse, dl)
        b = O.vocab_parallel_logits_backward(X, E, g, t, r)
        dX += b["dX"]
        dE.append(b["dE"])
    dE = np.concatenate(dE, axis=0)
    eps = 1e-6
    for M, G in ((X, dX), (E, dE)):
        fd = np.zeros_like(M)
        for idx in np.ndindex(M.shape):
            keep = M[idx]
            M[idx] = keep + eps
            lp = loss(X, E)
            M[idx] = keep - eps
            lm = loss(X, E)
            M[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        assert np.allclose(G, fd, rtol=1e-6, atol=1e-8)
    # a mistake in the backward's operands shows: dE from X^T dlogits (transposed) has the wrong shape / values
    assert not np.allclose(dX, dlogits_all(shards, tg, lse, dl, t) @ E[::-1])


def dlogits_all(shards, tg, lse, dl, t):
    return np.concatenate([O.vocab_parallel_cross_entropy_backward(shards[r], tg, r, lse, dl) for r in range(t)],
                          axis=1)
