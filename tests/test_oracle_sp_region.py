"""Pins of the oracle's sequence-parallel region ops (LayerNorm, dropout + residual) against closed forms,
invariants, finite differences and boundary cases.  The pages place these per-token ops on each rank's [s/t, b, h]
slice between a reduce-scatter and the next all-gather ("Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" §5
and §6; "Sequence Parallel 与 Context Parallel", SP section); their arithmetic is the plain definition."""
import numpy as np
import pytest

import oracle as O
import tp_inputs as TI


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


def test_layernorm_closed_forms_and_invariances():
    r = np.random.default_rng(1)
    x = r.standard_normal((5, 16)) * 3 + 2
    y, mean, rstd = O.layernorm(x, np.ones(16), np.zeros(16), 1e-5)
    var = x.var(axis=1)
    assert np.allclose(mean, x.mean(axis=1)) and np.allclose(rstd, 1 / np.sqrt(var + 1e-5))
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), var / (var + 1e-5))  # normalized rows: variance var/(var+eps)
    # with eps = 0 the output ignores the row's scale and offset
    y0 = O.layernorm(x, np.ones(16), np.zeros(16), 0.0)[0]
    y1 = O.layernorm(2.5 * x - 7.0, np.ones(16), np.zeros(16), 0.0)[0]
    assert np.allclose(y0, y1)
    # gamma and beta act per column
    g, b = r.standard_normal(16), r.standard_normal(16)
    assert np.allclose(O.layernorm(x, g, b, 1e-5)[0], y * g + b)


def test_layernorm_backward_by_finite_differences():
    r = np.random.default_rng(2)
    x, dy = r.standard_normal((4, 6)), r.standard_normal((4, 6))
    g, b = r.standard_normal(6), r.standard_normal(6)
    eps = 1e-3
    dx, dg, db = O.layernorm_backward(x, g, dy, eps)

    def loss():
        return float((O.layernorm(x, g, b, eps)[0] * dy).sum())

    assert np.allclose(dx, _fd(loss, x), rtol=1e-6, atol=1e-8)
    assert np.allclose(dg, _fd(loss, g), rtol=1e-6, atol=1e-8)
    assert np.allclose(db, _fd(loss, b), rtol=1e-6, atol=1e-8)
    # shift invariance of the output makes each row of dx sum to zero
    assert np.allclose(dx.sum(axis=1), 0, atol=1e-12)


def test_dropout_boundaries_and_rate():
    p = 0.1
    thr = int(np.floor(p * 2 ** 32))
    bits = np.array([0, thr - 1, thr, 2 ** 32 - 1], dtype=np.uint32)
    assert list(O.dropout_keep(bits, p)) == [False, False, True, True]
    z, res = np.array([1.0, 2.0, 3.0, 4.0]), np.array([10.0, 20.0, 30.0, 40.0])
    assert np.allclose(O.dropout_add(z, res, bits, p), [10.0, 20.0, 30.0 + 3.0 / 0.9, 40.0 + 4.0 / 0.9])
    assert np.array_equal(O.dropout_add(z, res, bits, 0.0), z + res)  # p = 0 keeps everything, scale 1
    words = TI.random_words(0, TI.T_BITS, (1 << 20,))
    kept = O.dropout_keep(words, p).mean()
    assert abs(kept - (1 - p)) < 5 * np.sqrt(p * (1 - p) / words.size)


def test_dropout_backward_is_the_linear_map():
    r = np.random.default_rng(3)
    p = 0.25
    bits = TI.random_words(1, TI.T_BITS, (3, 5))
    z, res, dout = r.standard_normal((3, 5)), r.standard_normal((3, 5)), r.standard_normal((3, 5))
    dz, dres = O.dropout_add_backward(dout, bits, p)

    def loss():
        return float((O.dropout_add(z, res, bits, p) * dout).sum())

    assert np.allclose(dz, _fd(loss, z), rtol=1e-6, atol=1e-8)
    assert np.allclose(dres, _fd(loss, res), rtol=1e-6, atol=1e-8)


def test_ln_fold_identity_and_its_ingredients():
    """The folded form rstd (u A' - mean c) + b equals LayerNorm(u) A + a (exact chain); a dropped beta term, a
    wrong sign on the mean term or gamma left out of A' breaks it (checked by planting each); with A' kept in
    bf16 the identity holds for the kept A' exactly, and against the unrounded A to within its rounding."""
    rng = np.random.default_rng(41)
    rows, h, n = 7, 16, 10
    u = rng.standard_normal((rows, h)) * 1.5 + 0.7     # a non-zero mean, so the mean term matters
    g, be = 1 + 0.1 * rng.standard_normal(h), 0.1 * rng.standard_normal(h)
    A, a = rng.standard_normal((h, n)) * 0.3, rng.standard_normal(n) * 0.02
    y, mean, rstd = O.layernorm(u, g, be, 1e-5)
    ref = y @ A + a
    Af, c, b = O.ln_fold(g, be, A, a)
    assert np.allclose(O.ln_folded_linear(u, mean, rstd, Af, c, b), ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(c, (g[:, None] * A).sum(axis=0), rtol=1e-14) and np.allclose(b, be @ A + a, rtol=1e-14)
    # planted mistakes
    assert not np.allclose(O.ln_folded_linear(u, mean, rstd, Af, c, b - be @ A), ref, atol=1e-6)
    assert not np.allclose(O.ln_folded_linear(u, -mean, rstd, Af, c, b), ref, atol=1e-6)
    assert not np.allclose(O.ln_folded_linear(u, mean, rstd, A, A.sum(axis=0), b), ref, atol=1e-6)
    # bf16-kept A': exact identity for the kept weight, close to the exact chain
    As, cs, bs = O.ln_fold(g, be, A, a, store="bf16")
    assert np.array_equal(As, O.stored(g[:, None] * A, "bf16"))
    assert np.allclose(O.ln_folded_linear(u, mean, rstd, As, cs, bs), ((u - mean[:, None]) * rstd[:, None]) @ As + bs,
                       rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(O.ln_folded_linear(u, mean, rstd, As, cs, bs) - ref)) < 2e-2 * np.sqrt(np.mean(ref ** 2))
