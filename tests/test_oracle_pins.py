"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a wrong rounding rule) fails at least one of them.  None of these tests touches the HIP library.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")
MIB = float(1 << 20)


def golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


# ------------------------------------------------------------------------------------------------- number formats


def _f32_to_fraction(v: np.float32) -> Fraction:
    return Fraction(float(v))  # float32 -> float64 is exact


def _round_fraction(fr: Fraction, mant_bits: int) -> Fraction:
    """Round a rational to the nearest binary float with `mant_bits` significant bits (ties to even), unbounded
    exponent.  Written from the definition of round-to-nearest-even; independent of the oracle's bit tricks."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x7F80, 0x3E80], dtype=np.uint16)
    want = [1.0, -1.0, 2.0, 0.0, -0.0, math.inf, 0.25]
    got = O.bf16_bits_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w


def test_bf16_rounding_special_cases():
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,            # exactly half an ulp above 1.0: tie, 1.0 is even -> stays
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # tie between 0x3F81 (odd) and 0x3F82 (even) -> up
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,  # just above the tie -> up
        -(1.0 + 3 * 2.0 ** -8): 0xBF82,
        float(np.finfo(np.float32).max): 0x7F80,  # carries into the exponent: infinity
        math.inf: 0x7F80,
        -math.inf: 0xFF80,
    }
    for v, want in cases.items():
        got = int(O.f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])
        assert got == want, (v, hex(got), hex(want))
    nan_in = np.array([0x7F800001, 0xFFC00000, 0x7FFFFFFF], dtype=np.uint32).view(np.float32)
    out = O.f32_to_bf16_bits(nan_in)
    assert np.all(np.isnan(O.bf16_bits_to_f64(out)))
    assert (int(out[1]) & 0x8000) != 0  # sign kept


def test_bf16_rounding_matches_exact_rational_rounding():
    rng = np.random.default_rng(11)
    vals = rng.standard_normal(3000).astype(np.float32) * np.float32(100.0)
    # force many exact ties: low 16 bits = 0x8000
    u = vals.view(np.uint32).copy()
    u[:500] = (u[:500] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    vals = u.view(np.float32)
    got = O.bf16_bits_to_f64(O.f32_to_bf16_bits(vals))
    for v, g in zip(vals, got):
        want = _round_fraction(_f32_to_fraction(v), 8)
        assert Fraction(float(g)) == want, (v, g, float(want))


def test_bf16_rounding_matches_torch_library_conversion():
    import torch

    rng = np.random.default_rng(5)
    vals = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    lib = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(vals), lib)


def test_rank_order_fp32_reduction_matches_exact_rounding_per_step():
    rng = np.random.default_rng(3)
    t = 8
    parts = [(rng.standard_normal(200) * (10.0 ** rng.integers(-3, 4, 200))).astype(np.float32) for _ in range(t)]
    bias = rng.standard_normal(200).astype(np.float32)
    got = O.reduce_f32_rank_order(parts, bias)
    for j in range(200):
        acc = _f32_to_fraction(parts[0][j])
        for i in range(1, t):
            acc = _round_fraction(acc + _f32_to_fraction(parts[i][j]), 24)
        acc = _round_fraction(acc + _f32_to_fraction(bias[j]), 24)
        assert Fraction(float(got[j])) == acc


def test_rank_order_is_observable():
    # 2^24 + 1 - 2^24: summing in rank order loses the 1 (fp32 has 24 significant bits); another order would not.
    p = [np.array([2.0 ** 24], np.float32), np.array([1.0], np.float32), np.array([-(2.0 ** 24)], np.float32)]
    assert O.reduce_f32_rank_order(p)[0] == 0.0
    assert O.reduce_f32_rank_order([p[0], p[2], p[1]])[0] == 1.0


def test_reduce_storage_bf16_single_rounding():
    # two partials whose fp32 sum is an exact bf16 tie: rounding each partial first would give another answer
    pa = O.f32_to_bf16_bits(np.array([1.0], np.float32))
    pb = O.f32_to_bf16_bits(np.array([2.0 ** -8 + 2.0 ** -9], np.float32))  # 0.005859375, exact in bf16
    out = O.reduce_storage(np.stack([pa, pb]), "bf16")
    # 1 + 2^-8 + 2^-9 = 1.005859375: low bits above half of a bf16 ulp (2^-7) -> rounds up to 1 + 2^-7
    assert O.bf16_bits_to_f64(out)[0] == 1.0 + 2.0 ** -7


# -------------------------------------------------------------------------------------------------- activations


def test_gelu_against_math_erf_and_tanh():
    xs = np.linspace(-8, 8, 2001)
    ref = np.array([0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0))) for x in xs])
    assert np.max(np.abs(O.gelu(xs) - ref)) < 1e-15
    reft = np.array([0.5 * x * (1.0 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3))) for x in xs])
    assert np.max(np.abs(O.gelu_tanh(xs) - reft)) < 1e-14
    # the two forms differ a little (so a swap of variant is detectable)
    assert np.max(np.abs(O.gelu(xs) - O.gelu_tanh(xs))) > 1e-4


@pytest.mark.parametrize("f,df", [(O.gelu, O.gelu_grad), (O.gelu_tanh, O.gelu_tanh_grad), (O.silu, O.silu_grad)])
def test_activation_derivatives_by_central_differences(f, df):
    xs = np.linspace(-6, 6, 241) + 0.013
    h = 1e-5
    fd = (f(xs + h) - f(xs - h)) / (2 * h)
    assert np.max(np.abs(df(xs) - fd)) < 1e-8


def test_silu_closed_form_values():
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(O.silu_grad(0.0) - 0.5) < 1e-16


def test_nonlinearity_is_not_additive_relu_counterexample():
    g = golden()["relu_counterexample"]
    z0, z1 = g["z0"], g["z1"]
    assert O.relu(z0) + O.relu(z1) == g["sum_of_activations"]
    assert O.relu(z0 + z1) == g["activation_of_sum"]


def test_gelu_of_partial_sums_differs_from_sum_of_gelus():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((8, 4))
    A = rng.standard_normal((4, 6))
    p = O.row_parallel_linear(X, A, 2)
    lhs = O.gelu(p[0] + p[1])
    rhs = O.gelu(p[0]) + O.gelu(p[1])
    assert np.max(np.abs(lhs - rhs)) > 0.1


# ------------------------------------------------------------------------------------- worked split example


def brute_matmul(A, B):
    n, k = A.shape
    k2, m = B.shape
    assert k == k2
    C = np.zeros((n, m))
    for i in range(n):
        for j in range(m):
            s = 0.0
            for p in range(k):
                s += A[i, p] * B[p, j]
            C[i, j] = s
    return C


@pytest.mark.parametrize("Bsz", [1, 3, 5])
def test_worked_example_column_concat_and_row_sum(Bsz):
    g = golden()["worked_split_shapes"]
    rng = np.random.default_rng(Bsz)
    X = rng.standard_normal((Bsz, g["in_features"]))
    W = rng.standard_normal((g["in_features"], g["out_features"]))
    full = brute_matmul(X, W)
    cols = O.column_parallel_linear(X, W, g["t"])
    assert [c.shape for c in cols] == [(Bsz, g["column_shard_shape"][1])] * 2
    assert np.allclose(np.concatenate(cols, axis=1), full, rtol=0, atol=1e-13)
    rows = O.row_parallel_linear(X, W, g["t"])
    assert all(r.shape == full.shape for r in rows)
    assert np.allclose(rows[0] + rows[1], full, rtol=0, atol=1e-13)
    # each row partial is X_i W_i with X_i the matching 2 input columns and W_i the matching 2 rows of W
    assert np.allclose(rows[0], brute_matmul(X[:, :2], W[:2, :]), atol=1e-13)


def test_column_input_grad_is_sum_over_branches_scalar_closed_form():
    # y_k = x w_k (one output column per device), L = y1 y2: dL/dy = [y2, y1]; dL/dx = 2 x w1 w2
    for x, w1, w2 in [(0.7, -1.3, 2.1), (-2.0, 0.5, 0.25), (3.0, 3.0, -1.0)]:
        X = np.array([[x]])
        W = np.array([[w1, w2]])
        y = O.column_parallel_linear(X, W, 2)
        dY = [y[1].copy(), y[0].copy()]
        dX = O.column_parallel_input_grad(dY, W, 2)
        assert abs(dX[0, 0] - 2 * x * w1 * w2) < 1e-14


def test_row_input_grads_are_separate_and_weight_grads_local():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((3, 4))
    W = rng.standard_normal((4, 8))
    dY = rng.standard_normal((3, 8))
    parts = O.row_parallel_input_grads(dY, W, 2)
    assert np.allclose(np.concatenate(parts, axis=1), brute_matmul(dY, W.T), atol=1e-13)
    dYs = [dY[:, :4], dY[:, 4:]]
    dWs = O.column_parallel_weight_grads(X, dYs)
    assert np.allclose(np.concatenate(dWs, axis=1), brute_matmul(X.T, dY), atol=1e-13)
    assert np.allclose(O.column_parallel_input_grad(dYs, W, 2), brute_matmul(dY, W.T), atol=1e-13)


# ---------------------------------------------------------------------------------------------------- MLP block


def _loss(X, A, B, dZ, act, a=None, c=None):
    return float(np.sum(O.mlp_forward(X, A, B, act, a, c)["Z"] * dZ))


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "swiglu", "relu"])
def test_mlp_backward_by_finite_differences(act):
    rng = np.random.default_rng(42)
    M, h, f = 6, 5, 8
    wa = 2 * f if act == "swiglu" else f
    X = rng.standard_normal((M, h))
    A = rng.standard_normal((h, wa)) * 0.7
    B = rng.standard_normal((f, h)) * 0.7
    a = rng.standard_normal(wa) * 0.3
    c = rng.standard_normal(h) * 0.3
    dZ = rng.standard_normal((M, h))
    fw = O.mlp_forward(X, A, B, act, a, c)
    g = O.mlp_backward(X, A, B, fw["U"], fw["Y"], dZ, act)
    eps = 1e-6
    for name, arr, grad in [("X", X, g["dX"]), ("A", A, g["dA"]), ("B", B, g["dB"]), ("a", a, g["da"]),
                            ("c", c, g["dc"])]:
        for idx in [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(6)]:
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(X, A, B, dZ, act, a, c)
            arr[idx] = old - eps
            lm = _loss(X, A, B, dZ, act, a, c)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (act, name, idx, fd, grad[idx])


def test_mlp_forward_against_brute_force():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((3, 4))
    A = rng.standard_normal((4, 8))
    B = rng.standard_normal((8, 4))
    U = brute_matmul(X, A)
    Y = np.vectorize(lambda u: 0.5 * u * (1 + math.erf(u / math.sqrt(2))))(U)
    Z = brute_matmul(Y, B)
    fw = O.mlp_forward(X, A, B, "gelu")
    assert np.allclose(fw["Z"], Z, atol=1e-12)


@pytest.mark.parametrize("act,t", [("gelu", 2), ("gelu", 4), ("swiglu", 2), ("gelu_tanh", 4), ("relu", 2)])
def test_shards_sum_to_unsharded_block(act, t):
    rng = np.random.default_rng(9)
    M, h, f = 10, 6, 16
    wa = 2 * f if act == "swiglu" else f
    X = rng.standard_normal((M, h))
    A = rng.standard_normal((h, wa)) * 0.5
    B = rng.standard_normal((f, h)) * 0.5
    a = rng.standard_normal(wa) * 0.1
    c = rng.standard_normal(h) * 0.1
    dZ = rng.standard_normal((M, h))
    full = O.mlp_forward(X, A, B, act, a, c)
    bw = O.mlp_backward(X, A, B, full["U"], full["Y"], dZ, act)
    zs, dxs = [], []
    for r in range(t):
        fw = O.mlp_shard_forward(X, A, B, t, r, act, a)
        sb = O.mlp_shard_backward(X, A, B, dZ, t, r, act, a)
        zs.append(fw["Z"])
        dxs.append(sb["dX"])
        cols = O.mlp_shard_columns(f, t, r, act)
        # shard-local gradients are slices of the unsharded ones (no communication needed for dW)
        assert np.allclose(sb["dA"], bw["dA"][:, cols], atol=1e-12)
        assert np.allclose(sb["da"], bw["da"][cols], atol=1e-12)
        w = f // t
        assert np.allclose(sb["dB"], bw["dB"][r * w:(r + 1) * w], atol=1e-12)
    assert np.allclose(O.allreduce_sum(zs, c), full["Z"], atol=1e-12)
    assert np.allclose(O.allreduce_sum(dxs), bw["dX"], atol=1e-12)


# ------------------------------------------------------------------------------------------------- shard layout


def _coded(rows, cols):
    """A matrix whose entry encodes its own (row, col) so that selections can be checked by decoding."""
    return (np.arange(rows)[:, None] * 100000 + np.arange(cols)[None, :]).astype(np.int64)


def test_shard_layouts_by_decoding_indices():
    h, ffn, t = 6, 12, 3
    fc1 = _coded(h, ffn)
    for r in range(t):
        sh = O.shard_weight(O.W_FC1, fc1, t, r)
        assert sh.shape == (h, ffn // t)
        assert np.all(sh % 100000 == np.arange(r * 4, r * 4 + 4)[None, :])
        gu = O.shard_weight(O.W_FC1_GATE_UP, _coded(h, 2 * ffn), t, r)
        cols = gu[0] % 100000
        assert list(cols) == list(range(r * 4, r * 4 + 4)) + list(range(ffn + r * 4, ffn + r * 4 + 4))
        fc2 = O.shard_weight(O.W_FC2, _coded(ffn, h), t, r)
        assert list(fc2[:, 0] // 100000) == list(range(r * 4, r * 4 + 4))


def test_qkv_grouping_by_decoding_indices():
    h, a, d, t = 4, 4, 3, 2
    ad = a * d
    W = _coded(h, 3 * ad)
    for r in range(t):
        sh = O.shard_weight(O.W_QKV, W, t, r, a=a, d=d)
        assert sh.shape == (h, (a // t) * 3 * d)
        cols = list(sh[0] % 100000)
        expect = []
        for jj in range(a // t):
            j = r * (a // t) + jj
            expect += [j * d + e for e in range(d)]           # q_j
            expect += [ad + j * d + e for e in range(d)]      # k_j
            expect += [2 * ad + j * d + e for e in range(d)]  # v_j
        assert cols == expect
        proj = O.shard_weight(O.W_PROJ, _coded(ad, h), t, r, a=a, d=d)
        assert list(proj[:, 0] // 100000) == list(range(r * (a // t) * d, (r + 1) * (a // t) * d))


def test_divisibility_rules():
    x = np.zeros((10, 2, 4))
    with pytest.raises(ValueError):
        O.split_dim0(x, 4, 0)
    with pytest.raises(ValueError):
        O.shard_weight(O.W_FC1, np.zeros((4, 10)), 4, 0)
    with pytest.raises(ValueError):
        O.local_head_ids(6, 4, 0)


def test_split_gather_round_trip_and_reduce_scatter():
    rng = np.random.default_rng(2)
    s, b, h, t = 8, 2, 3, 4
    full = rng.standard_normal((s, b, h))
    sl = [O.split_dim0(full, t, r) for r in range(t)]
    assert all(x.shape == (s // t, b, h) for x in sl)
    assert np.array_equal(O.gather_dim0(sl), full)
    parts = [rng.standard_normal((s, b, h)) for _ in range(t)]
    total = parts[0] + parts[1] + parts[2] + parts[3]
    for r in range(t):
        assert np.allclose(O.reduce_scatter_dim0(parts, t, r), total[r * 2:(r + 1) * 2], atol=1e-14)


# ---------------------------------------------------------------------------------------------------- attention


def test_attention_against_torch_sdpa_fp64():
    import torch

    rng = np.random.default_rng(4)
    s, b, a, d, h = 12, 2, 4, 8, 16
    X = rng.standard_normal((s * b, h))
    Wqkv = rng.standard_normal((h, 3 * a * d)) * 0.3
    Wo = rng.standard_normal((a * d, h)) * 0.3
    for causal in (True, False):
        out = O.attention_forward(X, Wqkv, Wo, s, b, a, d, causal)
        QKV = torch.from_numpy(X @ Wqkv).reshape(s, b, 3, a, d)
        q = QKV[:, :, 0].permute(1, 2, 0, 3)
        k = QKV[:, :, 1].permute(1, 2, 0, 3)
        v = QKV[:, :, 2].permute(1, 2, 0, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)  # [b, a, s, d]
        ref = ref.permute(2, 0, 1, 3).reshape(s * b, a * d).numpy()
        assert np.allclose(out["O"], ref, atol=1e-12)
        assert np.allclose(out["Z"], ref @ Wo, atol=1e-11)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    s, d = 7, 4
    K = rng.standard_normal((s, d))
    V = rng.standard_normal((s, d))
    Q = rng.standard_normal((s, d))
    Oc, lse = O.attention_core(Q, K, V, causal=True)
    assert np.allclose(Oc[0], V[0], atol=1e-15)          # the first query sees only the first key
    assert abs(lse[0] - float(Q[0] @ K[0]) / 2.0) < 1e-14  # lse of one visible score is the score (1/sqrt(4))
    Oz, lz = O.attention_core(np.zeros((s, d)), K, V, causal=True)
    for q in range(s):                                   # zero query: uniform weights over the visible keys
        assert np.allclose(Oz[q], V[:q + 1].mean(axis=0), atol=1e-14)
        assert abs(lz[q] - math.log(q + 1)) < 1e-14


def test_attention_shards_sum_to_unsharded_and_rows_sample_exactly():
    rng = np.random.default_rng(6)
    s, b, a, d, t = 9, 2, 4, 3, 2
    h = a * d
    X = rng.standard_normal((s * b, h))
    Wqkv = rng.standard_normal((h, 3 * a * d)) * 0.4
    Wo = rng.standard_normal((a * d, h)) * 0.4
    bq = rng.standard_normal(3 * a * d) * 0.1
    full = O.attention_forward(X, Wqkv, Wo, s, b, a, d, True, bq)
    zs = []
    for r in range(t):
        sh = O.attention_shard_forward(X, Wqkv, Wo, s, b, a, d, t, r, True, bq)
        heads = O.local_head_ids(a, t, r)
        for jj, j in enumerate(heads):
            assert np.allclose(sh["O"][:, jj * d:(jj + 1) * d], full["O"][:, j * d:(j + 1) * d], atol=1e-13)
            assert np.allclose(sh["lse"][:, jj], full["lse"][:, j], atol=1e-13)
        rows = [0, 5, 17, 8]
        part = O.attention_rows(sh["QKV"], s, b, len(heads), d, rows, True)
        assert np.allclose(part["O"], sh["O"][rows], atol=1e-13)
        assert np.allclose(part["lse"], np.stack([sh["lse"][r_ % b, :, r_ // b] for r_ in rows]), atol=1e-13)
        zs.append(sh["Z"])
    assert np.allclose(O.allreduce_sum(zs), full["Z"], atol=1e-12)


# --------------------------------------------------------------------------------------------------- accounting


@pytest.mark.parametrize("key", ["calculator_default", "calculator_8p3b_width"])
def test_calculator_numbers(key):
    g = golden()[key]
    h, f, t, b, s, e = g["h"], g["f"], g["t"], g["b"], g["s"], g["elem_bytes"]
    p = O.linear_params_per_rank(h, f, t)
    assert p == g["params_per_rank_per_layer"]
    assert p * e / MIB == g["weights_mib"]
    n = O.allreduce_payload_elems(b, s, h)
    assert n * e / MIB == g["allreduce_mib"]
    assert O.allreduce_calls_per_layer() * n * e / MIB == g["allreduce_per_layer_mib"]
    assert O.ring_elems_per_card_per_layer(b, s, h, t) * e / MIB == g["ring_per_card_mib"]


def test_llama70b_activation_sizes():
    g = golden()["llama70b_activation"]
    n = O.allreduce_payload_elems(g["b"], g["s"], g["h"])
    assert n * g["elem_bytes"] / MIB == g["activation_mib_per_card_no_sp"]
    sl = O.split_dim0(np.zeros((g["s"], 1, 1)), g["t"], 0).shape[0]
    assert sl * g["b"] * g["h"] * g["elem_bytes"] / MIB == g["activation_mib_per_card_sp"]


@pytest.mark.parametrize("act", ["gelu", "swiglu", "relu"])
def test_sampled_mlp_helpers_match_full_oracle(act):
    rng = np.random.default_rng(12)
    M, h, f, t = 14, 6, 16, 4
    wa = 2 * f if act == "swiglu" else f
    X = rng.standard_normal((M, h))
    A = rng.standard_normal((h, wa)) * 0.5
    B = rng.standard_normal((f, h)) * 0.5
    a = rng.standard_normal(wa) * 0.1
    dZ = rng.standard_normal((M, h))
    rows = [0, 3, 13, 7]
    for r in range(t):
        fw = O.mlp_shard_forward(X, A, B, t, r, act, a)
        bw = O.mlp_shard_backward(X, A, B, dZ, t, r, act, a)
        sr = O.mlp_shard_rows(X[rows], dZ[rows], A, B, t, r, act, a)
        for k in ("U", "Y", "Z"):
            assert np.allclose(sr[k], fw[k][rows], atol=1e-13)
        for k in ("dU", "dX"):
            assert np.allclose(sr[k], bw[k][rows], atol=1e-13)
        js = [0, 2, 3]
        wc = O.mlp_shard_weight_grad_cols(X, dZ, A, B, t, r, js, act, a)
        assert np.allclose(wc["dB_rows"], bw["dB"][js], atol=1e-13)
        assert np.allclose(wc["dA_cols"], bw["dA"][:, wc["sel"]], atol=1e-13)
        assert np.allclose(wc["da_cols"], bw["da"][wc["sel"]], atol=1e-13)


def test_stored_rounding_is_fp32_then_bf16():
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -9, -3.0, 1e-3])
    got = O.stored(x, "bf16")
    # 1 + 2^-8 + 2^-30: fp32 keeps 1 + 2^-8 (2^-30 is below fp32's half ulp), then the bf16 tie goes to even 1.0
    assert got[0] == 1.0
    assert got[1] == 1.0 and got[2] == -3.0
    assert abs(got[3] - 1e-3) <= 2.0 ** -9 * 1e-3
    assert np.array_equal(O.stored(x, "f32"), x.astype(np.float32).astype(np.float64))
