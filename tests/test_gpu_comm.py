"""GPU parity of the bandwidth kernels against the oracle, bit for bit: the g / f reduction (all-reduce form), the
dim-0 reduce-scatter, the dim-0 gather and the shard packer.  All calls go through the C ABI."""
import numpy as np
import pytest

import oracle as O
import tp_inputs as TI
from parity_utils import dev, empty, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_block_columnparallel_amd as pkg

    return pkg.load()


def _reduce_case(L, t, n, h, dtype, with_bias, seed=0):
    say(f"partial_reduce t={t} n={n} h={h} {dtype} bias={with_bias}")
    parts = TI.partials(seed, t, (n // h, h), dtype)
    bias = TI.tensor(seed, 9, (h,), 1.0, dtype) if with_bias else None
    want = O.reduce_storage(parts, dtype, bias)
    out = empty((n // h, h), dtype)
    L.tp_partial_reduce(n, h, t, dev(parts, dtype), None if bias is None else dev(bias, dtype), out)
    got = host(out)
    assert np.array_equal(got.view(np.uint32) if dtype == "f32" else got,
                          want.view(np.uint32) if dtype == "f32" else want)


@pytest.mark.parametrize("t", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_reduce_bit_exact(L, t, dtype):
    _reduce_case(L, t, 64 * 1000, 64, dtype, with_bias=False)
    _reduce_case(L, t, 96 * 77, 96, dtype, with_bias=True, seed=1)


def test_partial_reduce_ragged_and_unaligned_tail(L):
    # n not a multiple of the 16-byte vector, odd h: the element-wise path covers everything
    _reduce_case(L, 8, 13 * 37, 13, "bf16", with_bias=True)
    _reduce_case(L, 3, 7 * 5, 7, "f32", with_bias=True)
    _reduce_case(L, 8, 8 * 1001 + 0, 8, "bf16", with_bias=False)


def test_partial_reduce_special_values(L):
    # inf, NaN and rounding ties survive the fp32 rank-order sum + one bf16 rounding exactly as specified
    t, n, h = 2, 64, 64
    a = np.zeros((t, n), np.float32)
    a[0, 0], a[1, 0] = np.inf, 1.0
    a[0, 1], a[1, 1] = np.nan, 1.0
    a[0, 2], a[1, 2] = 1.0, 2.0 ** -8 + 2.0 ** -9
    a[0, 3], a[1, 3] = 3.0e38, 3.0e38  # overflows fp32 -> inf
    a[0, 4], a[1, 4] = -np.inf, np.inf  # NaN
    parts = O.f32_to_bf16_bits(a)
    want = O.reduce_storage(parts, "bf16")
    out = empty((n,), "bf16")
    L.tp_partial_reduce(n, h, t, dev(parts, "bf16"), None, out)
    got = host(out)
    nan_w = np.isnan(O.bf16_bits_to_f64(want))
    assert np.array_equal(np.isnan(O.bf16_bits_to_f64(got)), nan_w)
    assert np.array_equal(got[~nan_w], want[~nan_w])


@pytest.mark.parametrize("name", ["mlp_h3072_ffn12288_t8_b8_s1024", "sp_swiglu_h8192_ffn28672_t8_s4096",
                                  "attn_h6144_a64_d96_t8_s4096"])
def test_reduce_scatter_dim0_full_size(L, name):
    w = TI.WORKLOADS[name]
    say(f"reduce_scatter_dim0 {name}")
    parts = TI.partials(0, w.t, (w.s, w.b, w.h), "bf16")
    bias = TI.tensor(0, 9, (w.h,), 1.0, "bf16")
    dims = L.make_dims(s=w.s, b=w.b, h=w.h, t=w.t)
    P = dev(parts, "bf16")
    Bd = dev(bias, "bf16")
    full_want = O.reduce_storage(parts, "bf16", bias)
    out_all = empty((w.t, w.s // w.t, w.b, w.h), "bf16")
    L.tp_reduce_scatter_dim0(dims, -1, P, Bd, out_all)
    assert np.array_equal(host(out_all).reshape(full_want.shape), full_want)
    for r in (0, w.t - 1, 3):
        out = empty((w.s // w.t, w.b, w.h), "bf16")
        L.tp_reduce_scatter_dim0(dims, r, P, Bd, out)
        assert np.array_equal(host(out), O.split_dim0(full_want, w.t, r))


def test_reduce_scatter_full_size_calculator_default(L):
    w = TI.MLP_CALC
    say("reduce_scatter_dim0 h4096 s2048 b8 t8 (1 GiB of partials)")
    parts = TI.partials(0, w.t, (w.s, w.b, w.h), "bf16")
    dims = L.make_dims(s=w.s, b=w.b, h=w.h, t=w.t)
    out = empty((w.s, w.b, w.h), "bf16")
    L.tp_reduce_scatter_dim0(dims, -1, dev(parts, "bf16"), None, out)
    want = O.reduce_storage(parts, "bf16")
    assert np.array_equal(host(out), want)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(16, 2, 64, 2), (4096, 1, 8192, 8), (24, 3, 5, 4)])
def test_gather_dim0_bit_exact(L, dtype, shape):
    s, b, h, t = shape
    say(f"gather_dim0 s={s} b={b} h={h} t={t} {dtype}")
    full = TI.tensor(3, 0, (s, b, h), 1.0, dtype)
    slices = np.stack([O.split_dim0(full, t, r) for r in range(t)])
    out = empty((s, b, h), dtype)
    L.tp_gather_dim0(L.make_dims(s=s, b=b, h=h, t=t), dev(slices, dtype), out)
    assert np.array_equal(host(out).view(np.uint8), O.gather_dim0(list(slices)).view(np.uint8))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shard_packer_bit_exact_all_kinds(L, dtype):
    h, ffn, t, a, d = 48, 96, 4, 8, 6  # d=6: element-wise path for QKV kinds; FC kinds vectorise in bf16
    cases = [
        ("fc1", O.W_FC1, (h, ffn), dict(h=h, ffn=ffn, t=t)),
        ("fc1_gate_up", O.W_FC1_GATE_UP, (h, 2 * ffn), dict(h=h, ffn=ffn, t=t)),
        ("fc2", O.W_FC2, (ffn, h), dict(h=h, ffn=ffn, t=t)),
        ("b_fc1", O.B_FC1, (ffn,), dict(h=h, ffn=ffn, t=t)),
        ("b_fc1_gate_up", O.B_FC1_GATE_UP, (2 * ffn,), dict(h=h, ffn=ffn, t=t)),
        ("qkv", O.W_QKV, (h, 3 * a * d), dict(h=h, a=a, d=d, t=t)),
        ("proj", O.W_PROJ, (a * d, h), dict(h=h, a=a, d=d, t=t)),
        ("b_qkv", O.B_QKV, (3 * a * d,), dict(h=h, a=a, d=d, t=t)),
    ]
    for name, kind, shape, dd in cases:
        full = TI.tensor(5, kind, shape, 1.0, dtype)
        dims = L.make_dims(**dd)
        F = dev(full, dtype)
        for r in range(t):
            want = O.shard_weight(kind, full, t, r, ffn=dd.get("ffn", 0), a=dd.get("a", 0), d=dd.get("d", 0))
            out = empty(want.shape, dtype)
            L.tp_shard_weights(dims, r, name, F, out)
            assert np.array_equal(host(out).view(np.uint8), want.view(np.uint8)), (name, r)


@pytest.mark.parametrize("name", ["mlp_h4096_ffn16384_t8_b8_s2048", "sp_swiglu_h8192_ffn28672_t8_s4096",
                                  "attn_h6144_a64_d96_t8_s4096"])
def test_shard_packer_full_size(L, name):
    w = TI.WORKLOADS[name]
    say(f"shard packer full size {name}")
    if w.kind == "mlp":
        kind, wname = (O.W_FC1_GATE_UP, "fc1_gate_up") if w.act == "swiglu" else (O.W_FC1, "fc1")
        full = TI.tensor(0, 1, (w.h, (2 if w.act == "swiglu" else 1) * w.ffn), 0.02, "bf16")
        dims = L.make_dims(h=w.h, ffn=w.ffn, t=w.t)
    else:
        kind, wname = O.W_QKV, "qkv"
        full = TI.tensor(0, 1, (w.h, 3 * w.a * w.d), 0.02, "bf16")
        dims = L.make_dims(h=w.h, a=w.a, d=w.d, t=w.t)
    F = dev(full, "bf16")
    for r in (0, w.t - 1):
        want = O.shard_weight(kind, full, w.t, r, ffn=w.ffn, a=w.a, d=w.d)
        out = empty(want.shape, "bf16")
        L.tp_shard_weights(dims, r, wname, F, out)
        assert np.array_equal(host(out), want)
