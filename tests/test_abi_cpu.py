"""The C ABI on the CPU: the library loads, exports every function include/tpshard.h declares, and every invalid
argument is rejected with its documented status before any HIP call (so none of these calls touches a GPU).

Pointers here are fake, well-aligned addresses: validation never dereferences them, and every case below fails
validation, so nothing is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")


@pytest.fixture(scope="module")
def L():
    import attention_block_columnparallel_amd as pkg

    return pkg.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(tp_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ["tp_shard_weights", "tp_mlp_fwd", "tp_mlp_bwd", "tp_mlp_bwd_phase", "tp_attn_fwd", "tp_attn_bwd",
              "tp_attn_bwd_workspace", "tp_partial_reduce",
              "tp_reduce_scatter_dim0", "tp_gather_dim0", "tp_sp_dropout_add_ln_fwd", "tp_sp_dropout_add_ln_bwd",
              "tp_sp_ln_bwd_workspace", "tp_vocab_ce_fwd_local", "tp_vocab_ce_combine", "tp_vocab_ce_bwd",
              "tp_status_str"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(L.LIB_PATH)
    for n in declared_functions():
        assert hasattr(raw, n), n
    assert set(L.EXPORTED) == set(declared_functions())


def test_abi_version_and_status_strings(L):
    assert L.lib.tp_abi_version() == 2
    for code in range(0, -9, -1):
        s = L.status_str(code)
        assert isinstance(s, str) and s and s != "unknown status"
    assert L.status_str(-99) == "unknown status"


A = 0x100000  # fake 16-byte-aligned addresses, far apart (no overlap)


def addr(i):
    return A * (i + 1)


def mlp_args(L, **over):
    d = dict(s=16, b=2, h=64, ffn=256, t=2)
    d.update({k: v for k, v in over.items() if k in d})
    dims = L.make_dims(**d)
    return dims


BF16, F32 = 1, 0


def test_mlp_fwd_validation(L):
    dims = mlp_args(L)
    P = [addr(i) for i in range(7)]
    call = lambda dims, rank=0, act=0, dt=BF16, p=P: L.tp_mlp_fwd(dims, rank, act, p[0], p[1], p[2], p[3], p[4],
                                                                  p[5], p[6], stream=0, dtype=dt, check=False)
    assert L.lib.tp_mlp_fwd(None, 0, 0, BF16, *P, None) == -1
    assert call(dims, p=[None] + P[1:]) == -1                       # X NULL
    assert call(dims, rank=2, p=P[:2] + [None] + P[3:]) == -5       # a NULL bias is allowed: the rank check decides
    assert call(mlp_args(L, s=0)) == -2
    assert call(mlp_args(L, ffn=255)) == -3                         # ffn % t
    assert call(dims, rank=2) == -5
    assert call(dims, rank=-1) == -5
    assert call(dims, dt=7) == -4
    assert call(dims, act=9) == -7
    assert call(mlp_args(L, h=60)) == -7                            # bf16 rows must be multiples of 8
    assert call(dims, p=[P[0] + 2] + P[1:]) == -7                   # misaligned bf16 pointer
    # Y_i overlapping X
    assert call(dims, p=P[:5] + [P[0] + 64] + P[6:]) == -6
    # two outputs overlapping each other
    assert call(dims, p=P[:4] + [P[4], P[4] + 128, P[6]]) == -6


def test_mlp_bwd_validation(L):
    dims = mlp_args(L)
    P = [addr(i) for i in range(11)]
    call = lambda dims, rank=0, act=0, dt=BF16, p=P: L.tp_mlp_bwd(dims, rank, act, *p, stream=0, dtype=dt, check=False)
    assert call(dims, p=P[:6] + [None] + P[7:]) == -1               # dU workspace required
    assert call(mlp_args(L, ffn=100, t=3)) == -3
    assert call(dims, rank=5) == -5
    assert call(dims, act=-1) == -7
    assert call(dims, p=P[:9] + [P[0]] + P[10:]) == -6              # dB_i aliases X


def test_attn_fwd_validation(L):
    P = [addr(i) for i in range(8)]
    call = lambda dims, rank=0, dt=BF16, p=P: L.tp_attn_fwd(dims, rank, True, *p, stream=0, dtype=dt, check=False)
    ok = dict(s=64, b=1, h=128, a=4, d=32, t=2)
    assert call(L.make_dims(**{**ok, "a": 3})) == -3               # heads % t
    assert call(L.make_dims(**{**ok, "d": 16})) == -3              # h != a*d
    assert call(L.make_dims(**{**ok, "h": 1024, "d": 256})) == -7  # d > 128
    assert call(L.make_dims(**{**ok, "h": 48, "d": 12})) == -7     # bf16 needs d % 8 == 0
    assert call(L.make_dims(**ok), rank=2) == -5
    assert call(L.make_dims(**ok), p=P[:4] + [P[0]] + P[5:]) == -6  # QKV_i aliases X


def test_attn_bwd_validation(L):
    # X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dZ, dO_ws, rec_ws, dQKV_i, dWqkv_i, dbqkv_i, dWo_i, dX_i
    P = [addr(i) for i in range(14)]
    call = lambda dims, rank=0, dt=BF16, p=P: L.tp_attn_bwd(dims, rank, True, *p, stream=0, dtype=dt, check=False)
    ok = dict(s=64, b=1, h=128, a=4, d=32, t=2)
    for i in range(14):
        if i != 11:                                                  # dbqkv_i is nullable
            assert call(L.make_dims(**ok), p=P[:i] + [None] + P[i + 1:]) == -1, i
    assert call(L.make_dims(**{**ok, "s": 0})) == -2
    assert call(L.make_dims(**{**ok, "a": 3})) == -3               # heads % t
    assert call(L.make_dims(**{**ok, "d": 16})) == -3              # h != a*d
    assert call(L.make_dims(**ok), rank=2) == -5
    assert call(L.make_dims(**ok), dt=5) == -4
    assert call(L.make_dims(**{**ok, "h": 1024, "d": 256})) == -7  # d > 128
    assert call(L.make_dims(**{**ok, "h": 48, "d": 12})) == -7     # bf16 needs d % 8 == 0
    assert call(L.make_dims(**ok), p=P[:9] + [P[0]] + P[10:]) == -6  # dQKV_i aliases X
    assert call(L.make_dims(**ok), p=P[:8] + [P[5]] + P[9:]) == -6   # rec_ws aliases lse_i


def test_reduce_and_gather_validation(L):
    P = [addr(i) for i in range(3)]
    assert L.tp_partial_reduce(0, 8, 2, P[0], None, P[1], stream=0, dtype=BF16, check=False) == -2
    assert L.tp_partial_reduce(100, 64, 2, P[0], None, P[1], stream=0, dtype=BF16, check=False) == -2  # n % h
    assert L.tp_partial_reduce(128, 64, 2, None, None, P[1], stream=0, dtype=BF16, check=False) == -1
    assert L.tp_partial_reduce(128, 64, 2, P[0], None, P[0] + 256, stream=0, dtype=BF16, check=False) == -6
    assert L.tp_partial_reduce(128, 64, 2, P[0], None, P[1], stream=0, dtype=3, check=False) == -4
    dims = L.make_dims(s=10, b=2, h=8, t=4)                          # s % t != 0
    assert L.tp_reduce_scatter_dim0(dims, 0, P[0], None, P[1], stream=0, dtype=BF16, check=False) == -3
    assert L.tp_gather_dim0(dims, P[0], P[1], stream=0, dtype=BF16, check=False) == -3
    dims = L.make_dims(s=8, b=2, h=8, t=4)
    assert L.tp_reduce_scatter_dim0(dims, 4, P[0], None, P[1], stream=0, dtype=BF16, check=False) == -5
    assert L.tp_reduce_scatter_dim0(dims, -2, P[0], None, P[1], stream=0, dtype=BF16, check=False) == -5


def test_shard_weights_validation(L):
    P = [addr(i) for i in range(2)]
    dims = L.make_dims(h=64, ffn=256, t=3)
    assert L.tp_shard_weights(dims, 0, "fc1", P[0], P[1], stream=0, dtype=BF16, check=False) == -3
    dims = L.make_dims(h=64, ffn=256, t=2)
    assert L.tp_shard_weights(dims, 2, "fc1", P[0], P[1], stream=0, dtype=BF16, check=False) == -5
    assert L.tp_shard_weights(dims, 0, 99, P[0], P[1], stream=0, dtype=BF16, check=False) == -7
    assert L.tp_shard_weights(dims, 0, "fc1", P[0], P[0] + 64, stream=0, dtype=BF16, check=False) == -6
    dims = L.make_dims(h=96, a=4, d=24, t=8)
    assert L.tp_shard_weights(dims, 0, "qkv", P[0], P[1], stream=0, dtype=BF16, check=False) == -3


def test_python_wrapper_raises_tperror(L):
    with pytest.raises(L.TpError) as ei:
        L.tp_partial_reduce(100, 64, 2, addr(0), None, addr(1), stream=0, dtype=BF16)
    assert "TP_E_SHAPE" in str(ei.value)


def test_sp_region_validation(L):
    P = [addr(i) for i in range(16)]
    rows, h = 16, 64

    def fwd(rows=rows, h=h, p=0.1, eps=1e-5, dt=BF16, ptrs=None):
        q = ptrs or P[:10]  # z, residual, bits, gamma, beta, out, y, mean, rstd, mask
        return L.tp_sp_dropout_add_ln_fwd(rows, h, p, eps, *q, stream=0, dtype=dt, check=False)

    def bwd(rows=rows, h=h, p=0.1, dt=BF16, ptrs=None):
        q = ptrs or P[:12]  # u, gamma, mean, rstd, dy, dres_in, mask, dres, dz, dgamma, dbeta, ws
        return L.tp_sp_dropout_add_ln_bwd(rows, h, p, *q, stream=0, dtype=dt, check=False)

    for i in (0, 3, 4):                                      # z, gamma, beta are required
        assert fwd(ptrs=P[:i] + [None] + P[i + 1:10]) == -1, i
    # y may be left out only when out, mean and rstd are written (the LayerNorm-folded GEMM's input)
    assert fwd(ptrs=P[:5] + [None, None] + P[7:10]) == -1
    assert fwd(ptrs=P[:6] + [None, None] + P[8:10]) == -1
    assert fwd(ptrs=P[:6] + [None] + P[7:8] + [None] + P[9:10]) == -1
    assert fwd(ptrs=P[:5] + [P[0], None] + P[7:10]) == -6    # without y, out over z is still caught
    assert fwd(ptrs=P[:2] + [None] + P[3:10]) == -1          # random words required when p > 0
    # ... not when p == 0: then the misaligned y decides (every case here must fail validation: nothing launches)
    assert fwd(p=0.0, ptrs=P[:2] + [None] + P[3:6] + [P[6] + 2] + P[7:10]) == -7
    assert fwd(rows=0) == -2
    assert fwd(p=1.0) == -2 and fwd(p=-0.1) == -2 and fwd(p=float("nan")) == -2
    assert fwd(eps=-1.0) == -2
    assert fwd(dt=9) == -4
    assert fwd(h=60) == -7                                   # h % 8
    assert fwd(h=12288 + 8) == -7                            # largest supported row
    assert fwd(ptrs=P[:6] + [P[6] + 2] + P[7:10]) == -7      # misaligned y
    assert fwd(ptrs=P[:5] + [P[0]] + P[6:10]) == -6          # out aliases z
    assert fwd(ptrs=P[:9] + [P[7]]) == -6                    # mask overlaps mean
    for i in (0, 1, 2, 3, 4, 9, 10, 11):                     # u, gamma, mean, rstd, dy, dgamma, dbeta, ws required
        assert bwd(ptrs=P[:i] + [None] + P[i + 1:12]) == -1, i
    assert bwd(ptrs=P[:6] + [None] + P[7:12]) == -1          # mask required when p > 0
    assert bwd(rows=-3) == -2
    assert bwd(h=20) == -7
    assert bwd(ptrs=P[:11] + [P[11] + 4]) == -7              # misaligned workspace
    assert bwd(ptrs=P[:8] + [P[4]] + P[9:12]) == -6          # dz aliases dy
    assert bwd(ptrs=P[:11] + [P[9] + 16]) == -6              # workspace overlaps dgamma
    # the no-allocation variant: same checks without the workspace, and sizes beyond its fixed 16 MiB scratch
    # refused (TP_E_SCRATCH) before any HIP call
    def bwd_na(rows=rows, h=h, p=0.1, dt=BF16, ptrs=None):
        q = ptrs or P[:11]
        return L.tp_sp_dropout_add_ln_bwd_noalloc(rows, h, p, *q, stream=0, dtype=dt, check=False)

    for i in (0, 1, 2, 3, 4, 9, 10):
        assert bwd_na(ptrs=P[:i] + [None] + P[i + 1:11]) == -1, i
    assert bwd_na(h=20) == -7
    assert bwd_na(ptrs=P[:8] + [P[4]] + P[9:11]) == -6
    assert bwd_na(rows=512, h=12288) == -9                   # 256 x 2 x 12288 fp32 = 24 MiB
    assert bwd_na(rows=171, h=12288) == -9                   # 171 x 2 x 12288 x 4 B > 16 MiB
    assert bwd_na(rows=171, h=12288, ptrs=P[:8] + [P[4]] + P[9:11]) == -9  # the size check comes first
    assert bwd_na(rows=170, h=12288, ptrs=P[:8] + [P[4]] + P[9:11]) == -6  # 170 rows fit: on to the alias check
    assert L.tp_sp_ln_bwd_workspace(512, 8192) == 16 << 20     # the largest that fits: the SP workload's rows
    assert L.status_str(-9).startswith("the call needs more scratch")
    assert L.tp_sp_ln_bwd_workspace(2048, 4096) == 256 * 2 * 4096 * 4
    assert L.tp_sp_ln_bwd_workspace(3, 64) == 3 * 2 * 64 * 4
    assert L.tp_sp_ln_bwd_workspace(0, 64) == 0


def test_mlp_bwd_phase_validation(L):
    P = [addr(i) for i in range(11)]  # X, A_i, B_i, U_i, Y_i, dZ, dU_ws, dA_i, da_i, dB_i, dX_i
    dims = L.make_dims(s=16, b=2, h=64, ffn=256, t=2)

    def call(phase, p=P, dims=dims, rank=0):
        return L.tp_mlp_bwd_phase(dims, rank, "gelu", phase, *p, stream=0, dtype=BF16, check=False)

    # the dgrad half needs A_i, B_i, U_i, dX_i but not X, Y_i, dA_i, dB_i; the wgrad half the other way round
    assert call("dgrad", [P[0]] + [None] + P[2:]) == -1
    assert call("dgrad", P[:10] + [None]) == -1
    assert call("wgrad", [None] + P[1:]) == -1
    assert call("wgrad", P[:9] + [None, P[10]]) == -1
    assert call("all", P[:4] + [None] + P[5:]) == -1
    assert call(7) == -7                                                  # unknown phase
    assert call("dgrad", dims=L.make_dims(s=16, b=2, h=64, ffn=255, t=2)) == -3
    assert call("wgrad", rank=2) == -5
    # unused operands are not checked: a misaligned X does not matter to the dgrad half, a misaligned dU does
    assert call("dgrad", [P[0] + 2] + P[1:6] + [P[6] + 2] + P[7:]) == -7
    # dU_ws is written by the dgrad half (may not alias an input) and only read by the wgrad half
    assert call("dgrad", P[:6] + [P[5]] + P[7:]) == -6                    # dU_ws aliases dZ
    assert call("wgrad", P[:9] + [P[6]] + P[10:]) == -6                   # dB_i aliases dU_ws (an input here)


def test_timing_filter_arguments(L):
    assert L.lib.tp_timing_filter(b"gemm_bf16_big_pair") == 0
    assert L.lib.tp_timing_filter(b"x" * 64) == -2
    assert L.lib.tp_timing_filter(None) == 0


def test_vocab_ce_validation(L):
    P = [addr(i) for i in range(6)]
    assert L.tp_vocab_ce_fwd_local(16, 64, 0, None, P[1], P[2], stream=0, dtype=BF16, check=False) == -1
    assert L.tp_vocab_ce_fwd_local(0, 64, 0, P[0], P[1], P[2], stream=0, dtype=BF16, check=False) == -2
    assert L.tp_vocab_ce_fwd_local(16, 64, -1, P[0], P[1], P[2], stream=0, dtype=BF16, check=False) == -5
    assert L.tp_vocab_ce_fwd_local(16, 64, 0, P[0], P[1], P[2], stream=0, dtype=4, check=False) == -4
    assert L.tp_vocab_ce_fwd_local(16, 60, 0, P[0], P[1], P[2], stream=0, dtype=BF16, check=False) == -7
    assert L.tp_vocab_ce_fwd_local(16, 64, 0, P[0], P[1], P[2] + 4, stream=0, dtype=BF16, check=False) == -7
    assert L.tp_vocab_ce_fwd_local(16, 64, 0, P[0], P[1], P[0] + 64, stream=0, dtype=BF16, check=False) == -6
    assert L.tp_vocab_ce_fwd_local(1 << 21, 1 << 20, 0, P[0], P[1], P[2], stream=0, dtype=BF16, check=False) == -2
    assert L.tp_vocab_ce_combine(16, 0, P[0], P[1], P[2], P[3], stream=0, check=False) == -2
    assert L.tp_vocab_ce_combine(16, 2, P[0], None, P[2], P[3], stream=0, check=False) == -1
    assert L.tp_vocab_ce_combine(16, 2, P[0] + 8, P[1], P[2], P[3], stream=0, check=False) == -7
    assert L.tp_vocab_ce_combine(16, 2, P[0], P[1], P[2], P[2] + 8, stream=0, check=False) == -6  # lse overlaps loss
    assert L.tp_vocab_ce_bwd(16, 64, 0, P[0], P[1], P[2], None, P[4], stream=0, dtype=BF16, check=False) == -1
    assert L.tp_vocab_ce_bwd(16, 64, 0, P[0], P[1], P[2], P[3], P[0] + 32, stream=0, dtype=BF16, check=False) == -6
    assert L.tp_vocab_ce_bwd(16, 12, 0, P[0], P[1], P[2], P[3], P[4], stream=0, dtype="f32", check=False) == -7


def test_gqa_dims_validation(L):
    P = [addr(i) for i in range(8)]
    ok = dict(s=16, b=2, h=64, a=8, d=8, t=2)

    def fwd(**kw):
        return L.tp_attn_fwd(L.make_dims(**{**ok, **kw}), 0, True, *P[:7], P[7], stream=0, dtype=BF16, check=False)

    assert fwd(g=-2) == -2
    assert fwd(g=3) == -3          # a % g
    assert fwd(g=1) == -3          # g % t: a rank would not own a whole group
    assert fwd(g=4, d=12, h=96) == -7   # valid groups; bf16 d % 8 decides
    dims = L.make_dims(h=64, a=8, d=8, t=4, g=2)
    assert L.tp_shard_weights(dims, 0, "qkv", P[0], P[1], stream=0, dtype=BF16, check=False) == -3
    dims = L.make_dims(h=64, a=8, d=8, t=2, g=4)
    assert L.tp_shard_weights(dims, 2, "b_qkv", P[0], P[1], stream=0, dtype=BF16, check=False) == -5
    bw = L.tp_attn_bwd(L.make_dims(**{**ok, "g": 6}), 0, True, *P, P[0] + 0x800000, P[1] + 0x800000,
                       P[2] + 0x800000, P[3] + 0x800000, P[4] + 0x800000, P[5] + 0x800000, stream=0, dtype=BF16,
                       check=False)
    assert bw == -3


def test_attn_bwd_workspace_size(L):
    # multi-head: the per-block records only; grouped-query: plus a/g partial dK | dV rows per KV head
    assert L.tp_attn_bwd_workspace(L.make_dims(s=100, b=2, h=64, a=8, d=8, t=2)) == 2 * 4 * 2 * 256 * 4
    g = L.make_dims(s=100, b=2, h=64, a=8, d=8, t=2, g=2)
    assert L.tp_attn_bwd_workspace(g) == (2 * 4 * 2 * 256 + 100 * 2 * 1 * 16 * 4) * 4
    assert L.tp_attn_bwd_workspace(L.make_dims(s=100, b=2, h=64, a=8, d=8, t=2, g=3)) == 0


def test_binding_checks_tensor_extents_before_the_call(L):
    """The binding refuses a view that is not contiguous, a buffer shorter than the extent the call works out from
    its sizes, and a tensor that is not on a GPU -- with ValueError, before the library runs (its kernels trust
    the extents)."""
    import torch

    dims = L.make_dims(s=16, b=2, h=64, t=2)
    n = 16 * 2 * 64
    full = torch.zeros(n, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="not contiguous"):
        L.tp_gather_dim0(dims, torch.zeros(64, 2 * n // 64, dtype=torch.bfloat16).t(), addr(1), stream=0)
    with pytest.raises(ValueError, match="the call needs"):
        L.tp_gather_dim0(dims, full[: n - 8], addr(1), stream=0)
    with pytest.raises(ValueError, match="not on a GPU"):
        L.tp_gather_dim0(dims, full, addr(1), stream=0)
    # the extent follows the call's own sizes: rank r's reduce-scatter slice is n / t, every slice n
    part = torch.zeros(2 * n, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out: 2048 bytes, the call needs 4096"):
        L.tp_reduce_scatter_dim0(dims, -1, addr(0), None, torch.zeros(n // 2, dtype=torch.bfloat16), stream=0,
                                 dtype=BF16)
    with pytest.raises(ValueError, match="not on a GPU"):
        L.tp_reduce_scatter_dim0(dims, 1, addr(0), None, torch.zeros(n // 2, dtype=torch.bfloat16), stream=0,
                                 dtype=BF16)
    with pytest.raises(ValueError, match="partials: 4096 bytes, the call needs 8192"):
        L.tp_reduce_scatter_dim0(dims, 1, part[:n], None, addr(1), stream=0)
    # SwiGLU doubles the column shard: A_i of [64, 128] is short for ffn = 256, t = 2
    md = L.make_dims(s=16, b=2, h=64, ffn=256, t=2)
    with pytest.raises(ValueError, match="A_i"):
        L.tp_mlp_fwd(md, 0, "swiglu", addr(0), torch.zeros(64 * 128, dtype=torch.bfloat16), None, addr(2), addr(3),
                     addr(4), addr(5), stream=0, dtype=BF16)


def test_built_library_matches_the_sources():
    """build() records a hash of the sources and flags next to the library; load() rebuilds when it no longer
    matches, so a library built from other sources is never used."""
    from attention_block_columnparallel_amd.build import built_hash, is_current, source_hash

    assert is_current() and built_hash() == source_hash()
    assert source_hash(("-DSOMETHING_ELSE",)) != source_hash()


def test_source_hash_does_not_depend_on_where_the_tree_is(tmp_path):
    """The same sources at another path (a copy of the tree elsewhere, as on a machine that runs it from a scratch
    directory) hash the same, so a library built here is not rebuilt there; a changed source still changes it."""
    import importlib
    import importlib.util
    import shutil

    B = importlib.import_module("attention_block_columnparallel_amd.build")  # the module, not the build() it exports

    root2 = tmp_path / "elsewhere"
    shutil.copytree(B.CSRC, root2 / "attention_block_columnparallel_amd" / "csrc")
    shutil.copytree(B.INCLUDE, root2 / "include")
    shutil.copy(B.__file__, root2 / "attention_block_columnparallel_amd" / "build.py")
    spec = importlib.util.spec_from_file_location("build_copy", root2 / "attention_block_columnparallel_amd" / "build.py")
    B2 = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(B2)
    assert B2.ROOT != B.ROOT and B2.source_hash() == B.source_hash()
    with open(root2 / "include" / "tpshard.h", "a") as f:
        f.write("\n")
    assert B2.source_hash() != B.source_hash()


def test_vocab_logits_validation(L):
    P = [addr(i) for i in range(6)]

    def fwd(rows=64, h=32, v=48, dt=BF16, ptrs=None):
        q = ptrs or P[:3]  # X, E_i, logits_i
        return L.tp_vocab_logits_fwd(rows, h, v, *q, stream=0, dtype=dt, check=False)

    def bwd(rows=64, h=32, v=48, dt=BF16, ptrs=None):
        q = ptrs or P[:5]  # X, E_i, dlogits_i, dX_i, dE_i
        return L.tp_vocab_logits_bwd(rows, h, v, *q, stream=0, dtype=dt, check=False)

    for i in range(3):
        assert fwd(ptrs=P[:i] + [None] + P[i + 1:3]) == -1, i
    assert fwd(rows=0) == -2 and fwd(v=-8) == -2
    assert fwd(dt=5) == -4
    assert fwd(v=44) == -7 and fwd(h=30) == -7                        # bf16 rows of 8
    assert fwd(ptrs=[P[0], P[1] + 2, P[2]]) == -7                      # misaligned E_i
    assert fwd(ptrs=[P[0], P[1], P[0]]) == -6                          # logits over X
    assert bwd(ptrs=[P[0], P[1], P[2], None, None]) == -1              # no output
    assert bwd(ptrs=[P[0], None, P[2], P[3], None]) == -1              # dX needs E_i
    assert bwd(ptrs=[None, P[1], P[2], None, P[4]]) == -1              # dE needs X
    assert bwd(ptrs=[P[0], P[1], P[2], P[2], P[4]]) == -6              # dX over dlogits
    assert bwd(v=12) == -7


def test_ln_fold_validation(L):
    P = [addr(i) for i in range(11)]
    dims = L.make_dims(s=16, b=2, h=128, ffn=256, t=2)

    def fold(dims=dims, act="gelu", dt=BF16, ptrs=None):
        q = ptrs or P[:7]  # gamma, beta, A_i, a_i, A_ln, c_ln, b_ln
        return L.tp_ln_fold_weights(dims, act, *q, stream=0, dtype=dt, check=False)

    def fwd(dims=dims, rank=0, act="gelu", dt=BF16, ptrs=None):
        q = ptrs or P[:10]  # X, mean, rstd, A_ln, c_ln, b_ln, B_i, U_i, Y_i, Z_i
        return L.tp_ln_mlp_fwd(dims, rank, act, *q, stream=0, dtype=dt, check=False)

    for i in (0, 1, 2, 4, 5, 6):
        assert fold(ptrs=P[:i] + [None] + P[i + 1:7]) == -1, i
    for i in range(10):
        assert fwd(ptrs=P[:i] + [None] + P[i + 1:10]) == -1, i
    assert fold(dt=F32) == -7 and fwd(dt=F32) == -7          # bf16 only
    assert fwd(dims=L.make_dims(s=16, b=2, h=96, ffn=256, t=2)) == -7   # h % 64
    assert fwd(dims=L.make_dims(s=16, b=2, h=64, ffn=256, t=2)) == -7   # h >= 128
    assert fwd(dims=L.make_dims(s=16, b=2, h=128, ffn=255, t=2)) == -3  # ffn % t
    assert fwd(dims=L.make_dims(s=16, b=2, h=128, ffn=250, t=2)) == -7  # ffn/t % 8
    assert fwd(rank=2) == -5
    assert fwd(dims=L.make_dims(s=0, b=2, h=128, ffn=256, t=2)) == -2
    assert fold(ptrs=P[:4] + [P[2]] + P[5:7]) == -6           # A_ln over A_i
    assert fwd(ptrs=P[:7] + [P[0]] + P[8:10]) == -6           # U_i over X
