"""The no-allocation variant of the sequence-parallel region's backward (tp_sp_dropout_add_ln_bwd_noalloc), through
the C ABI: its outputs equal, bit for bit, those of tp_sp_dropout_add_ln_bwd with a caller workspace (the same
kernels, with the library's fixed 16 MiB scratch in place of the workspace), on two calls in a row -- the first
filling the scratch (512 rows of 8192: 256 partial rows of 2 x 8192 fp32), the second smaller, so a stale partial
row left by the first call would show -- in bf16 with dropout and in fp32 without."""
import numpy as np
import pytest
import torch

import tp_inputs as TI
from parity_utils import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_block_columnparallel_amd as pkg

    return pkg.load()


def _case(L, rows, h, dtype, p, seed):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    sp = TI.sp_region_inputs(rows, h, dtype, seed=seed)
    z, res = dev(sp["z"], dtype), dev(sp["residual"], dtype)
    gam, bet = dev(sp["gamma"], dtype), dev(sp["beta"], dtype)
    bits = torch.from_numpy(sp["bits"].view(np.int32)).cuda()
    u, y = torch.empty((rows, h), dtype=tdt, device="cuda"), torch.empty((rows, h), dtype=tdt, device="cuda")
    mean, rstd = torch.empty(rows, device="cuda"), torch.empty(rows, device="cuda")
    mask = torch.empty((rows, h // 8), dtype=torch.uint8, device="cuda")
    L.tp_sp_dropout_add_ln_fwd(rows, h, p, 1e-5, z, res, bits, gam, bet, u, y, mean, rstd, mask)
    dy, dres_in = dev(sp["dy"], dtype), dev(sp["residual"], dtype)
    outs = {}
    for variant in ("workspace", "noalloc"):
        dres, dz = torch.empty_like(u), torch.empty_like(u)
        dg, db = torch.empty(h, device="cuda"), torch.empty(h, device="cuda")
        if variant == "workspace":
            ws = torch.empty(L.tp_sp_ln_bwd_workspace(rows, h) // 4, device="cuda")
            L.tp_sp_dropout_add_ln_bwd(rows, h, p, u, gam, mean, rstd, dy, dres_in, mask, dres, dz, dg, db, ws)
        else:
            L.tp_sp_dropout_add_ln_bwd_noalloc(rows, h, p, u, gam, mean, rstd, dy, dres_in, mask, dres, dz, dg, db)
        torch.cuda.synchronize()
        outs[variant] = (dres, dz, dg, db)
    for name, a, b in zip(("dres", "dz", "dgamma", "dbeta"), outs["workspace"], outs["noalloc"]):
        ia = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
        ib = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
        assert torch.equal(ia, ib), f"{name} rows={rows} h={h} {dtype}: no-allocation result differs"


def test_noalloc_matches_workspace_twice_second_smaller(L):
    say("SP backward no-allocation variant: 512 x 8192 bf16 p=0.1 (fills the scratch), then 100 x 1024 bf16")
    _case(L, 512, 8192, "bf16", 0.1, seed=21)
    _case(L, 100, 1024, "bf16", 0.1, seed=22)


def test_noalloc_fp32_no_dropout_twice(L):
    say("SP backward no-allocation variant: 300 x 2048 fp32 p=0, then 40 x 520 fp32")
    _case(L, 300, 2048, "f32", 0.0, seed=23)
    _case(L, 40, 520, "f32", 0.0, seed=24)


def test_noalloc_rejects_oversize_before_any_launch(L):
    # 256 workgroups x 2 x 12288 fp32 = 24 MiB > 16 MiB: rejected by the host check, no kernel runs
    # (raw addresses: the library refuses the size before it would touch any of them, and the binding's own extent
    # check applies to tensors only)
    rows, h = 512, 12288
    t = torch.empty(8, dtype=torch.bfloat16, device="cuda").data_ptr()
    f = torch.empty(8, device="cuda").data_ptr()
    st = L.tp_sp_dropout_add_ln_bwd_noalloc(rows, h, 0.0, t, t, f, f, t, None, None, None, t, f, f, dtype="bf16",
                                            check=False)
    assert st == -9 and L.STATUS[st] == "TP_E_SCRATCH"
