"""Every kernel family gives the same bits when run twice on the same inputs (no atomics, fixed reduction orders):
the attention forward and backward (multi-head and grouped-query, with the split-K GEMMs), the sequence-parallel
region forward and backward, and the vocab-parallel cross entropy.  The MLP GEMMs have their own run-twice test
in test_gpu_mlp.py."""
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


def _bits(x):
    x = x.detach()
    if x.dtype in (torch.bfloat16, torch.float16):
        return x.view(torch.int16).clone()
    if x.dtype == torch.float32:
        return x.view(torch.int32).clone()
    return x.clone()


def _same(a: dict, b: dict, what: str):
    for k in a:
        if a[k] is not None:
            assert torch.equal(_bits(a[k]), _bits(b[k])), f"{what}: {k} differs between two runs"


@pytest.mark.parametrize("g,t", [(0, 2), (2, 2), (8, 8)])
def test_attention_forward_backward_twice(L, g, t):
    from test_gpu_gqa import run_rank

    a, d = 8, 64
    w = TI.Workload("det_attn", "attn", s=200, b=2, h=a * d, a=a, d=d, t=t, g=g or a, causal=True, dtype="bf16")
    say(f"attention fwd+bwd twice s=200 b=2 a={a} g={g or a} d={d} t={t}")
    inp = TI.attn_inputs(w, with_bias=True, seed=31)
    r1 = run_rank(L, w, inp, t - 1, "bf16", True, True)
    r2 = run_rank(L, w, inp, t - 1, "bf16", True, True)
    _same(r1, r2, "attention")


def test_sp_region_twice(L):
    rows, h, p = 300, 4096, 0.1
    say(f"SP region fwd+bwd twice rows={rows} h={h}")
    sp = TI.sp_region_inputs(rows, h, "bf16", seed=32)
    bits = torch.from_numpy(sp["bits"].view(np.int32)).cuda()
    args = [dev(sp[k], "bf16") for k in ("z", "residual")]
    gam, bet, dy = dev(sp["gamma"], "bf16"), dev(sp["beta"], "bf16"), dev(sp["dy"], "bf16")

    def once():
        u, y = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda"), torch.empty((rows, h), dtype=torch.bfloat16,
                                                                                        device="cuda")
        mean, rstd = torch.empty(rows, device="cuda"), torch.empty(rows, device="cuda")
        mask = torch.empty((rows, h // 8), dtype=torch.uint8, device="cuda")
        L.tp_sp_dropout_add_ln_fwd(rows, h, p, 1e-5, args[0], args[1], bits, gam, bet, u, y, mean, rstd, mask)
        dres, dz = torch.empty_like(u), torch.empty_like(u)
        dg, db = torch.empty(h, device="cuda"), torch.empty(h, device="cuda")
        ws = torch.empty(L.tp_sp_ln_bwd_workspace(rows, h) // 4, device="cuda")
        L.tp_sp_dropout_add_ln_bwd(rows, h, p, u, gam, mean, rstd, dy, None, mask, dres, dz, dg, db, ws)
        torch.cuda.synchronize()
        return dict(u=u, y=y, mean=mean, rstd=rstd, mask=mask, dres=dres, dz=dz, dg=dg, db=db)

    _same(once(), once(), "SP region")


def test_vocab_ce_twice(L):
    from test_gpu_vocab_ce import run

    rows, V, t = 257, 51200, 8
    say(f"vocab CE twice rows={rows} V={V} t={t}")
    inp = TI.vocab_ce_inputs(rows, V, "bf16", seed=33)
    a = run(L, inp, rows, V, t, "bf16")
    b = run(L, inp, rows, V, t, "bf16")
    _same(dict(stats=a[0], loss=a[1], lse=a[2]), dict(stats=b[0], loss=b[1], lse=b[2]), "vocab CE")
    for r in range(t):
        assert torch.equal(_bits(a[3][r]), _bits(b[3][r])), f"vocab CE dlogits rank {r} differs"
