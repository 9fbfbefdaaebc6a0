"""Communication / computation overlap of the MLP step (two streams), against the serial step and the oracle.

The overlapped schedule changes only when the kernels run, never what they compute: the forward runs the block on
consecutive row ranges of the sequence with each range's reduce-scatter on a second stream, and the backward
runs every rank's dgrad half, then the dX reduce-scatter on the second stream beside every rank's wgrad half.  So
every output must equal the serial step's bit for bit (same kernels, same inputs), and the serial step's outputs
are checked against the fp64 oracle.  Cases: GeLU with biases and SwiGLU, t = 4 with two and four row ranges, at
sizes spanning several tiles with ragged tails, repeated so that a reduction still running from one step would
show in the next.
"""
import numpy as np
import pytest
import torch

import oracle as O
import tp_inputs as TI
from parity_utils import check_close, dev, empty, f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_block_columnparallel_amd as pkg

    return pkg.load()


def _bits(x):
    return x.reshape(-1).view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).clone()


@pytest.mark.parametrize("act,chunks,with_bias", [("gelu", 2, True), ("swiglu", 4, False)])
def test_overlapped_step_equals_serial_step(L, act, chunks, with_bias):
    from attention_block_columnparallel_amd.block import MlpBlock

    w = TI.Workload("ovl", "mlp", s=96, b=2, h=264, ffn=4 * 200, t=4, act=act, dtype="bf16")
    say(f"overlapped MLP step act={act} chunks={chunks} bias={with_bias} (s={w.s} b={w.b} h={w.h} ffn={w.ffn} t={w.t})")
    inp = TI.mlp_inputs(w, with_bias=with_bias, seed=5)
    a = dev(inp["a"], "bf16") if with_bias else None
    c = dev(inp["c"], "bf16") if with_bias else None
    blk = MlpBlock(w.s, w.b, w.h, w.ffn, w.t, act, dev(inp["A"], "bf16"), dev(inp["B"], "bf16"), a, c)
    X, dZ = dev(inp["X"], "bf16"), dev(inp["dZ"], "bf16")
    shape_rs = (w.t, w.s // w.t, w.b, w.h)

    # serial: every rank forward, g-bar, every rank backward, f
    Zs, dXs = empty(shape_rs, "bf16"), empty(shape_rs, "bf16")
    blk.forward_ranks(X)
    blk.reduce_forward(sp=True, out=Zs)
    blk.backward_ranks(X, dZ)
    blk.reduce_backward(sp=True, out=dXs)
    torch.cuda.synchronize()
    ref = {"Z": _bits(Zs), "dX": _bits(dXs), "U": _bits(blk.U), "Y": _bits(blk.Y), "dA": _bits(blk.dA),
           "dB": _bits(blk.dB)}
    if with_bias:
        ref["da"] = _bits(blk.da)

    for rep in range(3):
        for name in ("U", "Y", "Zp", "dA", "dB", "dXp"):
            getattr(blk, name).fill_(float("nan"))
        Zo, dXo = torch.full(shape_rs, float("nan"), dtype=torch.bfloat16, device="cuda"), empty(shape_rs, "bf16")
        dXo.fill_(float("nan"))
        blk.step_overlapped(X, dZ, Zo, dXo, chunks=chunks)
        torch.cuda.synchronize()
        got = {"Z": _bits(Zo), "dX": _bits(dXo), "U": _bits(blk.U), "Y": _bits(blk.Y), "dA": _bits(blk.dA),
               "dB": _bits(blk.dB)}
        if with_bias:
            got["da"] = _bits(blk.da)
        for k in ref:
            assert torch.equal(got[k], ref[k]), (rep, k)

    # and the serial step itself against the oracle
    Xo = O.as_f64(inp["X"], "bf16").reshape(w.M, w.h)
    A, B = O.as_f64(inp["A"], "bf16"), O.as_f64(inp["B"], "bf16")
    ao = O.as_f64(inp["a"], "bf16") if with_bias else None
    co = O.as_f64(inp["c"], "bf16") if with_bias else None
    full = O.mlp_forward(Xo, A, B, act, ao, co)
    bwd = O.mlp_backward(Xo, A, B, full["U"], full["Y"], O.as_f64(inp["dZ"], "bf16").reshape(w.M, w.h), act)
    check_close(f64(Zs).reshape(w.M, w.h), full["Z"], "bf16", "Z")
    check_close(f64(dXs).reshape(w.M, w.h), bwd["dX"], "bf16", "dX")
    for r in range(w.t):
        cols = O.mlp_shard_columns(w.ffn, w.t, r, act)
        check_close(f64(blk.dA[r]), bwd["dA"][:, cols], "bf16", f"dA[{r}]")


def test_phase_split_equals_full_backward(L):
    """tp_mlp_bwd_phase dgrad then wgrad gives tp_mlp_bwd's bits (fp32 too)."""
    for dtype in ("bf16", "f32"):
        w = TI.Workload("ph", "mlp", s=40, b=3, h=136, ffn=2 * 184, t=2, act="gelu", dtype=dtype)
        say(f"phase split {dtype}")
        inp = TI.mlp_inputs(w, with_bias=True, seed=9)
        dims = L.make_dims(s=w.s, b=w.b, h=w.h, ffn=w.ffn, t=w.t)
        f = w.f_l
        A_i = dev(O.shard_weight(0, inp["A"], w.t, 1, ffn=w.ffn), dtype)
        B_i = dev(O.shard_weight(2, inp["B"], w.t, 1, ffn=w.ffn), dtype)
        X, dZ = dev(inp["X"], dtype).reshape(w.M, w.h), dev(inp["dZ"], dtype).reshape(w.M, w.h)
        U, Y, Z = empty((w.M, f), dtype), empty((w.M, f), dtype), empty((w.M, w.h), dtype)
        L.tp_mlp_fwd(dims, 1, "gelu", X, A_i, None, B_i, U, Y, Z)
        outs = []
        for split in (False, True):
            dU, dA, da, dB, dX = (empty((w.M, f), dtype), empty((w.h, f), dtype), empty((f,), dtype),
                                  empty((f, w.h), dtype), empty((w.M, w.h), dtype))
            if split:
                L.tp_mlp_bwd_phase(dims, 1, "gelu", "dgrad", None, A_i, B_i, U, None, dZ, dU, None, None, None, dX)
                L.tp_mlp_bwd_phase(dims, 1, "gelu", "wgrad", X, None, None, None, Y, dZ, dU, dA, da, dB, None)
            else:
                L.tp_mlp_bwd(dims, 1, "gelu", X, A_i, B_i, U, Y, dZ, dU, dA, da, dB, dX)
            outs.append([_bits(v) for v in (dU, dA, da, dB, dX)])
        torch.cuda.synchronize()
        for x, y in zip(*outs):
            assert torch.equal(x, y)


def test_pipelined_gather_equals_serial_gather(L):
    """The SP entry all-gather pipelined with the forward (range c's slices gathered on the second stream while
    range c - 1 computes) gives the serial gather + forward + reduce-scatter bit for bit."""
    from attention_block_columnparallel_amd.block import MlpBlock

    w = TI.Workload("ovl_ag", "mlp", s=64, b=3, h=136, ffn=4 * 104, t=4, act="gelu", dtype="bf16")
    say(f"pipelined all-gather + forward (s={w.s} b={w.b} h={w.h} ffn={w.ffn} t={w.t}, 2 and 4 ranges)")
    inp = TI.mlp_inputs(w, with_bias=True, seed=8)
    blk = MlpBlock(w.s, w.b, w.h, w.ffn, w.t, w.act, dev(inp["A"], "bf16"), dev(inp["B"], "bf16"),
                   dev(inp["a"], "bf16"), dev(inp["c"], "bf16"))
    slices = dev(np.stack([O.split_dim0(inp["X"], w.t, r) for r in range(w.t)]), "bf16")
    shape_rs = (w.t, w.s // w.t, w.b, w.h)
    X = empty((w.s, w.b, w.h), "bf16")
    L.tp_gather_dim0(blk.dims, slices, X)
    Zs = empty(shape_rs, "bf16")
    blk.forward_ranks(X)
    blk.reduce_forward(sp=True, out=Zs)
    torch.cuda.synchronize()
    ref_Z, ref_U = _bits(Zs), _bits(blk.U)
    assert torch.equal(_bits(X), _bits(dev(inp["X"], "bf16")))
    for chunks in (2, 4):
        X2 = torch.full((w.s, w.b, w.h), float("nan"), dtype=torch.bfloat16, device="cuda")
        Zo = torch.full(shape_rs, float("nan"), dtype=torch.bfloat16, device="cuda")
        blk.U.fill_(float("nan"))
        done = blk.forward_pipelined(X2, Zo, chunks=chunks, slices=slices)
        torch.cuda.current_stream().wait_event(done)
        torch.cuda.synchronize()
        assert torch.equal(_bits(X2), _bits(X)), chunks
        assert torch.equal(_bits(Zo), ref_Z), chunks
        assert torch.equal(_bits(blk.U), ref_U), chunks
