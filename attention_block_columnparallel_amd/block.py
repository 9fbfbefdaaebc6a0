"""Rank-loop driver: runs all t shards of a block back to back on one GPU through the C ABI.

Device memory comes from torch; every computation is a call into libtpshard.  The t ranks' partial sums are
written side by side ([t][s, b, h]) and reduced on the device by tp_partial_reduce (g / f, all-reduce form) or
tp_reduce_scatter_dim0 (g-bar under sequence parallelism) -- the arrangement of "Tensor Parallelism (TP) 与
Sequence Parallelism (SP)" §2 (f / g) and §5 (their SP variants), with the collectives replaced by an on-device
reduction over local buffers.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import load


def _dt(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class MlpBlock:
    """All t shards of one MLP block Z = act(X A + a) B (+ c).

    A_full [h, ffn] (SwiGLU: [h, 2ffn] = [gate | up]), B_full [ffn, h], a_full / c_full optional, all device
    tensors of the activation dtype.  The shards are packed once by tp_shard_weights."""

    def __init__(self, s: int, b: int, h: int, ffn: int, t: int, act: str, A_full: torch.Tensor,
                 B_full: torch.Tensor, a_full: Optional[torch.Tensor] = None, c_full: Optional[torch.Tensor] = None,
                 stream=None):
        L = load()
        self.L = L
        self.s, self.b, self.h, self.ffn, self.t, self.act = s, b, h, ffn, t, act
        self.dims = L.make_dims(s=s, b=b, h=h, ffn=ffn, t=t)
        dev, dt = A_full.device, A_full.dtype
        self.dtype = dt
        f = ffn // t
        self.f = f
        self.n1 = 2 * f if act == "swiglu" else f
        M = s * b
        self.M = M
        wk = "fc1_gate_up" if act == "swiglu" else "fc1"
        bk = "b_fc1_gate_up" if act == "swiglu" else "b_fc1"
        self.A = torch.empty((t, h, self.n1), dtype=dt, device=dev)
        self.B = torch.empty((t, f, h), dtype=dt, device=dev)
        self.a = torch.empty((t, self.n1), dtype=dt, device=dev) if a_full is not None else None
        self.c = c_full
        for r in range(t):
            L.tp_shard_weights(self.dims, r, wk, A_full, self.A[r], stream)
            L.tp_shard_weights(self.dims, r, "fc2", B_full, self.B[r], stream)
            if a_full is not None:
                L.tp_shard_weights(self.dims, r, bk, a_full, self.a[r], stream)
        # saved activations and partial sums, one slot per rank
        self.U = torch.empty((t, M, self.n1), dtype=dt, device=dev)
        self.Y = torch.empty((t, M, f), dtype=dt, device=dev)
        self.Zp = torch.empty((t, M, h), dtype=dt, device=dev)
        self.Z = torch.empty((M, h), dtype=dt, device=dev)
        self.dU = torch.empty((M, self.n1), dtype=dt, device=dev)  # workspace reused by every rank
        self.dA = torch.empty((t, h, self.n1), dtype=dt, device=dev)
        self.da = torch.empty((t, self.n1), dtype=dt, device=dev) if a_full is not None else None
        self.dB = torch.empty((t, f, h), dtype=dt, device=dev)
        self.dXp = torch.empty((t, M, h), dtype=dt, device=dev)
        self.dX = torch.empty((M, h), dtype=dt, device=dev)

    # -- forward: every rank's column + row GEMMs, then g
    def forward_ranks(self, X: torch.Tensor, stream=None):
        for r in range(self.t):
            self.L.tp_mlp_fwd(self.dims, r, self.act, X, self.A[r], None if self.a is None else self.a[r], self.B[r],
                              self.U[r], self.Y[r], self.Zp[r], stream)

    def reduce_forward(self, sp: bool = False, stream=None, out: Optional[torch.Tensor] = None):
        out = self.Z if out is None else out
        if sp:
            self.L.tp_reduce_scatter_dim0(self.dims, -1, self.Zp, self.c, out, stream)
        else:
            self.L.tp_partial_reduce(self.M * self.h, self.h, self.t, self.Zp, self.c, out, stream)
        return out

    def forward(self, X: torch.Tensor, sp: bool = False, stream=None) -> torch.Tensor:
        self.forward_ranks(X, stream)
        return self.reduce_forward(sp, stream)

    # -- backward: every rank's dgrad / wgrad GEMMs, then f on the dX partials
    def backward_ranks(self, X: torch.Tensor, dZ: torch.Tensor, stream=None):
        for r in range(self.t):
            self.L.tp_mlp_bwd(self.dims, r, self.act, X, self.A[r], self.B[r], self.U[r], self.Y[r], dZ, self.dU,
                              self.dA[r], None if self.da is None else self.da[r], self.dB[r], self.dXp[r], stream)

    def reduce_backward(self, sp: bool = False, stream=None, out: Optional[torch.Tensor] = None):
        out = self.dX if out is None else out
        if sp:
            self.L.tp_reduce_scatter_dim0(self.dims, -1, self.dXp, None, out, stream)
        else:
            self.L.tp_partial_reduce(self.M * self.h, self.h, self.t, self.dXp, None, out, stream)
        return out

    def backward(self, X: torch.Tensor, dZ: torch.Tensor, sp: bool = False, stream=None) -> torch.Tensor:
        self.backward_ranks(X, dZ, stream)
        return self.reduce_backward(sp, stream)


    # -- the same step with the reductions on a second stream (communication / computation overlap)
    def forward_pipelined(self, X: torch.Tensor, out_rs: torch.Tensor, chunks: int = 2, comm=None, stream=None,
                          slices: Optional[torch.Tensor] = None):
        """Forward with the g-bar reduce-scatter pipelined along s: the block is run on `chunks` consecutive row
        ranges of the sequence (the MLP is row-wise, so each range is an exact forward of its rows), and as soon
        as every rank has finished range c, the reduce-scatter of the rank slices inside range c runs on `comm`
        while range c + 1 computes ("Tensor Parallelism (TP) 与 Sequence Parallelism (SP)" §5: SP's g is a
        reduce-scatter; the pages' tp_comm_overlap pipelines it with the GEMMs).  out_rs [t, s/t, b, h] receives
        every rank's slice, bit for bit what reduce_forward(sp=True) gives.  With `slices` ([t, s/t, b, h], the
        sequence-parallel input) the all-gather into X is pipelined too: range c's slices are gathered on `comm`
        (the SP f: an all-gather along s) and range c's GEMMs start when they have landed, while range c + 1's
        slices are still being gathered.  Returns the event that marks the last reduction on `comm`."""
        L, t = self.L, self.t
        if self.t % chunks != 0 or self.s % chunks != 0:
            raise ValueError("chunks must divide t (and s)")
        cur = torch.cuda.current_stream() if stream is None else stream
        comm = self._comm(comm)
        rows = (self.s // chunks) * self.b
        dims_c = L.make_dims(s=self.s // chunks, b=self.b, h=self.h, ffn=self.ffn, t=t)
        per = t // chunks
        Xr = X.reshape(self.M, self.h)  # [s, b, h] as s-major rows
        gathered = []
        if slices is not None:
            # every range's gather is queued on comm up front; range c's GEMMs wait for range c's event only
            dims_g = L.make_dims(s=self.s // chunks, b=self.b, h=self.h, t=per)
            src = slices.reshape(t, -1)
            start = torch.cuda.Event()
            start.record(cur)  # X may still be read by earlier work on the compute stream
            comm.wait_event(start)
            for c in range(chunks):
                L.tp_gather_dim0(dims_g, src[c * per:(c + 1) * per], Xr[c * rows:(c + 1) * rows], comm)
                ev = torch.cuda.Event()
                ev.record(comm)
                gathered.append(ev)
        for c in range(chunks):
            sl = slice(c * rows, (c + 1) * rows)
            if gathered:
                cur.wait_event(gathered[c])
            for r in range(t):
                L.tp_mlp_fwd(dims_c, r, self.act, Xr[sl], self.A[r], None if self.a is None else self.a[r], self.B[r],
                             self.U[r][sl], self.Y[r][sl], self.Zp[r][sl], cur)
            ready = torch.cuda.Event()
            ready.record(cur)
            comm.wait_event(ready)
            for j in range(c * per, (c + 1) * per):
                L.tp_reduce_scatter_dim0(self.dims, j, self.Zp, self.c, out_rs[j], comm)
        done = torch.cuda.Event()
        done.record(comm)
        return done

    def backward_overlapped(self, X: torch.Tensor, dZ: torch.Tensor, out_rs: torch.Tensor, comm=None, stream=None):
        """Backward with the dX reduction beside the weight gradients: every rank's dgrad half first (dU_i and the
        dX_i partial), then the reduce-scatter of the dX partials on `comm` while every rank's wgrad half runs on
        the compute stream ([ATLAS] §5: the dgrad reduction and the wgrad GEMMs are independent).  Each rank keeps
        its own dU_i until its wgrad.  Outputs are bit for bit those of backward_ranks + reduce_backward(sp=True).
        Returns the event that marks the reduction's end on `comm`."""
        L, t = self.L, self.t
        cur = torch.cuda.current_stream() if stream is None else stream
        comm = self._comm(comm)
        if getattr(self, "dUr", None) is None:
            self.dUr = torch.empty((t, self.M, self.n1), dtype=self.dtype, device=self.A.device)
        for r in range(t):
            L.tp_mlp_bwd_phase(self.dims, r, self.act, "dgrad", None, self.A[r], self.B[r], self.U[r], None, dZ,
                               self.dUr[r], None, None, None, self.dXp[r], cur)
        ready = torch.cuda.Event()
        ready.record(cur)
        comm.wait_event(ready)
        L.tp_reduce_scatter_dim0(self.dims, -1, self.dXp, None, out_rs, comm)
        done = torch.cuda.Event()
        done.record(comm)
        for r in range(t):
            L.tp_mlp_bwd_phase(self.dims, r, self.act, "wgrad", X, None, None, None, self.Y[r], dZ, self.dUr[r],
                               self.dA[r], None if self.da is None else self.da[r], self.dB[r], None, cur)
        return done

    def step_overlapped(self, X: torch.Tensor, dZ: torch.Tensor, Z_rs: torch.Tensor, dX_rs: torch.Tensor,
                        chunks: int = 2, comm=None, stream=None):
        """forward_pipelined, then backward_overlapped; the compute stream waits for the last reduction."""
        cur = torch.cuda.current_stream() if stream is None else stream
        self.forward_pipelined(X, Z_rs, chunks, comm, cur)
        done = self.backward_overlapped(X, dZ, dX_rs, comm, cur)
        cur.wait_event(done)

    def _comm(self, comm):
        if comm is not None:
            return comm
        if getattr(self, "_comm_stream", None) is None:
            self._comm_stream = torch.cuda.Stream(device=self.A.device)  # default priority
        return self._comm_stream


class AttnBlock:
    """All t shards of one attention block: QKV column-parallel by head, local causal attention, row-parallel
    output projection, partial sums reduced on the device."""

    def __init__(self, s: int, b: int, h: int, a: int, d: int, t: int, Wqkv_full: torch.Tensor,
                 Wo_full: torch.Tensor, bqkv_full: Optional[torch.Tensor] = None,
                 c_full: Optional[torch.Tensor] = None, causal: bool = True, stream=None, g: int = 0):
        """g: KV heads of grouped-query attention (0: g = a); Wqkv_full [h, (a + 2g)d] = [Wq | Wk | Wv]."""
        L = load()
        self.L = L
        self.s, self.b, self.h, self.a, self.d, self.t, self.causal = s, b, h, a, d, t, causal
        self.g = g or a
        self.dims = L.make_dims(s=s, b=b, h=h, a=a, d=d, t=t, g=self.g)
        dev, dt = Wqkv_full.device, Wqkv_full.dtype
        hl = a // t
        self.hl = hl
        self.nqkv = (hl + 2 * (self.g // t)) * d  # a rank's QKV columns
        M = s * b
        self.M = M
        self.Wqkv = torch.empty((t, h, self.nqkv), dtype=dt, device=dev)
        self.Wo = torch.empty((t, hl * d, h), dtype=dt, device=dev)
        self.bqkv = torch.empty((t, self.nqkv), dtype=dt, device=dev) if bqkv_full is not None else None
        self.c = c_full
        for r in range(t):
            L.tp_shard_weights(self.dims, r, "qkv", Wqkv_full, self.Wqkv[r], stream)
            L.tp_shard_weights(self.dims, r, "proj", Wo_full, self.Wo[r], stream)
            if bqkv_full is not None:
                L.tp_shard_weights(self.dims, r, "b_qkv", bqkv_full, self.bqkv[r], stream)
        self.QKV = torch.empty((t, M, self.nqkv), dtype=dt, device=dev)
        self.O = torch.empty((t, M, hl * d), dtype=dt, device=dev)
        self.lse = torch.empty((t, b, hl, s), dtype=torch.float32, device=dev)
        self.Zp = torch.empty((t, M, h), dtype=dt, device=dev)
        self.Z = torch.empty((M, h), dtype=dt, device=dev)

    def _alloc_backward(self):
        if getattr(self, "dQKV", None) is not None:
            return
        t, M, hl, d, h = self.t, self.M, self.hl, self.d, self.h
        dev, dt = self.Wqkv.device, self.Wqkv.dtype
        nqb = (self.s + 63) // 64
        self.dO = torch.empty((M, hl * d), dtype=dt, device=dev)  # workspace reused by every rank
        self.rec = torch.empty(self.L.tp_attn_bwd_workspace(self.dims) // 4, dtype=torch.float32, device=dev)
        self.dQKV = torch.empty((t, M, self.nqkv), dtype=dt, device=dev)
        self.dWqkv = torch.empty((t, h, self.nqkv), dtype=dt, device=dev)
        self.dbqkv = torch.empty((t, self.nqkv), dtype=dt, device=dev) if self.bqkv is not None else None
        self.dWo = torch.empty((t, hl * d, h), dtype=dt, device=dev)
        self.dXp = torch.empty((t, M, h), dtype=dt, device=dev)
        self.dX = torch.empty((M, h), dtype=dt, device=dev)

    # -- backward: every rank's gradients (after forward_ranks on the same X), then f on the dX partials
    def backward_ranks(self, X: torch.Tensor, dZ: torch.Tensor, stream=None):
        self._alloc_backward()
        for r in range(self.t):
            self.L.tp_attn_bwd(self.dims, r, self.causal, X, self.Wqkv[r], self.Wo[r], self.QKV[r], self.O[r],
                               self.lse[r], dZ, self.dO, self.rec, self.dQKV[r], self.dWqkv[r],
                               None if self.dbqkv is None else self.dbqkv[r], self.dWo[r], self.dXp[r], stream)

    def backward(self, X: torch.Tensor, dZ: torch.Tensor, sp: bool = False, stream=None) -> torch.Tensor:
        self.backward_ranks(X, dZ, stream)
        if sp:
            self.L.tp_reduce_scatter_dim0(self.dims, -1, self.dXp, None, self.dX, stream)
        else:
            self.L.tp_partial_reduce(self.M * self.h, self.h, self.t, self.dXp, None, self.dX, stream)
        return self.dX

    def forward_ranks(self, X: torch.Tensor, stream=None):
        for r in range(self.t):
            self.L.tp_attn_fwd(self.dims, r, self.causal, X, self.Wqkv[r], None if self.bqkv is None else self.bqkv[r],
                               self.Wo[r], self.QKV[r], self.O[r], self.lse[r], self.Zp[r], stream)

    def forward(self, X: torch.Tensor, sp: bool = True, stream=None) -> torch.Tensor:
        self.forward_ranks(X, stream)
        if sp:
            self.L.tp_reduce_scatter_dim0(self.dims, -1, self.Zp, self.c, self.Z, stream)
        else:
            self.L.tp_partial_reduce(self.M * self.h, self.h, self.t, self.Zp, self.c, self.Z, stream)
        return self.Z
