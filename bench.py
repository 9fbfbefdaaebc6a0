#!/usr/bin/env python3
"""Benchmark of the tensor-parallel MLP block on one MI355X.

One step = the whole hot path over one batch of seeded synthetic input at the default-calculator width
(h=4096, ffn=16384, t=8, b=8, s=2048, GeLU, bf16): for every rank i the column GEMM with fused GeLU, the row GEMM
into partial buffer i; the g reduction (dim-0 reduce-scatter over the 8 partial buffers, every rank's slice);
for every rank the backward dgrad / wgrad GEMMs into dX partial i; the f reduction of the dX partials (same
kernel).  Inputs and weights are resident in HBM before the timed region; the shards are packed once, before it.

Prints ONE JSON line.  value = algorithmic GEMM flops of the step / wall time of the step (whole job, including
both reductions), in TFLOP/s.  A census pass of K steps first brackets every library launch with HIP events (the
"kernels" table and the step's dominant kernel); the timed region then runs K more steps with events around the
dominant kernel's launches only, since every event pair adds launch latency.  roofline = that kernel's
algorithmic flops per launch over its average HIP-event duration inside the timed region, against the dense bf16
MFMA peak.  rs_dim0 = the reduce-scatter kernel (census pass) against HBM bandwidth.  traffic = HBM bytes per
launch from the committed rocprofv3 counter summary under profiles/ (null once the kernel source differs from the
one profiled).  cpu_baseline = the fp64 oracle on a bounded sample.

overlap, attention_block(_gqa), gather_dim0, sp_region, ln_fused, output_layer and the two other MLP workloads = the other
rows of the hot path, timed after the step (not part of value): the same step with its reductions on a second
stream beside the GEMMs (serial vs overlapped ms/step); the attention block forward and backward at the 22B-class
shape and at the Llama-70B-sized grouped-query shape; the dim-0 gather at the Llama-70B-sized SP shape (rotating
over buffer sets larger than the Infinity Cache); the sequence-parallel region (dropout + residual + LayerNorm,
forward and backward) on every rank's rows at that same shape; the SP entry with the LayerNorm folded into the
column GEMM against the LayerNorm output written and read back; the vocab-parallel output layer (logits GEMM, cross
entropy, backward GEMMs, dX all-reduce) at 16384 token rows, h=4096 and a 51200-entry vocab; the 8.3B-width MLP
(h=3072, ffn=12288, s=1024, b=8; all-reduce form) and the sequence-parallel SwiGLU MLP (h=8192, ffn=28672,
s=4096, b=1; all-gather in, reduce-scatter out), each a whole fwd+bwd step with per-kernel rates.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "TP-shard MLP fwd+bwd TFLOP/s & % bf16 MFMA peak; dim0 reduce-scatter GB/s"
PEAK_BF16_FLOPS = 2.5e15  # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12   # MI355X HBM3E


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mlp_h4096_ffn16384_t8_b8_s2048")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the overlap, attention-block, gather, SP-region, output-layer and other-MLP legs")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one dim-0 gather (a plain copy) of this many MiB, for counter calibration")
    return ap.parse_args(argv)


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def profiled_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE,
    scaled by a plain copy's readings), or None when there is none or the kernel's source has changed since."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    src = "comm_kernels.hip" if kernel.startswith("reduce") else "gemm_bf16.hip"
    with open(os.path.join(root, "attention_block_columnparallel_amd", "csrc", src), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 4 and parts[0] == "traffic" and parts[1] == kernel:
                return int(parts[2]) if parts[3] == sha else None
    return None


def attention_block_measure(L, steps: int, warmup: int, w=None) -> dict:
    """The attention block at the 22B-class shape (h=6144, 64 heads of 96, s=4096, t=8, causal), or the workload w
    (the Llama-70B-sized grouped-query shape: 64 query and 8 KV heads of 128).  Forward: for every
    rank the QKV GEMM, local causal attention and output projection into partial i, then the dim-0 reduce-scatter.
    Backward: for every rank tp_attn_bwd (dO GEMM, attention core backward, the weight-gradient pair, the dX GEMM),
    then the reduce-scatter of the dX partials.  Per-kernel HIP-event durations from a pass with every launch
    bracketed; the block times (ms_per_step, tflops_block) from a pass without those events.  Causal attention
    counts only unmasked query-key pairs (forward 4 d, backward 10 d flops per pair)."""
    import numpy as np
    import torch

    import tp_inputs as TI
    from attention_block_columnparallel_amd.block import AttnBlock

    w = TI.ATTN_22B if w is None else w

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    inp = TI.attn_inputs(w)
    X = dev(inp["X"])
    blk = AttnBlock(w.s, w.b, w.h, w.a, w.d, w.t, dev(inp["Wqkv"]), dev(inp["Wo"]), causal=True, g=w.g)
    for _ in range(warmup):
        blk.forward(X, sp=True)
    torch.cuda.synchronize()
    timer = L.LaunchTimer(capacity=steps * (4 * w.t + 1) + 8)  # forward
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    with timer:
        for _ in range(steps):
            blk.forward(X, sp=True)
    e1.record()
    torch.cuda.synchronize()
    hl, M = w.a // w.t, w.s * w.b
    nqkv = blk.nqkv  # the rank's QKV columns: (a/t + 2 g/t) d
    fl = {"qkv": 2.0 * M * w.h * nqkv, "attention": 4.0 * w.d * (w.s * (w.s + 1) / 2) * w.b * hl,
          "proj": 2.0 * M * hl * w.d * w.h}
    # launch order per step: for each rank the QKV GEMM (a split-K GEMM and its partial sum when the GEMM fills few
    # CUs), attention, the output projection; then the reduce-scatter
    roles = {}
    seq = []
    for name, ms in timer.results():
        if name.startswith("reduce"):
            role = "reduce_scatter"
        elif name.startswith("attn_fwd"):
            role = "attention"
        elif name.startswith("gemm_bf16_splitk_"):  # the partial sum of a split-K GEMM
            role = seq[-1]
        else:
            role = "proj" if seq and seq[-1] == "attention" else "qkv"
        seq.append(role)
        r = roles.setdefault(role, {"kernels": {}, "ms": 0.0})
        r["ms"] += ms
        r["kernels"][name] = r["kernels"].get(name, 0.0) + ms

    def block_ms(fn):  # the block's own time, without per-launch events
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a0.record()
        for _ in range(steps):
            fn()
        a1.record()
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / steps

    def role_fields(roles, flops, nbytes_rs):
        out = {}
        for role, r in roles.items():
            per = 1 if role == "reduce_scatter" else w.t
            us = 1e3 * r["ms"] / steps / per
            k = {"us_per_rank" if per > 1 else "us_per_step": round(us, 2),
                 "kernels_us_per_rank" if per > 1 else "kernels_us_per_step":
                     {n: round(1e3 * v / steps / per, 2) for n, v in r["kernels"].items()}}
            if role in flops:
                k["tflops"] = round(flops[role] / (us * 1e-6) / 1e12, 1)
                k["frac_bf16_peak"] = round(flops[role] / (us * 1e-6) / PEAK_BF16_FLOPS, 4)
            else:
                k["bytes"] = nbytes_rs
                k["gbps"] = round(nbytes_rs / (us * 1e-6) / 1e9, 1)
            out[role] = k
        return out

    out = {"workload": w.name, "ms_per_step": round(block_ms(lambda: blk.forward(X, sp=True)), 4),
           "ms_per_step_with_launch_events": round(e0.elapsed_time(e1) / steps, 4)}
    total_fl = w.t * sum(fl.values())
    out["tflops_block"] = round(total_fl / (out["ms_per_step"] * 1e-3) / 1e12, 1)
    rs_bytes = (w.t + 1) * M * w.h * 2
    out["roles"] = role_fields(roles, fl, rs_bytes)
    # backward: every rank's tp_attn_bwd, then the f reduction of the dX partials (dim-0 reduce-scatter)
    dZ = dev(inp["dZ"])
    for _ in range(warmup):
        blk.backward(X, dZ, sp=True)
    torch.cuda.synchronize()
    timer = L.LaunchTimer(capacity=steps * (10 * w.t + 1) + 8)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    with timer:
        for _ in range(steps):
            blk.backward(X, dZ, sp=True)
    e1.record()
    torch.cuda.synchronize()
    pairs = w.s * (w.s + 1) / 2 * w.b * hl
    bfl = {"dO_gemm": 2.0 * M * w.h * hl * w.d, "attention_core_bwd": 10.0 * w.d * pairs,
           "wgrad_pair": 2.0 * M * hl * w.d * w.h + 2.0 * M * w.h * nqkv, "dX_gemm": 2.0 * M * nqkv * w.h}
    roles = {}
    seq = []
    for name, ms in timer.results():
        if name.startswith("reduce"):
            role = "reduce_scatter"
        elif name.startswith("attn_bwd"):
            role = "attention_core_bwd"
        elif "_pair_" in name or name.endswith("MM_store"):
            role = "wgrad_pair"
        elif name.startswith("gemm_bf16_splitk_"):  # the partial sum of a split-K GEMM
            role = seq[-1]
        else:  # the two data-gradient GEMMs of a rank: dO first, dX after the weight gradients
            role = "dX_gemm" if seq and seq[-1] == "wgrad_pair" else "dO_gemm"
        seq.append(role)
        r = roles.setdefault(role, {"kernels": {}, "ms": 0.0})
        r["ms"] += ms
        r["kernels"][name] = r["kernels"].get(name, 0.0) + ms
    bwd = {"ms_per_step": round(block_ms(lambda: blk.backward(X, dZ, sp=True)), 4),
           "ms_per_step_with_launch_events": round(e0.elapsed_time(e1) / steps, 4)}
    bwd["tflops_block"] = round(w.t * sum(bfl.values()) / (bwd["ms_per_step"] * 1e-3) / 1e12, 1)
    bwd["roles"] = role_fields(roles, bfl, rs_bytes)
    out["backward"] = bwd
    del blk, X, dZ
    return out


def overlap_measure(blk, X, dZ, Z_rs, dX_rs, serial_step, steps: int, chunks: int = 2) -> dict:
    """The same MLP step with the reductions on a second stream: forward on `chunks` row ranges with each range's
    reduce-scatter beside the next range's GEMMs, and the backward's dX reduce-scatter beside every rank's wgrad
    half.  Serial and overlapped steps alternate over three rounds; medians of the per-round ms/step."""
    import torch

    def overlapped():
        blk.step_overlapped(X, dZ, Z_rs, dX_rs, chunks=chunks)

    runs = {"serial": serial_step, "overlapped": overlapped}
    for fn in runs.values():
        fn()
    torch.cuda.synchronize()
    times = {k: [] for k in runs}
    for _ in range(3):
        for name, fn in runs.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / steps)
    med = {k: sorted(v)[len(v) // 2] for k, v in times.items()}
    return {"chunks": chunks, "steps_per_round": steps, "serial_ms": round(med["serial"], 4),
            "overlapped_ms": round(med["overlapped"], 4), "speedup": round(med["serial"] / med["overlapped"], 4),
            "rounds_ms": {k: [round(x, 4) for x in v] for k, v in times.items()}}


def gather_measure(L, reps: int, sets: int = 6) -> dict:
    """The sequence-parallel entry gather: t = 8 slices [s/t, b, h] -> [s, b, h] at the Llama-70B-sized SP shape
    (s=4096, b=1, h=8192, bf16): reads and writes 64 MiB.  The launches rotate over `sets` source / destination
    pairs (768 MiB for 6), more than the 256 MB Infinity Cache holds, so each launch streams from HBM."""
    import torch

    t, s, b, h = 8, 4096, 1, 8192
    srcs = [torch.randn((t, s // t, b, h), device="cuda").to(torch.bfloat16) for _ in range(sets)]
    outs = [torch.empty((s, b, h), dtype=torch.bfloat16, device="cuda") for _ in range(sets)]
    dims = L.make_dims(s=s, b=b, h=h, t=t)
    for i in range(sets):
        L.tp_gather_dim0(dims, srcs[i], outs[i])
    torch.cuda.synchronize()
    with L.LaunchTimer(capacity=reps + 2) as lt:
        for i in range(reps):
            L.tp_gather_dim0(dims, srcs[i % sets], outs[i % sets])
    torch.cuda.synchronize()
    ms = sorted(m for _, m in lt.results())
    med = ms[len(ms) // 2]
    nbytes = 2 * s * b * h * 2
    del srcs, outs
    return {"workload": "gather_dim0_t8_s4096_b1_h8192", "buffer_sets": sets, "bytes_per_launch": nbytes,
            "median_us": round(1e3 * med, 2), "gbps": round(nbytes / (med * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (med * 1e-3) / PEAK_HBM_BYTES, 4)}


def mlp_gemm_flops(w, name: str) -> float:
    """Algorithmic flops of one launch of an MLP GEMM kernel at workload w (2 M N K per product)."""
    M, h, fl = w.M, w.h, w.f_l
    n1 = 2 * fl if w.act == "swiglu" else fl
    if "_pair_" in name:
        return 2.0 * M * h * (fl + n1)                       # dB_i and dA_i
    if name.endswith("swiglu_fwd") or name.endswith("bias_act") or name.endswith("KM_bias"):
        return 2.0 * M * h * n1                              # column GEMM
    if name.endswith("KM_store"):
        return 2.0 * M * fl * h                              # row GEMM
    if name.endswith("act_bwd") or name.endswith("swiglu_bwd"):
        return 2.0 * M * h * fl                              # dY = dZ B_i^T (+ act')
    if name.endswith("KK_store"):
        return 2.0 * M * n1 * h                              # dX_i = dU A_i^T
    return 0.0


def mlp_leg(L, w, steps: int, warmup: int = 2) -> dict:
    """Another MLP workload's whole step, all t ranks on the one GPU.  The 8.3B-width GeLU MLP (h=3072,
    ffn=12288, s=1024, b=8): every rank's forward, the all-reduce of the partials, every rank's backward, the
    all-reduce of the dX partials.  The sequence-parallel SwiGLU MLP (h=8192, ffn=28672, s=4096, b=1): the dim-0
    all-gather of the input's 512-token slices, every rank's forward, the reduce-scatter back to slices; then the
    all-gather of the upstream gradient's slices, every rank's backward, the reduce-scatter of the dX partials.
    Per-kernel HIP-event durations from a pass with every launch bracketed; ms_per_step and tflops_step from a pass
    without those events."""
    import numpy as np
    import torch

    import tp_inputs as TI
    from attention_block_columnparallel_amd.block import MlpBlock

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    sp = w.name.startswith("sp_")
    inp = TI.mlp_inputs(w)
    blk = MlpBlock(w.s, w.b, w.h, w.ffn, w.t, w.act, dev(inp["A"]), dev(inp["B"]))
    dims, t = blk.dims, w.t
    if sp:
        Xs = dev(inp["X"]).reshape(t, w.s // t, w.b, w.h)
        dZs = dev(inp["dZ"]).reshape(t, w.s // t, w.b, w.h)
        X = torch.empty((w.s, w.b, w.h), dtype=torch.bfloat16, device="cuda")
        dZ = torch.empty_like(X)
        Zo = torch.empty_like(Xs)
        dXo = torch.empty_like(Xs)
    else:
        X, dZ = dev(inp["X"]), dev(inp["dZ"])
        Zo = torch.empty((w.M, w.h), dtype=torch.bfloat16, device="cuda")
        dXo = torch.empty_like(Zo)
    del inp

    def step():
        if sp:
            L.tp_gather_dim0(dims, Xs, X)
            blk.forward_ranks(X)
            L.tp_reduce_scatter_dim0(dims, -1, blk.Zp, None, Zo)
            L.tp_gather_dim0(dims, dZs, dZ)
            blk.backward_ranks(X, dZ)
            L.tp_reduce_scatter_dim0(dims, -1, blk.dXp, None, dXo)
        else:
            blk.forward_ranks(X)
            L.tp_partial_reduce(w.M * w.h, w.h, t, blk.Zp, None, Zo)
            blk.backward_ranks(X, dZ)
            L.tp_partial_reduce(w.M * w.h, w.h, t, blk.dXp, None, dXo)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    with L.LaunchTimer(capacity=steps * (6 * t + 4) + 8) as lt:
        for _ in range(steps):
            step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n1 = 2 * w.f_l if w.act == "swiglu" else w.f_l
    step_flops = 2.0 * w.M * w.h * (3 * n1 + 3 * w.f_l) * t
    n_bytes = w.M * w.h * 2
    kern = {}
    for name, kms in lt.results():
        kern.setdefault(name, []).append(kms)
    out = {"workload": w.name, "form": "SP: all-gather in, reduce-scatter out" if sp else "all-reduce (g and f)",
           "ms_per_step": round(ms, 4), "step_gflop": round(step_flops / 1e9, 1),
           "tflops_step": round(step_flops / (ms * 1e-3) / 1e12, 1),
           "frac_bf16_peak_step": round(step_flops / (ms * 1e-3) / PEAK_BF16_FLOPS, 4), "kernels": {}}
    for name, v in kern.items():
        avg = 1e3 * float(np.mean(v))
        k = {"launches_per_step": len(v) // steps, "avg_us": round(avg, 2)}
        fl = mlp_gemm_flops(w, name) if name.startswith("gemm") else 0.0
        if fl:
            k["tflops"] = round(fl / (avg * 1e-6) / 1e12, 1)
            k["frac_bf16_peak"] = round(fl / (avg * 1e-6) / PEAK_BF16_FLOPS, 4)
        elif name.startswith("reduce"):
            nb = (t + 1) * n_bytes  # t partials read, the reduced tensor (every rank's slice) written once
            k["gbps"] = round(nb / (avg * 1e-6) / 1e9, 1)
            k["frac_hbm"] = round(nb / (avg * 1e-6) / PEAK_HBM_BYTES, 4)
        elif name.startswith("copy"):
            k["gbps"] = round(2 * n_bytes / (avg * 1e-6) / 1e9, 1)
            k["frac_hbm"] = round(2 * n_bytes / (avg * 1e-6) / PEAK_HBM_BYTES, 4)
        out["kernels"][name] = k
    del blk, X, dZ, Zo, dXo
    return out


def output_layer_measure(L, reps: int) -> dict:
    """The vocab-parallel output layer and its cross entropy at s=2048, b=8 (16384 token rows), h=4096, a
    51200-entry vocab, t=8, bf16: per step, every rank's logits GEMM X E_r^T [16384, 6400] and the CE local pass,
    the combine, then every rank's CE backward and its two backward GEMMs (dE_r = dlogits^T X, dX_r = dlogits E_r),
    and the all-reduce of the dX partials.  Each GEMM is 2 * 16384 * 6400 * 4096 = 859 GFLOP."""
    import numpy as np
    import torch

    import tp_inputs as TI

    rows, h, V, t = 16384, 4096, 51200, 8
    v = V // t
    inp = TI.vocab_logits_inputs(rows, h, V, "bf16", seed=0)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    X = dev(inp["X"])
    E = dev(inp["E"])
    Es = [E[r * v:(r + 1) * v].contiguous() for r in range(t)]
    del E
    tg = torch.from_numpy(inp["targets"]).cuda()
    dl = torch.from_numpy(inp["dloss"]).cuda()
    del inp
    logits = [torch.empty((rows, v), dtype=torch.bfloat16, device="cuda") for _ in range(t)]
    dlog = torch.empty((rows, v), dtype=torch.bfloat16, device="cuda")
    stats = torch.empty((t, rows, 4), dtype=torch.float32, device="cuda")
    loss = torch.empty(rows, dtype=torch.float32, device="cuda")
    lse = torch.empty_like(loss)
    parts = torch.empty((t, rows, h), dtype=torch.bfloat16, device="cuda")
    dE = [torch.empty((v, h), dtype=torch.bfloat16, device="cuda") for _ in range(t)]
    dX = torch.empty((rows, h), dtype=torch.bfloat16, device="cuda")

    def step():
        for r in range(t):
            L.tp_vocab_logits_fwd(rows, h, v, X, Es[r], logits[r])
            L.tp_vocab_ce_fwd_local(rows, v, r, logits[r], tg, stats[r])
        L.tp_vocab_ce_combine(rows, t, stats, tg, loss, lse)
        for r in range(t):
            L.tp_vocab_ce_bwd(rows, v, r, logits[r], tg, lse, dl, dlog)
            L.tp_vocab_logits_bwd(rows, h, v, X, Es[r], dlog, parts[r], dE[r])
        L.tp_partial_reduce(rows * h, h, t, parts, None, dX)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    with L.LaunchTimer(capacity=reps * (6 * t + 2) + 8) as lt:
        for _ in range(reps):
            step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gf = 2.0 * rows * v * h
    alg_bytes = {"vocab_ce_local": rows * v * 2 + rows * 4 + rows * 16,
                 "vocab_ce_combine": t * rows * 16 + rows * 4 * 3,
                 "vocab_ce_bwd": rows * v * 2 * 2 + rows * 4 * 3,
                 "reduce_bf16_t8": (t + 1) * rows * h * 2}
    kern = {}
    for name, kms in lt.results():
        kern.setdefault(name, []).append(kms)
    out = {"workload": "vocab_output_layer_t8_s2048_b8_h4096_v51200", "ms_per_step": round(ms, 4),
           "step_gflop": round(3 * gf * t / 1e9, 1),
           "tflops_gemms_in_step": round(3 * gf * t / (ms * 1e-3) / 1e12, 1), "kernels": {}}
    for name, vv in kern.items():
        avg = 1e3 * float(np.mean(vv))
        k = {"launches_per_step": len(vv) // reps, "avg_us": round(avg, 2)}
        if name.startswith("gemm"):
            k["tflops"] = round(gf / (avg * 1e-6) / 1e12, 1)
            k["frac_bf16_peak"] = round(gf / (avg * 1e-6) / PEAK_BF16_FLOPS, 4)
        elif name in alg_bytes:
            k["gbps"] = round(alg_bytes[name] / (avg * 1e-6) / 1e9, 1)
            k["frac_hbm"] = round(alg_bytes[name] / (avg * 1e-6) / PEAK_HBM_BYTES, 4)
        out["kernels"][name] = k
    del X, Es, logits, dlog, parts, dE, dX
    return out


def sp_region_measure(L, reps: int) -> dict:
    """The sequence-parallel region at the SP SwiGLU shape (s=4096, b=1, h=8192, t=8, bf16; p=0.1): for each rank,
    dropout + residual + LayerNorm forward on its 512 rows, writing y into its rows of the gathered buffer; then
    for each rank the backward (with a residual-stream gradient coming in).  Algorithmic bytes per element:
    forward z, residual, out, y (2 each) + random word (4) + mask bit (1/8); backward u, dy, dres_in, dres, dz
    (2 each) + mask bit.  The per-workgroup partial rows of dgamma / dbeta are scratch, not counted."""
    import numpy as np
    import torch

    import tp_inputs as TI

    s, b, h, t, p, eps = 4096, 1, 8192, 8, 0.1, 1e-5
    rows = s // t * b
    inp = TI.sp_region_inputs(s * b, h, "bf16", seed=0)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    z, res, gam, bet, dy = (dev(inp[k]) for k in ("z", "residual", "gamma", "beta", "dy"))
    bits = torch.from_numpy(inp["bits"].view(np.int32)).cuda()
    U, Yg, dres, dz = (torch.empty_like(z) for _ in range(4))
    mean = torch.empty(s * b, dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)
    mask = torch.empty((s * b, h // 8), dtype=torch.uint8, device="cuda")
    parts = torch.empty((2 * t, h), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.tp_sp_ln_bwd_workspace(rows, h) // 4, dtype=torch.float32, device="cuda")

    def step():
        for r in range(t):
            sl = slice(r * rows, (r + 1) * rows)
            L.tp_sp_dropout_add_ln_fwd(rows, h, p, eps, z[sl], res[sl], bits[sl], gam, bet, U[sl], Yg[sl], mean[sl],
                                       rstd[sl], mask[sl])
        for r in range(t):
            sl = slice(r * rows, (r + 1) * rows)
            L.tp_sp_dropout_add_ln_bwd(rows, h, p, U[sl], gam, mean[sl], rstd[sl], dy[sl], res[sl], mask[sl],
                                       dres[sl], dz[sl], parts[r], parts[t + r], ws)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    with L.LaunchTimer(capacity=reps * 3 * t + 8) as lt:
        for _ in range(reps):
            step()
    torch.cuda.synchronize()
    n = rows * h
    alg = {"sp_dropout_add_ln_fwd": n * (2 * 4 + 4 + 0.125) + 2 * h * 2 + rows * 8,
           "sp_dropout_add_ln_bwd": n * (2 * 5 + 0.125) + h * 2 + rows * 8}
    kern = {}
    for name, ms in lt.results():
        kern.setdefault(name, []).append(ms)
    out = {"workload": "sp_region_t8_s4096_b1_h8192", "rows_per_rank": rows, "p": p, "kernels": {}}
    total_us = 0.0
    for name, v in kern.items():
        med = 1e3 * float(np.median(v))
        total_us += med * len(v) / reps
        k = {"launches_per_step": len(v) // reps, "median_us": round(med, 2)}
        if name in alg:
            k["bytes_per_launch"] = int(alg[name])
            k["gbps"] = round(alg[name] / (med * 1e-6) / 1e9, 1)
            k["frac_hbm"] = round(alg[name] / (med * 1e-6) / PEAK_HBM_BYTES, 4)
        out["kernels"][name] = k
    out["us_per_step_all_ranks"] = round(total_us, 1)
    del z, res, gam, bet, dy, bits, U, Yg, dres, dz
    return out


def ln_fused_measure(L, reps: int) -> dict:
    """The sequence-parallel entry of the SP SwiGLU MLP (s=4096, b=1, h=8192, ffn=28672, t=8, bf16, p=0.1) two ways,
    each for all 8 ranks: (a) every rank's dropout + residual + LayerNorm writes u (the residual stream) and y into
    its rows of the gathered buffer, then every rank's column GEMM (SwiGLU) and row GEMM read y; (b) every rank's
    dropout + residual writes u into the gathered buffer and the row statistics only, then every rank's
    LayerNorm-folded GEMM reads u (tp_ln_mlp_fwd).  The fold of the weights (tp_ln_fold_weights, once per weight
    update) is timed on its own.  Per-kernel HIP-event durations from a bracketed pass, the two forms' ms from
    passes without those events, alternated over three rounds (medians)."""
    import numpy as np
    import torch

    import tp_inputs as TI

    w = TI.MLP_SP_SWIGLU
    s, b, h, t, p, eps = w.s, w.b, w.h, w.t, 0.1, 1e-5
    rows, M = s // t * b, s * b

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    inp = TI.mlp_inputs(w, seed=0)
    sp = TI.sp_region_inputs(M, h, "bf16", seed=0)
    dims = L.make_dims(s=s, b=b, h=h, ffn=w.ffn, t=t)
    A_d, B_d = dev(inp["A"]), dev(inp["B"])
    del inp
    z, res, gam, bet = (dev(sp[k]) for k in ("z", "residual", "gamma", "beta"))
    bits = torch.from_numpy(sp["bits"].view(np.int32)).cuda()
    del sp
    bf = dict(dtype=torch.bfloat16, device="cuda")
    A = [torch.empty((h, w.n1), **bf) for _ in range(t)]
    B = [torch.empty((w.f_l, h), **bf) for _ in range(t)]
    A_ln = [torch.empty((h, w.n1), **bf) for _ in range(t)]
    cv = [torch.empty(w.n1, device="cuda") for _ in range(t)]
    bv = [torch.empty(w.n1, device="cuda") for _ in range(t)]
    for r in range(t):
        L.tp_shard_weights(dims, r, "fc1_gate_up", A_d, A[r])
        L.tp_shard_weights(dims, r, "fc2", B_d, B[r])
    del A_d, B_d
    u_res = torch.empty((M, h), **bf)      # (a) the residual stream
    gath = torch.empty((M, h), **bf)       # (a) gathered y, (b) gathered u
    mean, rstd = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    U, Y, Z = torch.empty((M, w.n1), **bf), torch.empty((M, w.f_l), **bf), torch.empty((t, M, h), **bf)

    def fold():
        for r in range(t):
            L.tp_ln_fold_weights(dims, "swiglu", gam, bet, A[r], None, A_ln[r], cv[r], bv[r])

    def unfused():
        for r in range(t):
            sl = slice(r * rows, (r + 1) * rows)
            L.tp_sp_dropout_add_ln_fwd(rows, h, p, eps, z[sl], res[sl], bits[sl], gam, bet, u_res[sl], gath[sl],
                                       mean[sl], rstd[sl], None)
        for r in range(t):
            L.tp_mlp_fwd(dims, r, "swiglu", gath, A[r], None, B[r], U, Y, Z[r])

    def fused():
        for r in range(t):
            sl = slice(r * rows, (r + 1) * rows)
            L.tp_sp_dropout_add_ln_fwd(rows, h, p, eps, z[sl], res[sl], bits[sl], gam, bet, gath[sl], None,
                                       mean[sl], rstd[sl], None)
        for r in range(t):
            L.tp_ln_mlp_fwd(dims, r, "swiglu", gath, mean, rstd, A_ln[r], cv[r], bv[r], B[r], U, Y, Z[r])

    fold()
    for fn in (unfused, fused):
        fn()
    torch.cuda.synchronize()
    kern = {}
    for name, fn in (("fold", fold), ("unfused", unfused), ("fused", fused)):
        with L.LaunchTimer(capacity=reps * 3 * t + 8) as lt:
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        per = {}
        for kn, kms in lt.results():
            per.setdefault(kn, []).append(kms)
        kern[name] = {kn: {"launches_per_call": len(v) // reps, "avg_us": round(1e3 * float(np.mean(v)), 2)}
                      for kn, v in per.items()}
    times = {"unfused": [], "fused": []}
    for _ in range(3):
        for name, fn in (("unfused", unfused), ("fused", fused)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) / reps)
    med = {k: sorted(v)[1] for k, v in times.items()}
    gf = 2.0 * M * h * (w.n1 + w.f_l) * t
    col = kern["fused"].get("gemm_bf16_big_KM_ln_swiglu", {}).get("avg_us")
    out = {"workload": "sp_entry_ln_swiglu_h8192_ffn28672_t8_s4096", "unfused_ms": round(med["unfused"], 4),
           "fused_ms": round(med["fused"], 4), "speedup": round(med["unfused"] / med["fused"], 4),
           "gemm_gflop": round(gf / 1e9, 1), "kernels": kern,
           "bytes_saved_per_layer": M * h * 2 * 2,  # the LayerNorm output's write and (a) the residual copy
           "fold_us_all_ranks": round(sum(k["avg_us"] * k["launches_per_call"] for k in kern["fold"].values()), 1)}
    if col:
        fl = 2.0 * M * h * w.n1
        out["ln_column_gemm"] = {"avg_us": col, "tflops": round(fl / (col * 1e-6) / 1e12, 1),
                                 "frac_bf16_peak": round(fl / (col * 1e-6) / PEAK_BF16_FLOPS, 4)}
    del A, B, A_ln, cv, bv, u_res, gath, U, Y, Z, z, res
    return out


def cpu_cores() -> dict:
    """The host's CPU count, the CPUs this process may run on, and the BLAS threads NumPy uses (the oracle's
    matrix products run on those)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return {"cpu_count": os.cpu_count(), "affinity": aff, "blas_threads": blas_threads()}


def cpu_baseline(w, inp, target_s: float) -> dict:
    """The oracle (fp64 NumPy, as it stands) on rank shards' fwd + bwd -- the same computation as the GPU's per-rank
    work.  The sample is R token rows of rank 0's shard when that alone takes about target_s; when rank 0's whole
    shard takes less, whole shards of ranks 0, 1, ... until target_s has passed.  Reported in algorithmic TFLOP/s.
    Two more oracle legs, each on a bounded sample of a few seconds: the causal attention forward of one rank at
    the 22B-class shape (the first heads of rank 0, each a whole 4096-token sequence; 4 d flops per unmasked
    query-key pair) and the fp32 rank-order reduce-scatter of the headline step's 8 partial buffers (a slice of
    the token rows), in GB/s of algorithmic bytes."""
    import numpy as np

    import oracle as O
    import tp_inputs as TI

    X = O.as_f64(inp["X"], w.dtype).reshape(w.M, w.h)
    dZ = O.as_f64(inp["dZ"], w.dtype).reshape(w.M, w.h)
    A, B = O.as_f64(inp["A"], w.dtype), O.as_f64(inp["B"], w.dtype)

    def run(R, rank=0):
        t0 = time.perf_counter()
        O.mlp_shard_forward(X[:R], A, B, w.t, rank, w.act)
        O.mlp_shard_backward(X[:R], A, B, dZ[:R], w.t, rank, w.act)
        return time.perf_counter() - t0

    R = 128
    dt = run(R)
    while dt < 0.5 and R < w.M:
        R = min(w.M, R * 4)
        dt = run(R)
    R2 = int(min(w.M, max(R, R * target_s / max(dt, 1e-6))))
    R2 = max(64, (R2 // 64) * 64)
    if R2 < w.M:
        dt2 = run(R2) if R2 != R else dt
        flops = 12.0 * R2 * w.h * w.f_l
        sample = (f"rank 0 shard fwd+bwd (fp64 NumPy) over {R2} of {w.M} token rows: {flops / 1e9:.1f} "
                  f"algorithmic GFLOP in {dt2:.2f} s")
    else:
        dt2 = dt if R == w.M else run(w.M)  # rank 0's whole shard
        ranks = 1
        while dt2 < target_s and ranks < w.t:
            dt2 += run(w.M, ranks)
            ranks += 1
        flops = 12.0 * w.M * w.h * w.f_l * ranks
        sample = (f"ranks 0-{ranks - 1} shards fwd+bwd (fp64 NumPy), all {w.M} token rows each: "
                  f"{flops / 1e9:.1f} algorithmic GFLOP in {dt2:.2f} s")
    del X, dZ, A, B
    cores = cpu_cores()
    out = {"value": flops / dt2 / 1e12, "unit": "TFLOP/s", "cores": cores["blas_threads"], "kind": "oracle",
           "sample": sample, "host": cores}

    # attention forward of rank 0's heads at the 22B-class shape, whole sequences, until ~target_s / 3
    aw = TI.ATTN_22B
    rng = np.random.default_rng(0)
    q, k, vv = (rng.standard_normal((aw.s, aw.d)) for _ in range(3))
    heads, t_att = 0, 0.0
    while t_att < target_s / 3 and heads < aw.a // aw.t:
        t0 = time.perf_counter()
        O.attention_core(q, k, vv, True)
        t_att += time.perf_counter() - t0
        heads += 1
    att_flops = 4.0 * aw.d * aw.s * (aw.s + 1) / 2 * heads
    out["attention_fwd"] = {"value": round(att_flops / t_att / 1e12, 4), "unit": "TFLOP/s",
                            "sample": f"{heads} of rank 0's {aw.a // aw.t} heads (s={aw.s}, d={aw.d}, causal), "
                                      f"{att_flops / 1e9:.1f} GFLOP in {t_att:.2f} s"}

    # fp32 rank-order reduce-scatter of 8 partial buffers, a slice of the headline step's token rows
    rows = 2048
    parts = [rng.standard_normal((rows, w.h)).astype(np.float32) for _ in range(w.t)]
    n_red, t_red = 0, 0.0
    while t_red < target_s / 6 and n_red < 50:
        t0 = time.perf_counter()
        O.reduce_f32_rank_order(parts)
        t_red += time.perf_counter() - t0
        n_red += 1
    red_bytes = (w.t + 1) * rows * w.h * 2.0 * n_red  # the bf16 step's algorithmic bytes for these rows
    out["reduce_scatter"] = {"value": round(red_bytes / t_red / 1e9, 2), "unit": "GB/s",
                             "sample": f"{n_red} passes over {rows} of {w.M} token rows x {w.t} partials "
                                       f"(fp32 rank-order sums), bytes counted as the bf16 step's"}

    # the 8.3B-width MLP: rank 0's whole shard fwd + bwd (about 0.46 TFLOP of fp64 work)
    w2 = TI.WORKLOADS["mlp_h3072_ffn12288_t8_b8_s1024"]
    if w2.name != w.name:
        inp2 = TI.mlp_inputs(w2)
        X2 = O.as_f64(inp2["X"], w2.dtype).reshape(w2.M, w2.h)
        dZ2 = O.as_f64(inp2["dZ"], w2.dtype).reshape(w2.M, w2.h)
        A2, B2 = O.as_f64(inp2["A"], w2.dtype), O.as_f64(inp2["B"], w2.dtype)
        t0 = time.perf_counter()
        O.mlp_shard_forward(X2, A2, B2, w2.t, 0, w2.act)
        O.mlp_shard_backward(X2, A2, B2, dZ2, w2.t, 0, w2.act)
        t2 = time.perf_counter() - t0
        fl2 = 12.0 * w2.M * w2.h * w2.f_l
        out[w2.name] = {"value": round(fl2 / t2 / 1e12, 4), "unit": "TFLOP/s",
                        "sample": f"rank 0's whole shard fwd+bwd (fp64 NumPy): {fl2 / 1e9:.1f} algorithmic GFLOP "
                                  f"in {t2:.2f} s"}
    return out


def main(argv=None) -> int:
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): every rank's "
              "shard runs back to back on that GPU and the reductions are on-device kernels; there is no "
              "multi-GPU path in this build.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import attention_block_columnparallel_amd as pkg
    import tp_inputs as TI
    from attention_block_columnparallel_amd.block import MlpBlock

    L = pkg.load()
    w = TI.WORKLOADS[args.workload]
    if w.kind != "mlp":
        print("bench.py times the MLP block workloads", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    inp = TI.mlp_inputs(w)
    X = dev(inp["X"])
    dZ = dev(inp["dZ"])
    blk = MlpBlock(w.s, w.b, w.h, w.ffn, w.t, w.act, dev(inp["A"]), dev(inp["B"]))
    dims = blk.dims
    Zrs = torch.empty((w.t, w.s // w.t, w.b, w.h), dtype=dt, device="cuda")
    dXrs = torch.empty((w.t, w.s // w.t, w.b, w.h), dtype=dt, device="cuda")

    def step():
        blk.forward_ranks(X)
        L.tp_reduce_scatter_dim0(dims, -1, blk.Zp, None, Zrs)  # g-bar, every rank's slice
        blk.backward_ranks(X, dZ)
        L.tp_reduce_scatter_dim0(dims, -1, blk.dXp, None, dXrs)  # f on the dX partials

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # kernel census: K steps with every library launch bracketed by HIP events (per-kernel durations; each event
    # pair adds launch latency, so this pass is not the timed region)
    launches_per_step = 6 * w.t + 2
    census = L.LaunchTimer(capacity=args.steps * launches_per_step + 8)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    with census:
        for _ in range(args.steps):
            step()
    e1.record()
    torch.cuda.synchronize()
    ms_census = e0.elapsed_time(e1) / args.steps

    M, h, f, t = w.M, w.h, w.f_l, w.t
    gemm_flops = 2.0 * M * h * f  # every GEMM of the step has this size
    step_flops = 12.0 * M * h * f * t

    kern = {}
    for name, ms in census.results():
        k = kern.setdefault(name, {"launches": 0, "total_ms": 0.0})
        k["launches"] += 1
        k["total_ms"] += ms
    rs_name = next((n for n in kern if n.startswith("reduce_bf16") or n.startswith("reduce_f32")), None)
    n_el = w.s * w.b * w.h
    rs_bytes = (t + 1) * n_el * (2 if w.dtype == "bf16" else 4)
    for name, k in kern.items():
        k["avg_us"] = 1e3 * k["total_ms"] / k["launches"]
        k["share"] = k["total_ms"] / (ms_census * args.steps)
        if name.startswith("gemm"):
            k["flops_per_launch"] = gemm_flops * (2 if "_pair_" in name else 1)
            k["tflops"] = k["flops_per_launch"] / (k["avg_us"] * 1e-6) / 1e12
        if name == rs_name:
            k["gbps"] = rs_bytes / (k["avg_us"] * 1e-6) / 1e9
    dom = max((n for n in kern if n.startswith("gemm")), key=lambda n: kern[n]["total_ms"])

    # timed region: K steps bracketed by synchronisation; HIP events bracket only the dominant kernel's launches
    timer = L.LaunchTimer(capacity=args.steps * launches_per_step + 8, only=dom)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    with timer:
        for _ in range(args.steps):
            step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    ms_wall = wall * 1e3 / args.steps
    ms_step = max(ms_per_step, ms_wall)
    value = step_flops / (ms_step * 1e-3) / 1e12
    dom_ms = [ms for name, ms in timer.results() if name == dom]
    dom_us = 1e3 * sum(dom_ms) / len(dom_ms)
    ach = kern[dom]["flops_per_launch"] / (dom_us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                "frac": round(ach * 1e12 / PEAK_BF16_FLOPS, 4), "traffic": profiled_traffic(w.name, dom), "kernel": dom,
                "flops_per_launch": kern[dom]["flops_per_launch"], "avg_us": round(dom_us, 2),
                "launches_timed": len(dom_ms)}
    gemm_ms = sum(k["total_ms"] for n, k in kern.items() if n.startswith("gemm")) / args.steps
    rs = kern[rs_name]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "s": w.s, "b": w.b, "h": w.h, "ffn": w.ffn, "t": w.t, "act": w.act,
                   "ranks": f"all {t} TP shards back to back on one GPU", "step_gflop": round(step_flops / 1e9, 1)},
        "frac_of_bf16_peak": round(value * 1e12 / PEAK_BF16_FLOPS, 4),
        "gemm_tflops_aggregate": round(step_flops / (gemm_ms * 1e-3) / 1e12, 2),
        "roofline": roofline,
        "rs_dim0": {"kernel": rs_name, "gbps": round(rs["gbps"], 1), "frac_hbm": round(rs["gbps"] * 1e9 / PEAK_HBM_BYTES, 4),
                    "bytes_per_launch": rs_bytes, "avg_us": round(rs["avg_us"], 2),
                    "traffic": profiled_traffic(w.name, rs_name)},
        "kernels": {n: {kk: (round(v, 4) if isinstance(v, float) else v) for kk, v in k.items()} for n, k in kern.items()},
        "kernel_census_ms_per_step": round(ms_census, 4),
    }
    if args.calib_copy_mib > 0:
        nbytes = args.calib_copy_mib << 20
        src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").zero_()
        dst = torch.empty_like(src)
        cd = L.make_dims(s=nbytes // 2 // 8, b=1, h=8, t=1)
        with L.LaunchTimer(capacity=4) as ct:
            L.tp_gather_dim0(cd, src, dst)
        torch.cuda.synchronize()
        (cname, cms), = ct.results()
        out["calib_copy"] = {"kernel": cname, "bytes_read": nbytes, "bytes_written": nbytes, "ms": round(cms, 4)}
    if not args.no_extra:
        out["overlap"] = overlap_measure(blk, X, dZ, Zrs, dXrs, step, max(3, args.steps // 2))
    del blk, X, dZ, Zrs, dXrs
    torch.cuda.empty_cache()
    if not args.no_extra:
        out["attention_block"] = attention_block_measure(L, max(2, args.steps // 2), 2)
        torch.cuda.empty_cache()
        out["attention_block_gqa"] = attention_block_measure(L, max(2, args.steps // 2), 2, TI.ATTN_GQA_70B)
        out["gather_dim0"] = gather_measure(L, 24)
        out["sp_region"] = sp_region_measure(L, 10)
        torch.cuda.empty_cache()
        out["ln_fused"] = ln_fused_measure(L, 5)
        torch.cuda.empty_cache()
        out["output_layer"] = output_layer_measure(L, 5)
        torch.cuda.empty_cache()
        for other in ("mlp_h3072_ffn12288_t8_b8_s1024", "sp_swiglu_h8192_ffn28672_t8_s4096"):
            if other != w.name:
                out[other] = mlp_leg(L, TI.WORKLOADS[other], max(3, args.steps // 2))
                torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
