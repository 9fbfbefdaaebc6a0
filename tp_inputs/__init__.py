"""Seeded synthetic inputs for the tensor-parallel block, shared by the tests, the bench and the oracle.

This module holds no arithmetic of the method itself: it draws normal variates, stores them in the activation
dtype, and names the workload shapes.  Both the HIP path and the oracle receive exactly the bits produced here.

Recipe (one stream per tensor, so adding a tensor never shifts another):
  rng = numpy.random.default_rng(SeedSequence([seed, tensor_id]))
  values = rng.standard_normal(shape, dtype=float32) * std
  bf16 storage: round-to-nearest-even of those fp32 values (torch's CPU conversion); fp32 storage keeps them as is.

Tensor ids: X=0, A (or Wqkv)=1, B (or Wo)=2, dZ=3, column bias=4, row bias=5, partial sums=7; the
sequence-parallel region adds LayerNorm gamma=8, beta=9, residual=10, dropout random words=11, dy=12; the
vocab-parallel cross entropy logits=13, targets=14, per-row loss gradients=15; the vocab-parallel output layer's
weight E [V, h] = 16 and a synthetic upstream logit gradient = 17.
Distributions follow the workloads of the pages: activations and upstream gradients N(0,1), weights N(0, 0.02^2)
(0.02 is the standard deviation, the GPT/Megatron init convention), biases N(0, 0.02^2); LayerNorm gamma
1 + N(0, 0.1^2) and beta N(0, 0.1^2) (a trained-looking affine, not the identity, so a dropped gamma or beta
shows).  Random words: rng.integers(0, 2^32) from the same per-tensor stream, one uint32 per element.
Cross entropy: logits N(0, 2^2); targets uniform over the vocab, with one row in 64 (chosen by the same stream)
set to -100, an ignored row; per-row loss gradients N(0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

T_X, T_A, T_B, T_DZ, T_BIAS_COL, T_BIAS_ROW = 0, 1, 2, 3, 4, 5
T_GAMMA, T_BETA, T_RESID, T_BITS, T_DY = 8, 9, 10, 11, 12
T_LOGITS, T_TARGETS, T_DLOSS = 13, 14, 15
T_EMBED, T_DLOGITS = 16, 17
LOGIT_STD = 2.0
WEIGHT_STD = 0.02


def normal_f32(seed: int, tensor_id: int, shape, std: float = 1.0) -> np.ndarray:
    """fp32 N(0, std^2) array from its own counter-free PCG64 stream keyed by (seed, tensor_id)."""
    rng = np.random.default_rng(np.random.SeedSequence([int(seed), int(tensor_id)]))
    out = rng.standard_normal(tuple(int(v) for v in shape), dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even) and return the raw 16-bit patterns as uint16.

    Uses torch's CPU conversion, a library routine; no method arithmetic happens here."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def tensor(seed: int, tensor_id: int, shape, std: float, dtype: str) -> np.ndarray:
    """A seeded input in its storage form: uint16 bf16 patterns for dtype 'bf16', float32 for 'f32'."""
    x = normal_f32(seed, tensor_id, shape, std)
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one workload in the pages' notation: s, b, h, ffn, a (heads), d (head dim), t (TP degree)."""

    name: str
    kind: str  # "mlp" or "attn"
    s: int
    b: int
    h: int
    t: int
    ffn: int = 0
    a: int = 0
    d: int = 0
    g: int = 0  # KV heads of grouped-query attention (0: g = a, multi-head)
    act: str = "gelu"  # gelu | gelu_tanh | swiglu | relu
    dtype: str = "bf16"  # bf16 | f32
    causal: bool = True
    sp: bool = False  # sequence parallel: dim-0 gather in, dim-0 reduce-scatter out
    seed: int = 0

    @property
    def M(self) -> int:
        return self.s * self.b

    @property
    def f_l(self) -> int:
        return self.ffn // self.t

    @property
    def n1(self) -> int:
        """Width of one rank's column-GEMM output (SwiGLU carries gate and up columns)."""
        return 2 * self.f_l if self.act == "swiglu" else self.f_l

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny fp32 MLP, the 8.3B-width MLP shard, the default-calculator MLP shard,
# a sequence-parallel SwiGLU MLP at Llama-70B width, and a 22B-width causal attention block shard.
TINY = Workload("tiny_mlp_f32_t2", "mlp", s=16, b=2, h=64, ffn=256, t=2, act="gelu", dtype="f32")
MLP_83B = Workload("mlp_h3072_ffn12288_t8_b8_s1024", "mlp", s=1024, b=8, h=3072, ffn=12288, t=8)
MLP_CALC = Workload("mlp_h4096_ffn16384_t8_b8_s2048", "mlp", s=2048, b=8, h=4096, ffn=16384, t=8)
MLP_SP_SWIGLU = Workload("sp_swiglu_h8192_ffn28672_t8_s4096", "mlp", s=4096, b=1, h=8192, ffn=28672, t=8,
                         act="swiglu", sp=True)
ATTN_22B = Workload("attn_h6144_a64_d96_t8_s4096", "attn", s=4096, b=1, h=6144, a=64, d=96, t=8, causal=True,
                    sp=True)

# Llama-70B-sized grouped-query attention ([ATLAS] §6: h 8192, 64 heads of 128, TP 8, s 4096, b 1; [SPCP] Table 4:
# 8 KV heads of 128): per rank 8 query heads sharing one KV head
ATTN_GQA_70B = Workload("attn_gqa_h8192_a64_g8_d128_t8_s4096", "attn", s=4096, b=1, h=8192, a=64, d=128, t=8, g=8,
                        causal=True, sp=True)
WORKLOADS = {w.name: w for w in (TINY, MLP_83B, MLP_CALC, MLP_SP_SWIGLU, ATTN_22B, ATTN_GQA_70B)}


def mlp_inputs(w: Workload, with_bias: bool = False, seed: Optional[int] = None) -> dict:
    """Full (unsharded) MLP inputs in storage form: X [s,b,h], A [h, ffn or 2ffn], B [ffn,h], dZ [s,b,h]."""
    sd = w.seed if seed is None else seed
    wa = 2 * w.ffn if w.act == "swiglu" else w.ffn
    out = {
        "X": tensor(sd, T_X, (w.s, w.b, w.h), 1.0, w.dtype),
        "A": tensor(sd, T_A, (w.h, wa), WEIGHT_STD, w.dtype),
        "B": tensor(sd, T_B, (w.ffn, w.h), WEIGHT_STD, w.dtype),
        "dZ": tensor(sd, T_DZ, (w.s, w.b, w.h), 1.0, w.dtype),
        "a": None,
        "c": None,
    }
    if with_bias:
        out["a"] = tensor(sd, T_BIAS_COL, (wa,), WEIGHT_STD, w.dtype)
        out["c"] = tensor(sd, T_BIAS_ROW, (w.h,), WEIGHT_STD, w.dtype)
    return out


def attn_inputs(w: Workload, with_bias: bool = False, seed: Optional[int] = None) -> dict:
    """Full attention inputs: X [s,b,h], Wqkv [h, (a + 2g)d] = [Wq|Wk|Wv] (head-major columns; g = a unless the
    workload sets g), Wo [ad, h], and the upstream gradient dZ [s,b,h] for the backward."""
    sd = w.seed if seed is None else seed
    ad = w.a * w.d
    nqkv = ad + 2 * (w.g or w.a) * w.d
    out = {
        "X": tensor(sd, T_X, (w.s, w.b, w.h), 1.0, w.dtype),
        "Wqkv": tensor(sd, T_A, (w.h, nqkv), WEIGHT_STD, w.dtype),
        "Wo": tensor(sd, T_B, (ad, w.h), WEIGHT_STD, w.dtype),
        "dZ": tensor(sd, T_DZ, (w.s, w.b, w.h), 1.0, w.dtype),
        "bqkv": None,
        "c": None,
    }
    if with_bias:
        out["bqkv"] = tensor(sd, T_BIAS_COL, (nqkv,), WEIGHT_STD, w.dtype)
        out["c"] = tensor(sd, T_BIAS_ROW, (w.h,), WEIGHT_STD, w.dtype)
    return out


def random_words(seed: int, tensor_id: int, shape) -> np.ndarray:
    """Uniform 32-bit random words (the dropout decisions' randomness, passed to both sides as an input)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, tensor_id]))
    return rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64).astype(np.uint32)


def sp_region_inputs(rows: int, h: int, dtype: str = "bf16", seed: int = 0) -> dict:
    """One rank's sequence-parallel slice [rows = s/t * b, h]: LayerNorm input x, gamma ~ 1 + N(0, 0.1^2),
    beta ~ N(0, 0.1^2), the block output z (after the reduce-scatter), the residual, upstream gradients dy / dout,
    and the dropout random words."""
    return {
        "x": tensor(seed, T_X, (rows, h), 1.0, dtype),
        "gamma": to_bf16_bits(1.0 + normal_f32(seed, T_GAMMA, (h,), 0.1)) if dtype == "bf16"
        else 1.0 + normal_f32(seed, T_GAMMA, (h,), 0.1),
        "beta": tensor(seed, T_BETA, (h,), 0.1, dtype),
        "z": tensor(seed, T_DZ, (rows, h), 1.0, dtype),
        "residual": tensor(seed, T_RESID, (rows, h), 1.0, dtype),
        "dy": tensor(seed, T_DY, (rows, h), 1.0, dtype),
        "bits": random_words(seed, T_BITS, (rows, h)),
    }


def vocab_ce_inputs(rows: int, vocab: int, dtype: str = "bf16", seed: int = 0) -> dict:
    """Full logits [rows, vocab] (rank r's shard is columns [r*vocab/t, (r+1)*vocab/t)), int32 targets [rows] with
    about 1/64 of the rows ignored (-100), and fp32 per-row loss gradients [rows]."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, T_TARGETS]))
    targets = rng.integers(0, vocab, size=rows).astype(np.int32)
    targets[rng.random(rows) < 1.0 / 64] = -100
    return {"logits": tensor(seed, T_LOGITS, (rows, vocab), LOGIT_STD, dtype), "targets": targets,
            "dloss": normal_f32(seed, T_DLOSS, (rows,))}


def vocab_logits_inputs(rows: int, h: int, vocab: int, dtype: str = "bf16", seed: int = 0) -> dict:
    """The vocab-parallel output layer: token activations X [rows, h] N(0, 1), the output weight E [vocab, h]
    N(0, 0.02^2) (one row per vocab entry; rank r's shard is rows [r*vocab/t, (r+1)*vocab/t)), targets and per-row
    loss gradients as in vocab_ce_inputs, and a synthetic upstream logit gradient dlogits [rows, vocab] N(0, 1) for
    testing the backward GEMMs on their own."""
    ce = vocab_ce_inputs(rows, vocab, dtype, seed)
    return {"X": tensor(seed, T_X, (rows, h), 1.0, dtype), "E": tensor(seed, T_EMBED, (vocab, h), WEIGHT_STD, dtype),
            "targets": ce["targets"], "dloss": ce["dloss"],
            "dlogits": tensor(seed, T_DLOGITS, (rows, vocab), 1.0, dtype)}


def partials(seed: int, t: int, shape, dtype: str = "bf16", tensor_id: int = 7) -> np.ndarray:
    """t stacked unit-normal partial-sum buffers [t, *shape] for the reduction kernels."""
    return tensor(seed, tensor_id, (t,) + tuple(shape), 1.0, dtype)
