"""ctypes binding of libtpshard: the C ABI's entry points under the same names.

Argument marshalling only: tensors become device pointers, dtypes become tp_dtype codes, the current HIP stream
is passed through, a non-zero status becomes TpError.  Every step of the computation runs in the library's HIP
kernels; nothing here computes.  If the shared object is missing this module raises at import: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtpshard.so")

TP_F32, TP_BF16 = 0, 1
ACTS = {"gelu": 0, "gelu_tanh": 1, "swiglu": 2, "relu": 3}
BWD_PHASES = {"all": 0, "dgrad": 1, "wgrad": 2}
(TP_W_FC1, TP_W_FC1_GATE_UP, TP_W_FC2, TP_W_QKV, TP_W_PROJ, TP_B_FC1, TP_B_FC1_GATE_UP, TP_B_QKV) = range(8)
WKINDS = {"fc1": TP_W_FC1, "fc1_gate_up": TP_W_FC1_GATE_UP, "fc2": TP_W_FC2, "qkv": TP_W_QKV, "proj": TP_W_PROJ,
          "b_fc1": TP_B_FC1, "b_fc1_gate_up": TP_B_FC1_GATE_UP, "b_qkv": TP_B_QKV}
STATUS = {0: "TP_OK", -1: "TP_E_NULL", -2: "TP_E_SHAPE", -3: "TP_E_DIVISIBILITY", -4: "TP_E_DTYPE", -5: "TP_E_RANK",
          -6: "TP_E_ALIAS", -7: "TP_E_UNSUPPORTED", -8: "TP_E_HIP", -9: "TP_E_SCRATCH"}
EXPORTED = ["tp_status_str", "tp_last_hip_error", "tp_abi_version", "tp_shard_weights", "tp_mlp_fwd", "tp_mlp_bwd",
            "tp_mlp_bwd_phase",
            "tp_attn_fwd", "tp_attn_bwd", "tp_attn_bwd_workspace", "tp_partial_reduce", "tp_reduce_scatter_dim0", "tp_gather_dim0", "tp_sp_dropout_add_ln_fwd",
            "tp_sp_dropout_add_ln_bwd", "tp_sp_dropout_add_ln_bwd_noalloc", "tp_sp_ln_bwd_workspace", "tp_vocab_ce_fwd_local", "tp_vocab_ce_combine",
            "tp_vocab_ce_bwd", "tp_timing_begin", "tp_timing_end",
            "tp_timing_kernel", "tp_timing_filter"]


class TpError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({_str(status)})"
        if status == -8:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


class tp_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("s", "b", "h", "ffn", "a", "d", "t", "g")]


def make_dims(s=0, b=0, h=0, ffn=0, a=0, d=0, t=1, g=0) -> tp_dims:
    """g: KV heads (query groups) of grouped-query attention; 0 = a (multi-head)."""
    return tp_dims(int(s), int(b), int(h), int(ffn), int(a), int(d), int(t), int(g))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run attention_block_columnparallel_amd.build.build() first")
    # Bind the HIP runtime that torch already loaded (same soname) when torch is present.
    try:
        import torch  # noqa: F401
    except Exception:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I, F64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    D = ctypes.POINTER(tp_dims)
    sig = {
        "tp_status_str": ([I], ctypes.c_char_p),
        "tp_last_hip_error": ([], I),
        "tp_abi_version": ([], I),
        "tp_shard_weights": ([D, I, I, I, P, P, P], I),
        "tp_mlp_fwd": ([D, I, I, I, P, P, P, P, P, P, P, P], I),
        "tp_mlp_bwd": ([D, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P], I),
        "tp_mlp_bwd_phase": ([D, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P], I),
        "tp_attn_fwd": ([D, I, I, I, P, P, P, P, P, P, P, P, P], I),
        "tp_attn_bwd": ([D, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P], I),
        "tp_attn_bwd_workspace": ([D], I64),
        "tp_partial_reduce": ([I64, I64, I, I, P, P, P, P], I),
        "tp_reduce_scatter_dim0": ([D, I, I, P, P, P, P], I),
        "tp_gather_dim0": ([D, I, P, P, P], I),
        "tp_sp_dropout_add_ln_fwd": ([I64, I64, I, F64, F64, P, P, P, P, P, P, P, P, P, P, P], I),
        "tp_sp_dropout_add_ln_bwd": ([I64, I64, I, F64, P, P, P, P, P, P, P, P, P, P, P, P, P], I),
        "tp_sp_dropout_add_ln_bwd_noalloc": ([I64, I64, I, F64, P, P, P, P, P, P, P, P, P, P, P, P], I),
        "tp_sp_ln_bwd_workspace": ([I64, I64], I64),
        "tp_vocab_ce_fwd_local": ([I64, I64, I, I, P, P, P, P], I),
        "tp_vocab_ce_combine": ([I64, I, P, P, P, P, P], I),
        "tp_vocab_ce_bwd": ([I64, I64, I, I, P, P, P, P, P, P], I),
        "tp_timing_begin": ([ctypes.POINTER(P), ctypes.POINTER(P), I], I),
        "tp_timing_end": ([], I),
        "tp_timing_kernel": ([I], ctypes.c_char_p),
        "tp_timing_filter": ([ctypes.c_char_p], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _str(status: int) -> str:
    return lib.tp_status_str(int(status)).decode()


def status_str(status: int) -> str:
    return _str(status)


def _ptr(x) -> Optional[int]:
    """Device (or host) address of a tensor, an int address, or None for NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _dtype_code(x, dtype=None) -> int:
    if dtype is not None:
        return {"f32": TP_F32, "bf16": TP_BF16}.get(dtype, dtype)
    import torch

    if x.dtype == torch.bfloat16:
        return TP_BF16
    if x.dtype == torch.float32:
        return TP_F32
    return -1  # rejected by the library with TP_E_DTYPE


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        if torch.cuda.is_available():
            return int(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status: int, where: str, raise_on_error: bool) -> int:
    if status != 0 and raise_on_error:
        raise TpError(status, where, lib.tp_last_hip_error())
    return status


def _act(act) -> int:
    return ACTS[act] if isinstance(act, str) else int(act)


def tp_shard_weights(dims: tp_dims, rank: int, kind, full, shard, stream=None, dtype=None, check=True) -> int:
    k = WKINDS[kind] if isinstance(kind, str) else int(kind)
    st = lib.tp_shard_weights(ctypes.byref(dims), int(rank), k, _dtype_code(full, dtype), _ptr(full), _ptr(shard),
                              _stream(stream))
    return _check(st, "tp_shard_weights", check)


def tp_mlp_fwd(dims: tp_dims, rank: int, act, X, A_i, a_i, B_i, U_i, Y_i, Z_i, stream=None, dtype=None,
               check=True) -> int:
    st = lib.tp_mlp_fwd(ctypes.byref(dims), int(rank), _act(act), _dtype_code(X, dtype), _ptr(X), _ptr(A_i),
                        _ptr(a_i), _ptr(B_i), _ptr(U_i), _ptr(Y_i), _ptr(Z_i), _stream(stream))
    return _check(st, "tp_mlp_fwd", check)


def tp_mlp_bwd(dims: tp_dims, rank: int, act, X, A_i, B_i, U_i, Y_i, dZ, dU_ws, dA_i, da_i, dB_i, dX_i,
               stream=None, dtype=None, check=True) -> int:
    st = lib.tp_mlp_bwd(ctypes.byref(dims), int(rank), _act(act), _dtype_code(X, dtype), _ptr(X), _ptr(A_i),
                        _ptr(B_i), _ptr(U_i), _ptr(Y_i), _ptr(dZ), _ptr(dU_ws), _ptr(dA_i), _ptr(da_i), _ptr(dB_i),
                        _ptr(dX_i), _stream(stream))
    return _check(st, "tp_mlp_bwd", check)


def tp_mlp_bwd_phase(dims: tp_dims, rank: int, act, phase, X, A_i, B_i, U_i, Y_i, dZ, dU_ws, dA_i, da_i, dB_i, dX_i,
                     stream=None, dtype=None, check=True) -> int:
    ph = BWD_PHASES[phase] if isinstance(phase, str) else int(phase)
    st = lib.tp_mlp_bwd_phase(ctypes.byref(dims), int(rank), _act(act), _dtype_code(dZ, dtype), ph, _ptr(X),
                              _ptr(A_i), _ptr(B_i), _ptr(U_i), _ptr(Y_i), _ptr(dZ), _ptr(dU_ws), _ptr(dA_i), _ptr(da_i),
                              _ptr(dB_i), _ptr(dX_i), _stream(stream))
    return _check(st, "tp_mlp_bwd_phase", check)


def tp_attn_fwd(dims: tp_dims, rank: int, causal: bool, X, Wqkv_i, bqkv_i, Wo_i, QKV_i, O_i, lse_i, Z_i,
                stream=None, dtype=None, check=True) -> int:
    st = lib.tp_attn_fwd(ctypes.byref(dims), int(rank), _dtype_code(X, dtype), 1 if causal else 0, _ptr(X),
                         _ptr(Wqkv_i), _ptr(bqkv_i), _ptr(Wo_i), _ptr(QKV_i), _ptr(O_i), _ptr(lse_i), _ptr(Z_i),
                         _stream(stream))
    return _check(st, "tp_attn_fwd", check)


def tp_attn_bwd(dims: tp_dims, rank: int, causal: bool, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dZ, dO_ws, rec_ws, dQKV_i,
                dWqkv_i, dbqkv_i, dWo_i, dX_i, stream=None, dtype=None, check=True) -> int:
    st = lib.tp_attn_bwd(ctypes.byref(dims), int(rank), _dtype_code(X, dtype), 1 if causal else 0, _ptr(X),
                         _ptr(Wqkv_i), _ptr(Wo_i), _ptr(QKV_i), _ptr(O_i), _ptr(lse_i), _ptr(dZ), _ptr(dO_ws),
                         _ptr(rec_ws), _ptr(dQKV_i), _ptr(dWqkv_i), _ptr(dbqkv_i), _ptr(dWo_i), _ptr(dX_i),
                         _stream(stream))
    return _check(st, "tp_attn_bwd", check)


def tp_attn_bwd_workspace(dims: tp_dims) -> int:
    return int(lib.tp_attn_bwd_workspace(ctypes.byref(dims)))


def tp_partial_reduce(n: int, h: int, t: int, partials, bias_c, out, stream=None, dtype=None, check=True) -> int:
    st = lib.tp_partial_reduce(int(n), int(h), int(t), _dtype_code(partials, dtype), _ptr(partials), _ptr(bias_c),
                               _ptr(out), _stream(stream))
    return _check(st, "tp_partial_reduce", check)


def tp_reduce_scatter_dim0(dims: tp_dims, rank: int, partials, bias_c, out, stream=None, dtype=None,
                           check=True) -> int:
    st = lib.tp_reduce_scatter_dim0(ctypes.byref(dims), int(rank), _dtype_code(partials, dtype), _ptr(partials),
                                    _ptr(bias_c), _ptr(out), _stream(stream))
    return _check(st, "tp_reduce_scatter_dim0", check)


def tp_gather_dim0(dims: tp_dims, slices, out, stream=None, dtype=None, check=True) -> int:
    st = lib.tp_gather_dim0(ctypes.byref(dims), _dtype_code(slices, dtype), _ptr(slices), _ptr(out), _stream(stream))
    return _check(st, "tp_gather_dim0", check)


def tp_sp_dropout_add_ln_fwd(rows: int, h: int, p: float, eps: float, z, residual, bits, gamma, beta, out, y, mean,
                             rstd, mask, stream=None, dtype=None, check=True) -> int:
    st = lib.tp_sp_dropout_add_ln_fwd(int(rows), int(h), _dtype_code(z, dtype), float(p), float(eps), _ptr(z),
                                      _ptr(residual), _ptr(bits), _ptr(gamma), _ptr(beta), _ptr(out), _ptr(y),
                                      _ptr(mean), _ptr(rstd), _ptr(mask), _stream(stream))
    return _check(st, "tp_sp_dropout_add_ln_fwd", check)


def tp_sp_dropout_add_ln_bwd(rows: int, h: int, p: float, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz, dgamma,
                             dbeta, ws, stream=None, dtype=None, check=True) -> int:
    st = lib.tp_sp_dropout_add_ln_bwd(int(rows), int(h), _dtype_code(u, dtype), float(p), _ptr(u), _ptr(gamma),
                                      _ptr(mean), _ptr(rstd), _ptr(dy), _ptr(dres_in), _ptr(mask), _ptr(dres),
                                      _ptr(dz), _ptr(dgamma), _ptr(dbeta), _ptr(ws), _stream(stream))
    return _check(st, "tp_sp_dropout_add_ln_bwd", check)


def tp_sp_dropout_add_ln_bwd_noalloc(rows: int, h: int, p: float, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz,
                                     dgamma, dbeta, stream=None, dtype=None, check=True) -> int:
    st = lib.tp_sp_dropout_add_ln_bwd_noalloc(int(rows), int(h), _dtype_code(u, dtype), float(p), _ptr(u),
                                              _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dy), _ptr(dres_in),
                                              _ptr(mask), _ptr(dres), _ptr(dz), _ptr(dgamma), _ptr(dbeta),
                                              _stream(stream))
    return _check(st, "tp_sp_dropout_add_ln_bwd_noalloc", check)


def tp_sp_ln_bwd_workspace(rows: int, h: int) -> int:
    return int(lib.tp_sp_ln_bwd_workspace(int(rows), int(h)))


def tp_vocab_ce_fwd_local(rows: int, v_local: int, rank: int, logits_i, targets, stats_i, stream=None, dtype=None,
                          check=True) -> int:
    st = lib.tp_vocab_ce_fwd_local(int(rows), int(v_local), int(rank), _dtype_code(logits_i, dtype), _ptr(logits_i),
                                   _ptr(targets), _ptr(stats_i), _stream(stream))
    return _check(st, "tp_vocab_ce_fwd_local", check)


def tp_vocab_ce_combine(rows: int, t: int, stats, targets, loss, lse, stream=None, check=True) -> int:
    st = lib.tp_vocab_ce_combine(int(rows), int(t), _ptr(stats), _ptr(targets), _ptr(loss), _ptr(lse),
                                 _stream(stream))
    return _check(st, "tp_vocab_ce_combine", check)


def tp_vocab_ce_bwd(rows: int, v_local: int, rank: int, logits_i, targets, lse, dloss, dlogits_i, stream=None,
                    dtype=None, check=True) -> int:
    st = lib.tp_vocab_ce_bwd(int(rows), int(v_local), int(rank), _dtype_code(logits_i, dtype), _ptr(logits_i),
                             _ptr(targets), _ptr(lse), _ptr(dloss), _ptr(dlogits_i), _stream(stream))
    return _check(st, "tp_vocab_ce_bwd", check)


class LaunchTimer:
    """Collects per-kernel HIP-event timings of every launch the library makes while armed.

    Usage: with LaunchTimer(capacity) as lt: ...calls...; then lt.results() -> [(kernel name, ms)] after a device
    synchronisation.  Events are created with torch (hipEvent_t handles) and owned here.  only="prefix" records
    just the launches whose kernel name starts with it."""

    def __init__(self, capacity: int = 2048, only: Optional[str] = None):
        self.only = only
        import torch

        self.capacity = capacity
        self._starts = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        self._stops = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        # force creation of the underlying hipEvent_t handles
        for e in self._starts + self._stops:
            e.record()
        torch.cuda.synchronize()
        self._sa = (ctypes.c_void_p * capacity)(*[e.cuda_event for e in self._starts])
        self._so = (ctypes.c_void_p * capacity)(*[e.cuda_event for e in self._stops])
        self.n = 0
        self.names = []

    def __enter__(self):
        st = lib.tp_timing_filter(self.only.encode() if self.only else None)
        if st != 0:
            raise TpError(st, "tp_timing_filter")
        st = lib.tp_timing_begin(self._sa, self._so, self.capacity)
        if st != 0:
            raise TpError(st, "tp_timing_begin")
        return self

    def __exit__(self, *exc):
        self.n = lib.tp_timing_end()
        lib.tp_timing_filter(None)
        self.names = [lib.tp_timing_kernel(i).decode() for i in range(self.n)]
        return False

    def results(self):
        return [(self.names[i], self._starts[i].elapsed_time(self._stops[i])) for i in range(self.n)]
