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
            "tp_vocab_ce_bwd", "tp_vocab_logits_fwd", "tp_vocab_logits_bwd", "tp_ln_fold_weights", "tp_ln_mlp_fwd", "tp_timing_begin", "tp_timing_end",
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
        "tp_vocab_logits_fwd": ([I64, I64, I64, I, P, P, P, P], I),
        "tp_vocab_logits_bwd": ([I64, I64, I64, I, P, P, P, P, P, P], I),
        "tp_ln_fold_weights": ([D, I, I, P, P, P, P, P, P, P, P], I),
        "tp_ln_mlp_fwd": ([D, I, I, I, P, P, P, P, P, P, P, P, P, P, P], I),
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


def _ptr(x, nbytes: int = 0, name: str = "tensor") -> Optional[int]:
    """Address of a tensor (an int address passes as is; None is NULL).

    A tensor must be contiguous and hold at least `nbytes` bytes -- the extent the library will read or write for
    this argument, worked out from the same sizes the call passes -- and live on a GPU; otherwise ValueError, before
    any call into the library (whose kernels trust those extents)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError(f"{name}: not contiguous (the library reads dense row-major memory)")
    have = x.numel() * x.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, the call needs {nbytes}")
    if x.device.type != "cuda":
        raise ValueError(f"{name}: on {x.device}, not on a GPU")
    return int(x.data_ptr())


def _es(code: int) -> int:
    """Bytes per element of a tp_dtype code (unknown codes: 0, and the library rejects the call)."""
    return {TP_F32: 4, TP_BF16: 2}.get(code, 0)


def _pos(*v) -> bool:
    return all(int(x) > 0 for x in v)


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


def _shard_sizes(dims: tp_dims, k: int):
    """(full, shard) element counts of tp_shard_weights' kinds, or (0, 0) where the sizes do not divide."""
    h, f, a, d, t = dims.h, dims.ffn, dims.a, dims.d, dims.t
    g = dims.g or a
    if not _pos(t) or h < 0 or f < 0 or a < 0 or d < 0 or (a and (a % t or g % t)) or f % t:
        return 0, 0
    return {TP_W_FC1: (h * f, h * f // t), TP_W_FC1_GATE_UP: (2 * h * f, 2 * h * f // t),
            TP_W_FC2: (f * h, f // t * h), TP_W_QKV: (h * (a + 2 * g) * d, h * (a // t + 2 * g // t) * d),
            TP_W_PROJ: (a * d * h, a // t * d * h), TP_B_FC1: (f, f // t), TP_B_FC1_GATE_UP: (2 * f, 2 * f // t),
            TP_B_QKV: ((a + 2 * g) * d, (a // t + 2 * g // t) * d)}.get(k, (0, 0))


def tp_shard_weights(dims: tp_dims, rank: int, kind, full, shard, stream=None, dtype=None, check=True) -> int:
    k = WKINDS[kind] if isinstance(kind, str) else int(kind)
    dt = _dtype_code(full, dtype)
    nf, ns = _shard_sizes(dims, k)
    es = _es(dt)
    st = lib.tp_shard_weights(ctypes.byref(dims), int(rank), k, dt, _ptr(full, nf * es, "full"),
                              _ptr(shard, ns * es, "shard"), _stream(stream))
    return _check(st, "tp_shard_weights", check)


def _mlp_bytes(dims: tp_dims, act, dt: int):
    """Bytes of the MLP tensors: X / dZ / Z_i / dX_i, A_i / dA_i, a_i, B_i / dB_i, U_i / dU, Y_i."""
    es, t = _es(dt), max(int(dims.t), 1)
    M, h, fl = dims.s * dims.b, dims.h, dims.ffn // t
    n1 = 2 * fl if _act(act) == ACTS["swiglu"] else fl
    if not _pos(M, h, fl):
        return dict(act=0, a=0, aN=0, b=0, u=0, y=0)
    return dict(act=M * h * es, a=h * n1 * es, aN=n1 * es, b=fl * h * es, u=M * n1 * es, y=M * fl * es)


def tp_mlp_fwd(dims: tp_dims, rank: int, act, X, A_i, a_i, B_i, U_i, Y_i, Z_i, stream=None, dtype=None,
               check=True) -> int:
    dt = _dtype_code(X, dtype)
    n = _mlp_bytes(dims, act, dt)
    st = lib.tp_mlp_fwd(ctypes.byref(dims), int(rank), _act(act), dt, _ptr(X, n["act"], "X"), _ptr(A_i, n["a"], "A_i"),
                        _ptr(a_i, n["aN"], "a_i"), _ptr(B_i, n["b"], "B_i"), _ptr(U_i, n["u"], "U_i"),
                        _ptr(Y_i, n["y"], "Y_i"), _ptr(Z_i, n["act"], "Z_i"), _stream(stream))
    return _check(st, "tp_mlp_fwd", check)


def tp_mlp_bwd(dims: tp_dims, rank: int, act, X, A_i, B_i, U_i, Y_i, dZ, dU_ws, dA_i, da_i, dB_i, dX_i,
               stream=None, dtype=None, check=True) -> int:
    return tp_mlp_bwd_phase(dims, rank, act, "all", X, A_i, B_i, U_i, Y_i, dZ, dU_ws, dA_i, da_i, dB_i, dX_i,
                            stream=stream, dtype=_dtype_code(X, dtype), check=check, _name="tp_mlp_bwd")


def tp_mlp_bwd_phase(dims: tp_dims, rank: int, act, phase, X, A_i, B_i, U_i, Y_i, dZ, dU_ws, dA_i, da_i, dB_i, dX_i,
                     stream=None, dtype=None, check=True, _name="tp_mlp_bwd_phase") -> int:
    ph = BWD_PHASES[phase] if isinstance(phase, str) else int(phase)
    dt = _dtype_code(dZ, dtype)
    n = _mlp_bytes(dims, act, dt)
    args = (ctypes.byref(dims), int(rank), _act(act), dt)
    ptrs = (_ptr(X, n["act"], "X"), _ptr(A_i, n["a"], "A_i"), _ptr(B_i, n["b"], "B_i"), _ptr(U_i, n["u"], "U_i"),
            _ptr(Y_i, n["y"], "Y_i"), _ptr(dZ, n["act"], "dZ"), _ptr(dU_ws, n["u"], "dU_ws"),
            _ptr(dA_i, n["a"], "dA_i"), _ptr(da_i, n["aN"], "da_i"), _ptr(dB_i, n["b"], "dB_i"),
            _ptr(dX_i, n["act"], "dX_i"))
    if _name == "tp_mlp_bwd":
        st = lib.tp_mlp_bwd(*args, *ptrs, _stream(stream))
    else:
        st = lib.tp_mlp_bwd_phase(*args, ph, *ptrs, _stream(stream))
    return _check(st, _name, check)


def _attn_bytes(dims: tp_dims, dt: int):
    """Bytes of the attention tensors: X / dZ / Z_i / dX_i, Wqkv_i, bqkv_i, Wo_i, QKV_i, O_i, lse_i."""
    es, t = _es(dt), max(int(dims.t), 1)
    M, h, a, d = dims.s * dims.b, dims.h, dims.a, dims.d
    g = dims.g or a
    if not _pos(M, h, a, d, g) or a % t or g % t:
        return dict(act=0, wq=0, bq=0, wo=0, qkv=0, o=0, lse=0)
    nq = (a // t + 2 * g // t) * d
    return dict(act=M * h * es, wq=h * nq * es, bq=nq * es, wo=a // t * d * h * es, qkv=M * nq * es,
                o=M * a // t * d * es, lse=dims.b * (a // t) * dims.s * 4)


def tp_attn_fwd(dims: tp_dims, rank: int, causal: bool, X, Wqkv_i, bqkv_i, Wo_i, QKV_i, O_i, lse_i, Z_i,
                stream=None, dtype=None, check=True) -> int:
    dt = _dtype_code(X, dtype)
    n = _attn_bytes(dims, dt)
    st = lib.tp_attn_fwd(ctypes.byref(dims), int(rank), dt, 1 if causal else 0, _ptr(X, n["act"], "X"),
                         _ptr(Wqkv_i, n["wq"], "Wqkv_i"), _ptr(bqkv_i, n["bq"], "bqkv_i"), _ptr(Wo_i, n["wo"], "Wo_i"),
                         _ptr(QKV_i, n["qkv"], "QKV_i"), _ptr(O_i, n["o"], "O_i"), _ptr(lse_i, n["lse"], "lse_i"),
                         _ptr(Z_i, n["act"], "Z_i"), _stream(stream))
    return _check(st, "tp_attn_fwd", check)


def tp_attn_bwd(dims: tp_dims, rank: int, causal: bool, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dZ, dO_ws, rec_ws, dQKV_i,
                dWqkv_i, dbqkv_i, dWo_i, dX_i, stream=None, dtype=None, check=True) -> int:
    dt = _dtype_code(X, dtype)
    n = _attn_bytes(dims, dt)
    ws = max(tp_attn_bwd_workspace(dims), 0)
    st = lib.tp_attn_bwd(ctypes.byref(dims), int(rank), dt, 1 if causal else 0, _ptr(X, n["act"], "X"),
                         _ptr(Wqkv_i, n["wq"], "Wqkv_i"), _ptr(Wo_i, n["wo"], "Wo_i"), _ptr(QKV_i, n["qkv"], "QKV_i"),
                         _ptr(O_i, n["o"], "O_i"), _ptr(lse_i, n["lse"], "lse_i"), _ptr(dZ, n["act"], "dZ"),
                         _ptr(dO_ws, n["o"], "dO_ws"), _ptr(rec_ws, ws, "rec_ws"), _ptr(dQKV_i, n["qkv"], "dQKV_i"),
                         _ptr(dWqkv_i, n["wq"], "dWqkv_i"), _ptr(dbqkv_i, n["bq"], "dbqkv_i"),
                         _ptr(dWo_i, n["wo"], "dWo_i"), _ptr(dX_i, n["act"], "dX_i"), _stream(stream))
    return _check(st, "tp_attn_bwd", check)


def tp_attn_bwd_workspace(dims: tp_dims) -> int:
    """Bytes of the rec_ws workspace tp_attn_bwd needs (0 for invalid dims)."""
    return int(lib.tp_attn_bwd_workspace(ctypes.byref(dims)))


def tp_partial_reduce(n: int, h: int, t: int, partials, bias_c, out, stream=None, dtype=None, check=True) -> int:
    dt = _dtype_code(partials, dtype)
    es, ok = _es(dt), _pos(n, h, t)
    st = lib.tp_partial_reduce(int(n), int(h), int(t), dt, _ptr(partials, t * n * es if ok else 0, "partials"),
                               _ptr(bias_c, h * es if ok else 0, "bias_c"), _ptr(out, n * es if ok else 0, "out"),
                               _stream(stream))
    return _check(st, "tp_partial_reduce", check)


def tp_reduce_scatter_dim0(dims: tp_dims, rank: int, partials, bias_c, out, stream=None, dtype=None,
                           check=True) -> int:
    dt = _dtype_code(partials, dtype)
    es, t = _es(dt), int(dims.t)
    ok = _pos(dims.s, dims.b, dims.h, t) and dims.s % t == 0
    n = dims.s * dims.b * dims.h if ok else 0
    st = lib.tp_reduce_scatter_dim0(ctypes.byref(dims), int(rank), dt, _ptr(partials, t * n * es, "partials"),
                                    _ptr(bias_c, dims.h * es if ok else 0, "bias_c"),
                                    _ptr(out, (n if rank < 0 else n // max(t, 1)) * es, "out"), _stream(stream))
    return _check(st, "tp_reduce_scatter_dim0", check)


def tp_gather_dim0(dims: tp_dims, slices, out, stream=None, dtype=None, check=True) -> int:
    dt = _dtype_code(slices, dtype)
    nb = dims.s * dims.b * dims.h * _es(dt) if _pos(dims.s, dims.b, dims.h) else 0
    st = lib.tp_gather_dim0(ctypes.byref(dims), dt, _ptr(slices, nb, "slices"), _ptr(out, nb, "out"),
                            _stream(stream))
    return _check(st, "tp_gather_dim0", check)


def _sp_bytes(rows: int, h: int, dt: int):
    es = _es(dt)
    if not _pos(rows, h):
        return dict(x=0, w=0, bits=0, stat=0, mask=0, f=0)
    return dict(x=rows * h * es, w=h * es, bits=rows * h * 4, stat=rows * 4, mask=rows * (h // 8), f=h * 4)


def tp_sp_dropout_add_ln_fwd(rows: int, h: int, p: float, eps: float, z, residual, bits, gamma, beta, out, y, mean,
                             rstd, mask, stream=None, dtype=None, check=True) -> int:
    dt = _dtype_code(z, dtype)
    n = _sp_bytes(rows, h, dt)
    st = lib.tp_sp_dropout_add_ln_fwd(int(rows), int(h), dt, float(p), float(eps), _ptr(z, n["x"], "z"),
                                      _ptr(residual, n["x"], "residual"), _ptr(bits, n["bits"], "bits"),
                                      _ptr(gamma, n["w"], "gamma"), _ptr(beta, n["w"], "beta"),
                                      _ptr(out, n["x"], "out"), _ptr(y, n["x"], "y"), _ptr(mean, n["stat"], "mean"),
                                      _ptr(rstd, n["stat"], "rstd"), _ptr(mask, n["mask"], "mask"), _stream(stream))
    return _check(st, "tp_sp_dropout_add_ln_fwd", check)


def _sp_bwd_ptrs(rows, h, dt, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz, dgamma, dbeta):
    n = _sp_bytes(rows, h, dt)
    return (_ptr(u, n["x"], "u"), _ptr(gamma, n["w"], "gamma"), _ptr(mean, n["stat"], "mean"),
            _ptr(rstd, n["stat"], "rstd"), _ptr(dy, n["x"], "dy"), _ptr(dres_in, n["x"], "dres_in"),
            _ptr(mask, n["mask"], "mask"), _ptr(dres, n["x"], "dres"), _ptr(dz, n["x"], "dz"),
            _ptr(dgamma, n["f"], "dgamma"), _ptr(dbeta, n["f"], "dbeta"))


def tp_sp_dropout_add_ln_bwd(rows: int, h: int, p: float, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz, dgamma,
                             dbeta, ws, stream=None, dtype=None, check=True) -> int:
    dt = _dtype_code(u, dtype)
    ptrs = _sp_bwd_ptrs(rows, h, dt, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz, dgamma, dbeta)
    st = lib.tp_sp_dropout_add_ln_bwd(int(rows), int(h), dt, float(p), *ptrs,
                                      _ptr(ws, max(tp_sp_ln_bwd_workspace(rows, h), 0), "ws"), _stream(stream))
    return _check(st, "tp_sp_dropout_add_ln_bwd", check)


def tp_sp_dropout_add_ln_bwd_noalloc(rows: int, h: int, p: float, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz,
                                     dgamma, dbeta, stream=None, dtype=None, check=True) -> int:
    dt = _dtype_code(u, dtype)
    ptrs = _sp_bwd_ptrs(rows, h, dt, u, gamma, mean, rstd, dy, dres_in, mask, dres, dz, dgamma, dbeta)
    st = lib.tp_sp_dropout_add_ln_bwd_noalloc(int(rows), int(h), dt, float(p), *ptrs, _stream(stream))
    return _check(st, "tp_sp_dropout_add_ln_bwd_noalloc", check)


def tp_sp_ln_bwd_workspace(rows: int, h: int) -> int:
    return int(lib.tp_sp_ln_bwd_workspace(int(rows), int(h)))


def tp_vocab_ce_fwd_local(rows: int, v_local: int, rank: int, logits_i, targets, stats_i, stream=None, dtype=None,
                          check=True) -> int:
    dt = _dtype_code(logits_i, dtype)
    ok = _pos(rows, v_local)
    st = lib.tp_vocab_ce_fwd_local(int(rows), int(v_local), int(rank), dt,
                                   _ptr(logits_i, rows * v_local * _es(dt) if ok else 0, "logits_i"),
                                   _ptr(targets, rows * 4 if ok else 0, "targets"),
                                   _ptr(stats_i, rows * 16 if ok else 0, "stats_i"), _stream(stream))
    return _check(st, "tp_vocab_ce_fwd_local", check)


def tp_vocab_ce_combine(rows: int, t: int, stats, targets, loss, lse, stream=None, check=True) -> int:
    ok = _pos(rows, t)
    st = lib.tp_vocab_ce_combine(int(rows), int(t), _ptr(stats, t * rows * 16 if ok else 0, "stats"),
                                 _ptr(targets, rows * 4 if ok else 0, "targets"),
                                 _ptr(loss, rows * 4 if ok else 0, "loss"), _ptr(lse, rows * 4 if ok else 0, "lse"),
                                 _stream(stream))
    return _check(st, "tp_vocab_ce_combine", check)


def tp_vocab_ce_bwd(rows: int, v_local: int, rank: int, logits_i, targets, lse, dloss, dlogits_i, stream=None,
                    dtype=None, check=True) -> int:
    dt = _dtype_code(logits_i, dtype)
    ok = _pos(rows, v_local)
    nb = rows * v_local * _es(dt) if ok else 0
    st = lib.tp_vocab_ce_bwd(int(rows), int(v_local), int(rank), dt, _ptr(logits_i, nb, "logits_i"),
                             _ptr(targets, rows * 4 if ok else 0, "targets"), _ptr(lse, rows * 4 if ok else 0, "lse"),
                             _ptr(dloss, rows * 4 if ok else 0, "dloss"), _ptr(dlogits_i, nb, "dlogits_i"),
                             _stream(stream))
    return _check(st, "tp_vocab_ce_bwd", check)


def tp_vocab_logits_fwd(rows: int, h: int, v_local: int, X, E_i, logits_i, stream=None, dtype=None,
                        check=True) -> int:
    dt = _dtype_code(X, dtype)
    es, ok = _es(dt), _pos(rows, h, v_local)
    st = lib.tp_vocab_logits_fwd(int(rows), int(h), int(v_local), dt, _ptr(X, rows * h * es if ok else 0, "X"),
                                 _ptr(E_i, v_local * h * es if ok else 0, "E_i"),
                                 _ptr(logits_i, rows * v_local * es if ok else 0, "logits_i"), _stream(stream))
    return _check(st, "tp_vocab_logits_fwd", check)


def tp_vocab_logits_bwd(rows: int, h: int, v_local: int, X, E_i, dlogits_i, dX_i, dE_i, stream=None, dtype=None,
                        check=True) -> int:
    dt = _dtype_code(dlogits_i, dtype)
    es, ok = _es(dt), _pos(rows, h, v_local)
    st = lib.tp_vocab_logits_bwd(int(rows), int(h), int(v_local), dt, _ptr(X, rows * h * es if ok else 0, "X"),
                                 _ptr(E_i, v_local * h * es if ok else 0, "E_i"),
                                 _ptr(dlogits_i, rows * v_local * es if ok else 0, "dlogits_i"),
                                 _ptr(dX_i, rows * h * es if ok else 0, "dX_i"),
                                 _ptr(dE_i, v_local * h * es if ok else 0, "dE_i"), _stream(stream))
    return _check(st, "tp_vocab_logits_bwd", check)


def tp_ln_fold_weights(dims: tp_dims, act, gamma, beta, A_i, a_i, A_ln, c_ln, b_ln, stream=None, dtype=None,
                       check=True) -> int:
    dt = _dtype_code(A_i, dtype)
    n = _mlp_bytes(dims, act, dt)
    nN = n["aN"] // 2 if _es(dt) else 0  # N1 elements
    hb = dims.h * _es(dt) if _pos(dims.h) else 0
    st = lib.tp_ln_fold_weights(ctypes.byref(dims), _act(act), dt, _ptr(gamma, hb, "gamma"), _ptr(beta, hb, "beta"),
                                _ptr(A_i, n["a"], "A_i"), _ptr(a_i, n["aN"], "a_i"), _ptr(A_ln, n["a"], "A_ln"),
                                _ptr(c_ln, nN * 4, "c_ln"), _ptr(b_ln, nN * 4, "b_ln"), _stream(stream))
    return _check(st, "tp_ln_fold_weights", check)


def tp_ln_mlp_fwd(dims: tp_dims, rank: int, act, X, ln_mean, ln_rstd, A_ln, c_ln, b_ln, B_i, U_i, Y_i, Z_i,
                  stream=None, dtype=None, check=True) -> int:
    dt = _dtype_code(X, dtype)
    n = _mlp_bytes(dims, act, dt)
    nN = n["aN"] // 2 if _es(dt) else 0
    rows = dims.s * dims.b if _pos(dims.s, dims.b) else 0
    st = lib.tp_ln_mlp_fwd(ctypes.byref(dims), int(rank), _act(act), dt, _ptr(X, n["act"], "X"),
                           _ptr(ln_mean, rows * 4, "ln_mean"), _ptr(ln_rstd, rows * 4, "ln_rstd"),
                           _ptr(A_ln, n["a"], "A_ln"), _ptr(c_ln, nN * 4, "c_ln"), _ptr(b_ln, nN * 4, "b_ln"),
                           _ptr(B_i, n["b"], "B_i"), _ptr(U_i, n["u"], "U_i"), _ptr(Y_i, n["y"], "Y_i"),
                           _ptr(Z_i, n["act"], "Z_i"), _stream(stream))
    return _check(st, "tp_ln_mlp_fwd", check)


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
