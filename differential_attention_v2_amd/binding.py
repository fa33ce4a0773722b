"""Thin ctypes binding over libdiffattn (argument marshalling only).

The raw functions carry the C names and arguments one to one.  ``prefill``,
``decode`` and ``v1_lambda`` are conveniences over torch tensors: they check
device, dtype, shape and contiguity, allocate outputs/workspace with torch (torch
is only the memory and stream provider) and pass raw pointers plus the current
HIP stream.  Every step of the computation runs in the library's kernels; if the
library is missing this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# DIFFATTN_LIBRARY may name another build of the same library (for example a
# sanitizer build of the host layer); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("DIFFATTN_LIBRARY") or os.path.join(PKG, "libdiffattn.so")

DIFFATTN_OK = 0
DIFFATTN_ERR_INVALID_ARG = 1
DIFFATTN_ERR_UNSUPPORTED = 2
DIFFATTN_ERR_WORKSPACE = 3
DIFFATTN_ERR_HIP = 4
DIFFATTN_BF16 = 0
DIFFATTN_FP32 = 1
DIFFATTN_FLAG_V1_RMSNORM = 0x1
DIFFATTN_NOALLOC_SCRATCH_BYTES = 32 << 20

_c_int, _c_uint, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_uint, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "diffattn_prefill_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                      _c_int, _c_uint, _c_float, _vp]),
    "diffattn_decode_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_int, _c_uint, _c_float, _c_int, _vp, _c_size, _vp]),
    "diffattn_decode_fwd_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_int, _c_uint, _c_float, _c_int, _vp]),
    "diffattn_prefill_fwd_window": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _c_uint, _c_float, _vp]),
    "diffattn_decode_fwd_varlen": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_int, _c_uint, _c_float, _c_int, _vp, _c_size, _vp]),
    "diffattn_prefill_fwd_train": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_int, _vp]),
    "diffattn_prefill_bwd": (_c_int, [_vp] * 12 + [_c_int] * 6 + [_vp, _c_size, _vp]),
    "diffattn_prefill_bwd_workspace_bytes": (_c_size, [_c_int] * 5),
    "diffattn_decode_varlen_workspace_bytes": (_c_size, [_c_int] * 6),
    "diffattn_decode_standard": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 6 + [_vp, _c_size, _vp]),
    "diffattn_decode_v1_layout": (_c_int, [_vp] * 5 + [_c_int] * 5 + [_c_uint, _c_float, _c_int, _vp, _c_size, _vp]),
    "diffattn_decode_compare_workspace_bytes": (_c_size, [_c_int] * 6),
    "diffattn_lambda_proj": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "diffattn_output_proj": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "diffattn_decode_num_splits": (_c_int, [_c_int] * 5),
    "diffattn_decode_workspace_bytes": (_c_size, [_c_int] * 6),
    "diffattn_v1_lambda": (_c_int, [_vp, _vp, _vp, _vp, _c_float, _vp, _c_int, _c_int, _c_int, _vp]),
    "diffattn_status_string": (ctypes.c_char_p, [_c_int]),
    "diffattn_version": (_c_int, []),
}

_lib = None


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: libdiffattn status {status} ({status_string(status)})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdiffattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m differential_attention_v2_amd.build_lib` "
                               "(or __graft_entry__.build()); there is no fallback path")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


# ---- raw C entry points, same names and arguments as include/diffattn.h ----
def diffattn_prefill_fwd(q, k, v, lam, out, B, T, Hq, Hkv, d, causal, dtype, flags, rms_eps, stream):
    return load_library().diffattn_prefill_fwd(q, k, v, lam, out, B, T, Hq, Hkv, d, causal, dtype, flags,
                                               rms_eps, stream)


def diffattn_decode_fwd(q, k_cache, v_cache, lam, out, B, L, Hq, Hkv, d, dtype, flags, rms_eps, num_splits,
                        workspace, workspace_bytes, stream):
    return load_library().diffattn_decode_fwd(q, k_cache, v_cache, lam, out, B, L, Hq, Hkv, d, dtype, flags,
                                              rms_eps, num_splits, workspace, workspace_bytes, stream)


def diffattn_decode_fwd_noalloc(q, k_cache, v_cache, lam, out, B, L, Hq, Hkv, d, dtype, flags, rms_eps, num_splits,
                                stream):
    return load_library().diffattn_decode_fwd_noalloc(q, k_cache, v_cache, lam, out, B, L, Hq, Hkv, d, dtype, flags,
                                                      rms_eps, num_splits, stream)


def diffattn_prefill_fwd_window(q, k, v, lam, out, B, T, Hq, Hkv, d, window, dtype, flags, rms_eps, stream):
    return load_library().diffattn_prefill_fwd_window(q, k, v, lam, out, B, T, Hq, Hkv, d, window, dtype, flags,
                                                      rms_eps, stream)


def diffattn_decode_fwd_varlen(q, k_cache, v_cache, lam, out, seq_lens, B, L, Hq, Hkv, d, window, dtype, flags,
                               rms_eps, num_splits, workspace, workspace_bytes, stream):
    return load_library().diffattn_decode_fwd_varlen(q, k_cache, v_cache, lam, out, seq_lens, B, L, Hq, Hkv, d,
                                                     window, dtype, flags, rms_eps, num_splits, workspace,
                                                     workspace_bytes, stream)


def diffattn_prefill_fwd_train(q, k, v, lam, out, o2, lse, B, T, Hq, Hkv, d, causal, stream):
    return load_library().diffattn_prefill_fwd_train(q, k, v, lam, out, o2, lse, B, T, Hq, Hkv, d, causal, stream)


def diffattn_prefill_bwd(q, k, v, lam, out, o2, lse, dout, dq, dk, dv, dlam, B, T, Hq, Hkv, d, causal,
                         workspace, workspace_bytes, stream):
    return load_library().diffattn_prefill_bwd(q, k, v, lam, out, o2, lse, dout, dq, dk, dv, dlam, B, T, Hq, Hkv,
                                               d, causal, workspace, workspace_bytes, stream)


def diffattn_prefill_bwd_workspace_bytes(B, T, Hq, Hkv, d):
    return load_library().diffattn_prefill_bwd_workspace_bytes(B, T, Hq, Hkv, d)


def diffattn_decode_varlen_workspace_bytes(B, L, Hq, Hkv, d, num_splits=0):
    return load_library().diffattn_decode_varlen_workspace_bytes(B, L, Hq, Hkv, d, num_splits)


def diffattn_decode_standard(q, k_cache, v_cache, out, B, L, H, Hkv, d, num_splits, workspace, workspace_bytes,
                             stream):
    return load_library().diffattn_decode_standard(q, k_cache, v_cache, out, B, L, H, Hkv, d, num_splits, workspace,
                                                   workspace_bytes, stream)


def diffattn_decode_v1_layout(q, k_cache, v_cache, lam, out, B, L, H, Hkv, d, flags, rms_eps, num_splits, workspace,
                              workspace_bytes, stream):
    return load_library().diffattn_decode_v1_layout(q, k_cache, v_cache, lam, out, B, L, H, Hkv, d, flags, rms_eps,
                                                    num_splits, workspace, workspace_bytes, stream)


def diffattn_decode_compare_workspace_bytes(B, L, H, Hkv, d, num_splits=0):
    return load_library().diffattn_decode_compare_workspace_bytes(B, L, H, Hkv, d, num_splits)


def diffattn_lambda_proj(x, w_lambda, lambda_out, rows, d_model, P, stream):
    return load_library().diffattn_lambda_proj(x, w_lambda, lambda_out, rows, d_model, P, stream)


def diffattn_output_proj(attn, w_o, y, rows, in_dim, out_dim, stream):
    return load_library().diffattn_output_proj(attn, w_o, y, rows, in_dim, out_dim, stream)


def diffattn_decode_num_splits(B, L, Hq, Hkv, d):
    return load_library().diffattn_decode_num_splits(B, L, Hq, Hkv, d)


def diffattn_decode_workspace_bytes(B, L, Hq, Hkv, d, num_splits=0):
    return load_library().diffattn_decode_workspace_bytes(B, L, Hq, Hkv, d, num_splits)


def diffattn_v1_lambda(lq1, lk1, lq2, lk2, lambda_init, lambda_out, P, d_lambda, rows, stream):
    return load_library().diffattn_v1_lambda(lq1, lk1, lq2, lk2, lambda_init, lambda_out, P, d_lambda, rows,
                                             stream)


def diffattn_status_string(status):
    return load_library().diffattn_status_string(status)


def diffattn_version():
    return load_library().diffattn_version()


def status_string(status: int) -> str:
    return diffattn_status_string(status).decode()


# ---- torch conveniences ----
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DIFFATTN_BF16
    if t.dtype == torch.float32:
        return DIFFATTN_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32")


def _check(t, name, shape, dtype):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def prefill(q, k, v, lam, causal: bool = True, v1_rmsnorm: bool = False, eps: float = 1e-5, out=None,
            stream=None):
    """out [B, T, P, d] = DiffAttn V2 prefill of q [B,T,Hq,d], k/v [B,T,Hkv,d], lam [B,T,P] (fp32)."""
    torch = _torch()
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    _check(q, "q", (B, T, Hq, d), q.dtype)
    _check(k, "k", (B, T, Hkv, d), q.dtype)
    _check(v, "v", (B, T, Hkv, d), q.dtype)
    _check(lam, "lam", (B, T, Hq // 2), torch.float32)
    if out is None:
        out = torch.empty((B, T, Hq // 2, d), dtype=q.dtype, device=q.device)
    _check(out, "out", (B, T, Hq // 2, d), q.dtype)
    st = diffattn_prefill_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(), out.data_ptr(), B, T, Hq,
                              Hkv, d, int(bool(causal)), _dtype_code(q),
                              DIFFATTN_FLAG_V1_RMSNORM if v1_rmsnorm else 0, float(eps), _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_prefill_fwd")
    return out


def prefill_window(q, k, v, lam, window: int, v1_rmsnorm: bool = False, eps: float = 1e-5, out=None,
                   stream=None):
    """out [B, T, P, d]: causal prefill where each query sees its last `window` keys (bf16)."""
    torch = _torch()
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    _check(q, "q", (B, T, Hq, d), torch.bfloat16)
    _check(k, "k", (B, T, Hkv, d), torch.bfloat16)
    _check(v, "v", (B, T, Hkv, d), torch.bfloat16)
    _check(lam, "lam", (B, T, Hq // 2), torch.float32)
    if out is None:
        out = torch.empty((B, T, Hq // 2, d), dtype=q.dtype, device=q.device)
    _check(out, "out", (B, T, Hq // 2, d), q.dtype)
    st = diffattn_prefill_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(), out.data_ptr(), B, T,
                                     Hq, Hkv, d, int(window), DIFFATTN_BF16,
                                     DIFFATTN_FLAG_V1_RMSNORM if v1_rmsnorm else 0, float(eps), _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_prefill_fwd_window")
    return out


def decode_varlen(q, k_cache, v_cache, lam, seq_lens=None, window: int = 0, v1_rmsnorm: bool = False,
                  eps: float = 1e-5, num_splits: int = 0, workspace=None, out=None, stream=None):
    """out [B, P, d]: decode over caches with seq_lens[b] valid rows (int32 device tensor or None)."""
    torch = _torch()
    B, Hq, d = q.shape
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(q, "q", (B, Hq, d), torch.bfloat16)
    _check(k_cache, "k_cache", (B, L, Hkv, d), torch.bfloat16)
    _check(v_cache, "v_cache", (B, L, Hkv, d), torch.bfloat16)
    _check(lam, "lam", (B, Hq // 2), torch.float32)
    if seq_lens is not None:
        _check(seq_lens, "seq_lens", (B,), torch.int32)
    if out is None:
        out = torch.empty((B, Hq // 2, d), dtype=q.dtype, device=q.device)
    _check(out, "out", (B, Hq // 2, d), q.dtype)
    if workspace is None:
        workspace = torch.empty(diffattn_decode_varlen_workspace_bytes(B, L, Hq, Hkv, d, num_splits),
                                dtype=torch.uint8, device=q.device)
    st = diffattn_decode_fwd_varlen(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lam.data_ptr(),
                                    out.data_ptr(), None if seq_lens is None else seq_lens.data_ptr(), B, L, Hq,
                                    Hkv, d, int(window), DIFFATTN_BF16, DIFFATTN_FLAG_V1_RMSNORM if v1_rmsnorm else 0,
                                    float(eps), int(num_splits), workspace.data_ptr(), workspace.numel(),
                                    _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_decode_fwd_varlen")
    return out


def decode_standard(q, k_cache, v_cache, num_splits: int = 0, workspace=None, out=None, stream=None):
    """out [B, H, d]: standard-transformer decode (one softmax per head) over bf16 caches."""
    torch = _torch()
    B, H, d = q.shape
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(q, "q", (B, H, d), torch.bfloat16)
    _check(k_cache, "k_cache", (B, L, Hkv, d), torch.bfloat16)
    _check(v_cache, "v_cache", (B, L, Hkv, d), torch.bfloat16)
    if out is None:
        out = torch.empty((B, H, d), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = torch.empty(diffattn_decode_compare_workspace_bytes(B, L, H, Hkv, d, num_splits),
                                dtype=torch.uint8, device=q.device)
    st = diffattn_decode_standard(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), B, L, H, Hkv,
                                  d, int(num_splits), workspace.data_ptr(), workspace.numel(), _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_decode_standard")
    return out


def decode_v1_layout(q, k_cache, v_cache, lam, v1_rmsnorm: bool = True, eps: float = 1e-5, num_splits: int = 0,
                     workspace=None, out=None, stream=None):
    """out [B, H, d]: DIFF V1 decode (q, k split into halves per branch, V read once per branch)."""
    torch = _torch()
    B, H, d = q.shape
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(q, "q", (B, H, d), torch.bfloat16)
    _check(k_cache, "k_cache", (B, L, Hkv, d), torch.bfloat16)
    _check(v_cache, "v_cache", (B, L, Hkv, d), torch.bfloat16)
    _check(lam, "lam", (B, H), torch.float32)
    if out is None:
        out = torch.empty((B, H, d), dtype=q.dtype, device=q.device)
    if workspace is None:
        workspace = torch.empty(diffattn_decode_compare_workspace_bytes(B, L, H, Hkv, d, num_splits),
                                dtype=torch.uint8, device=q.device)
    st = diffattn_decode_v1_layout(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lam.data_ptr(),
                                   out.data_ptr(), B, L, H, Hkv, d, DIFFATTN_FLAG_V1_RMSNORM if v1_rmsnorm else 0,
                                   float(eps), int(num_splits), workspace.data_ptr(), workspace.numel(),
                                   _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_decode_v1_layout")
    return out


def lambda_proj(x, w_lambda, out=None, stream=None):
    """lambda [rows, P] fp32 = sigmoid(x [rows, d_model] @ w_lambda [P, d_model]^T), bf16 inputs."""
    torch = _torch()
    rows, dm = x.shape
    P = w_lambda.shape[0]
    _check(x, "x", (rows, dm), torch.bfloat16)
    _check(w_lambda, "w_lambda", (P, dm), torch.bfloat16)
    if out is None:
        out = torch.empty((rows, P), dtype=torch.float32, device=x.device)
    _check(out, "out", (rows, P), torch.float32)
    st = diffattn_lambda_proj(x.data_ptr(), w_lambda.data_ptr(), out.data_ptr(), rows, dm, P, _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_lambda_proj")
    return out


def output_proj(attn, w_o, out=None, stream=None):
    """y [rows, out_dim] = attn [rows, in_dim] @ w_o [in_dim, out_dim], bf16 (the library's MFMA GEMM;
    in_dim % 32 == 0, out_dim % 8 == 0)."""
    torch = _torch()
    rows, kin = attn.shape
    nout = w_o.shape[1]
    _check(attn, "attn", (rows, kin), torch.bfloat16)
    _check(w_o, "w_o", (kin, nout), torch.bfloat16)
    if out is None:
        out = torch.empty((rows, nout), dtype=torch.bfloat16, device=attn.device)
    _check(out, "out", (rows, nout), torch.bfloat16)
    st = diffattn_output_proj(attn.data_ptr(), w_o.data_ptr(), out.data_ptr(), rows, kin, nout, _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_output_proj")
    return out


def prefill_train(q, k, v, lam, causal: bool = True, out=None, stream=None):
    """(out, o2, lse) of the bf16 training forward: out [B,T,P,d], o2 [B,T,P,d], lse [B,T,Hq] fp32.
    `out` may pass the three output tensors to fill."""
    torch = _torch()
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    _check(q, "q", (B, T, Hq, d), torch.bfloat16)
    _check(k, "k", (B, T, Hkv, d), torch.bfloat16)
    _check(v, "v", (B, T, Hkv, d), torch.bfloat16)
    _check(lam, "lam", (B, T, Hq // 2), torch.float32)
    if out is None:
        out = (torch.empty((B, T, Hq // 2, d), dtype=q.dtype, device=q.device),
               torch.empty((B, T, Hq // 2, d), dtype=q.dtype, device=q.device),
               torch.empty((B, T, Hq), dtype=torch.float32, device=q.device))
    out, o2, lse = out
    _check(out, "out", (B, T, Hq // 2, d), torch.bfloat16)
    _check(o2, "o2", (B, T, Hq // 2, d), torch.bfloat16)
    _check(lse, "lse", (B, T, Hq), torch.float32)
    st = diffattn_prefill_fwd_train(q.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(), out.data_ptr(),
                                    o2.data_ptr(), lse.data_ptr(), B, T, Hq, Hkv, d, int(bool(causal)),
                                    _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_prefill_fwd_train")
    return out, o2, lse


def prefill_backward(q, k, v, lam, out, o2, lse, dout, causal: bool = True, workspace=None, grads=None,
                     stream=None):
    """(dq, dk, dv, dlam) of L = sum(dout * out) for the bf16 prefill map."""
    torch = _torch()
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    P = Hq // 2
    _check(q, "q", (B, T, Hq, d), torch.bfloat16)
    _check(k, "k", (B, T, Hkv, d), torch.bfloat16)
    _check(v, "v", (B, T, Hkv, d), torch.bfloat16)
    _check(lam, "lam", (B, T, P), torch.float32)
    for name, t in (("out", out), ("o2", o2), ("dout", dout)):
        _check(t, name, (B, T, P, d), torch.bfloat16)
    _check(lse, "lse", (B, T, Hq), torch.float32)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(lam))
    dq, dk, dv, dlam = grads
    if workspace is None:
        n = diffattn_prefill_bwd_workspace_bytes(B, T, Hq, Hkv, d)
        if n == 0:
            raise ValueError("invalid backward sizes")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    st = diffattn_prefill_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), lam.data_ptr(), out.data_ptr(),
                              o2.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), dlam.data_ptr(), B, T, Hq, Hkv, d, int(bool(causal)),
                              workspace.data_ptr(), workspace.numel(), _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_prefill_bwd")
    return dq, dk, dv, dlam


def decode_workspace(B, L, Hq, Hkv, d, num_splits: int = 0, device="cuda"):
    torch = _torch()
    n = diffattn_decode_workspace_bytes(B, L, Hq, Hkv, d, num_splits)
    if n == 0:
        raise ValueError("invalid decode sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode(q, k_cache, v_cache, lam, v1_rmsnorm: bool = False, eps: float = 1e-5, num_splits: int = 0,
           workspace=None, out=None, stream=None):
    """out [B, P, d] = DiffAttn V2 decode of q [B,Hq,d] over caches [B,L,Hkv,d] with lam [B,P] (fp32)."""
    torch = _torch()
    B, Hq, d = q.shape
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(q, "q", (B, Hq, d), q.dtype)
    _check(k_cache, "k_cache", (B, L, Hkv, d), q.dtype)
    _check(v_cache, "v_cache", (B, L, Hkv, d), q.dtype)
    _check(lam, "lam", (B, Hq // 2), torch.float32)
    if out is None:
        out = torch.empty((B, Hq // 2, d), dtype=q.dtype, device=q.device)
    _check(out, "out", (B, Hq // 2, d), q.dtype)
    if workspace is None and q.dtype == torch.bfloat16:
        workspace = decode_workspace(B, L, Hq, Hkv, d, num_splits, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = diffattn_decode_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lam.data_ptr(), out.data_ptr(),
                             B, L, Hq, Hkv, d, _dtype_code(q), DIFFATTN_FLAG_V1_RMSNORM if v1_rmsnorm else 0,
                             float(eps), int(num_splits), ws_ptr, ws_bytes, _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_decode_fwd")
    return out


def decode_noalloc(q, k_cache, v_cache, lam, v1_rmsnorm: bool = False, eps: float = 1e-5, num_splits: int = 0,
                   out=None, stream=None):
    """decode() without a workspace: the key-range records use the library's fixed
    per-device scratch (diffattn_decode_fwd_noalloc; calls on one device must not
    overlap in time)."""
    torch = _torch()
    B, Hq, d = q.shape
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(q, "q", (B, Hq, d), q.dtype)
    _check(k_cache, "k_cache", (B, L, Hkv, d), q.dtype)
    _check(v_cache, "v_cache", (B, L, Hkv, d), q.dtype)
    _check(lam, "lam", (B, Hq // 2), torch.float32)
    if out is None:
        out = torch.empty((B, Hq // 2, d), dtype=q.dtype, device=q.device)
    _check(out, "out", (B, Hq // 2, d), q.dtype)
    st = diffattn_decode_fwd_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lam.data_ptr(),
                                     out.data_ptr(), B, L, Hq, Hkv, d, _dtype_code(q),
                                     DIFFATTN_FLAG_V1_RMSNORM if v1_rmsnorm else 0, float(eps), int(num_splits),
                                     _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_decode_fwd_noalloc")
    return out


def v1_lambda(lq1, lk1, lq2, lk2, lambda_init: float, rows: int, out=None, stream=None):
    """lambda [rows, P] = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init per pair, broadcast over rows."""
    torch = _torch()
    P, dl = lq1.shape
    for name, t in (("lq1", lq1), ("lk1", lk1), ("lq2", lq2), ("lk2", lk2)):
        _check(t, name, (P, dl), torch.float32)
    if out is None:
        out = torch.empty((rows, P), dtype=torch.float32, device=lq1.device)
    _check(out, "out", (rows, P), torch.float32)
    st = diffattn_v1_lambda(lq1.data_ptr(), lk1.data_ptr(), lq2.data_ptr(), lk2.data_ptr(), float(lambda_init),
                            out.data_ptr(), P, dl, rows, _stream(stream))
    if st != DIFFATTN_OK:
        raise DiffAttnError(st, "diffattn_v1_lambda")
    return out
