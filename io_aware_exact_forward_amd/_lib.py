"""ctypes binding of libfa_mi355x.so: the C entry points under their C names.

Argument marshalling only.  Every call goes to the HIP library; there is no
other implementation behind these names, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

FA_DTYPE_BF16 = 0
FA_DTYPE_F32 = 1

_STATUS_NAMES = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_HEAD_DIM",
    -4: "FA_ERR_DTYPE", -5: "FA_ERR_ALIGN", -6: "FA_ERR_SCALE", -7: "FA_ERR_ALIAS",
    -8: "FA_ERR_WORKSPACE", -9: "FA_ERR_HIP",
}

# Every symbol the header declares, with its ctypes signature.
_SIGNATURES = {
    "fa_forward": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "fa_naive_workspace_bytes": (ctypes.c_size_t, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "fa_naive_forward": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_split_workspace_bytes": (ctypes.c_size_t, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "fa_forward_split": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_forward_varlen": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "fa_backward_workspace_bytes": (ctypes.c_size_t, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "fa_backward": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_backward_dropout": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32,
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_backward_bias": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_backward_gqa": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
        ctypes.c_size_t, ctypes.c_void_p]),
    "fa_backward_varlen": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_naive_backward": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_forward_dropout": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32,
        ctypes.c_void_p]),
    "fa_forward_bias": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p]),
    "fa_forward_split_noalloc": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p]),
    "fa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fa_abi_version": (ctypes.c_int, []),
}

_lock = threading.Lock()
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib_path() -> str:
    return _build.lib_path()


def load() -> ctypes.CDLL:
    """Load the built library (building it first only if none is built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            _build.build()
        if not os.path.exists(path):
            raise FAError(-9, f"HIP library {path} is missing and could not be built")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def exported_symbols() -> list[str]:
    return list(_SIGNATURES)


def status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != 0:
        raise FAError(status, status_string(status))


def fa_forward(q, k, v, o, lse, B, H, N, d, scale, causal, key_len_mask, dtype, stream) -> int:
    """Raw C call; pointers and the stream are integers (0 = NULL)."""
    return load().fa_forward(q, k, v, o, lse, B, H, N, d, scale, int(causal),
                             key_len_mask or None, dtype, stream or None)


def fa_naive_workspace_bytes(B, H, N, dtype) -> int:
    return load().fa_naive_workspace_bytes(B, H, N, dtype)


def fa_naive_forward(q, k, v, o, lse, B, H, N, d, scale, causal, key_len_mask, dtype,
                     workspace, workspace_bytes, stream) -> int:
    return load().fa_naive_forward(q, k, v, o, lse, B, H, N, d, scale, int(causal),
                                   key_len_mask or None, dtype, workspace, workspace_bytes,
                                   stream or None)


def fa_split_workspace_bytes(B, H, Nq, Nk, d, num_splits) -> int:
    return load().fa_split_workspace_bytes(B, H, Nq, Nk, d, num_splits)


def fa_forward_split(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, key_len_mask, dtype,
                     num_splits, workspace, workspace_bytes, stream) -> int:
    return load().fa_forward_split(q or None, k or None, v or None, o or None, lse or None, B, H,
                                   Hkv, Nq, Nk, d, scale, int(causal), key_len_mask or None,
                                   dtype, num_splits, workspace or None, workspace_bytes,
                                   stream or None)


def fa_forward_varlen(q, k, v, o, lse, cu_q, cu_k, B, H, Hkv, total_q, total_k, max_q, max_k, d,
                      scale, causal, dtype, stream) -> int:
    return load().fa_forward_varlen(q or None, k or None, v or None, o or None, lse or None,
                                    cu_q or None, cu_k or None, B, H, Hkv, total_q, total_k,
                                    max_q, max_k, d, scale, int(causal), dtype, stream or None)


def fa_backward_workspace_bytes(B, H, N, d, dtype) -> int:
    return load().fa_backward_workspace_bytes(B, H, N, d, dtype)


def fa_backward(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, key_len_mask,
                dtype, workspace, workspace_bytes, stream) -> int:
    return load().fa_backward(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, int(causal),
                              key_len_mask or None, dtype, workspace or None, workspace_bytes,
                              stream or None)


def fa_backward_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                        key_len_mask, dtype, p_drop, seed, offset, workspace, workspace_bytes,
                        stream) -> int:
    return load().fa_backward_dropout(q or None, k or None, v or None, o or None, lse or None,
                                      dout or None, dq or None, dk or None, dv or None, B, H, N,
                                      d, scale, int(causal), key_len_mask or None, dtype,
                                      float(p_drop), int(seed), int(offset), workspace or None,
                                      workspace_bytes, stream or None)


def fa_backward_bias(q, k, v, o, lse, dout, dq, dk, dv, bias, B, H, N, d, scale, causal,
                     key_len_mask, dtype, bias_sb, bias_sh, bias_ld, workspace, workspace_bytes,
                     stream) -> int:
    return load().fa_backward_bias(q or None, k or None, v or None, o or None, lse or None,
                                   dout or None, dq or None, dk or None, dv or None, bias or None,
                                   B, H, N, d, scale, int(causal), key_len_mask or None, dtype,
                                   bias_sb, bias_sh, bias_ld, workspace or None, workspace_bytes,
                                   stream or None)


def fa_backward_gqa(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, Nq, Nk, d, scale, causal,
                    key_len_mask, dtype, workspace, workspace_bytes, stream) -> int:
    return load().fa_backward_gqa(q or None, k or None, v or None, o or None, lse or None,
                                  dout or None, dq or None, dk or None, dv or None, B, H, Hkv,
                                  Nq, Nk, d, scale, int(causal), key_len_mask or None, dtype,
                                  workspace or None, workspace_bytes, stream or None)


def fa_backward_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_q, cu_k, B, H, Hkv, total_q,
                       total_k, max_q, max_k, d, scale, causal, dtype, workspace,
                       workspace_bytes, stream) -> int:
    return load().fa_backward_varlen(q or None, k or None, v or None, o or None, lse or None,
                                     dout or None, dq or None, dk or None, dv or None,
                                     cu_q or None, cu_k or None, B, H, Hkv, total_q, total_k,
                                     max_q, max_k, d, scale, int(causal), dtype,
                                     workspace or None, workspace_bytes, stream or None)


def fa_naive_backward(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                      key_len_mask, dtype, workspace, workspace_bytes, stream) -> int:
    return load().fa_naive_backward(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale,
                                    int(causal), key_len_mask or None, dtype, workspace or None,
                                    workspace_bytes, stream or None)


def fa_forward_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, key_len_mask, dtype, p_drop,
                       seed, offset, stream) -> int:
    return load().fa_forward_dropout(q or None, k or None, v or None, o or None, lse or None, B, H,
                                     N, d, scale, int(causal), key_len_mask or None, dtype,
                                     p_drop, seed, offset, stream or None)


def fa_forward_bias(q, k, v, o, lse, bias, B, H, N, d, scale, causal, key_len_mask, dtype, sb,
                    sh, ld, stream) -> int:
    return load().fa_forward_bias(q or None, k or None, v or None, o or None, lse or None,
                                  bias or None, B, H, N, d, scale, int(causal),
                                  key_len_mask or None, dtype, sb, sh, ld, stream or None)


def fa_status_string(status) -> str:
    return status_string(status)


def fa_forward_split_noalloc(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, key_len_mask,
                             dtype, num_splits, stream) -> int:
    return load().fa_forward_split_noalloc(q or None, k or None, v or None, o or None,
                                           lse or None, B, H, Hkv, Nq, Nk, d, scale, int(causal),
                                           key_len_mask or None, dtype, num_splits,
                                           stream or None)


def fa_abi_version() -> int:
    return load().fa_abi_version()
