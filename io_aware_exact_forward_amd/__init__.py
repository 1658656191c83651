"""Exact attention forward for MI355X (gfx950): fused HIP kernels behind a C ABI.

The C entry points (include/fa_mi355x.h) are exposed under their own names by
``io_aware_exact_forward_amd._lib``; ``forward``, ``forward_split``,
``backward`` and ``naive_forward`` below are conveniences that take torch tensors (torch only provides device memory
and the stream), allocate the outputs and call those entry points.  Nothing
here computes attention itself.
"""
from __future__ import annotations

import math

from ._lib import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_F32,
    FAError,
    check,
    fa_abi_version,
    fa_backward,
    fa_backward_bias,
    fa_backward_dropout,
    fa_backward_gqa,
    fa_backward_varlen,
    fa_backward_workspace_bytes,
    fa_forward,
    fa_forward_split,
    fa_forward_split_noalloc,
    fa_forward_varlen,
    fa_forward_dropout,
    fa_forward_bias,
    fa_naive_backward,
    fa_naive_forward,
    fa_naive_workspace_bytes,
    fa_split_workspace_bytes,
    fa_status_string,
    load,
)

__all__ = [
    "forward", "forward_split", "backward", "naive_forward", "fa_forward", "fa_forward_split",
    "fa_forward_split_noalloc",
    "fa_backward", "fa_backward_workspace_bytes", "fa_naive_backward", "naive_backward",
    "fa_forward_varlen", "forward_varlen", "fa_forward_dropout", "forward_dropout",
    "fa_forward_bias", "forward_bias", "fa_backward_gqa", "backward_gqa", "fa_backward_varlen",
    "backward_varlen", "fa_backward_dropout", "backward_dropout",
    "fa_backward_bias", "backward_bias",
    "fa_split_workspace_bytes", "fa_naive_forward", "fa_naive_workspace_bytes",
    "fa_status_string", "fa_abi_version", "FAError", "FA_DTYPE_BF16", "FA_DTYPE_F32",
]


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise FAError(-4, f"unsupported dtype {t.dtype}")


def _output(t, shape, dtype, device, name):
    """A caller-supplied output (validated: its shape, dtype and device, and
    contiguous, since the C ABI cannot see buffer sizes), or a new tensor."""
    import torch
    if t is None:
        return torch.empty(tuple(shape), dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise FAError(-2, f"{name} must be {dtype} {tuple(shape)}; got {t.dtype} {tuple(t.shape)}")
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise FAError(-1, f"{name} must be a contiguous tensor on {device}")
    return t


def _workspace(ws, need, device):
    """(pointer, bytes) of a workspace: a new one of `need` bytes, or the
    caller's (a contiguous tensor on the device; its size in bytes)."""
    import torch
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    elif not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise FAError(-1, f"workspace must be a contiguous tensor on {device}")
    return ws, ws.data_ptr(), ws.numel() * ws.element_size()


def _same_device(device, *ts):
    for t in ts:
        if t is not None and t.device != device:
            raise FAError(-1, f"all tensors must be on {device}")


def _prepare(q, k, v, scale, key_len):
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise FAError(-2, f"q, k, v must share the shape [B, H, N, d]; got {tuple(q.shape)}, "
                          f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise FAError(-4, "q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise FAError(-1, "q, k, v must be contiguous device tensors")
    _same_device(q.device, k, v, key_len)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl = 0
    if key_len is not None:
        if key_len.dtype != torch.int32 or not key_len.is_cuda or key_len.numel() != B:
            raise FAError(-1, "key_len must be a device int32 tensor of B elements")
        if not key_len.is_contiguous():
            raise FAError(-1, "key_len must be contiguous")
        kl = key_len.data_ptr()
    return B, H, N, d, float(scale), kl


def forward(q, k, v, *, scale=None, causal=False, key_len=None, out=None, lse=None):
    """O, LSE = fa_forward(...) on torch's current stream of q's device."""
    import torch
    B, H, N, d, scale, kl = _prepare(q, k, v, scale, key_len)
    out = _output(out, q.shape, q.dtype, q.device, "out")
    lse = _output(lse, (B, H, N), torch.float32, q.device, "lse")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    check(fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     B, H, N, d, scale, int(bool(causal)), kl, _dtype_code(q), stream))
    return out, lse


def naive_forward(q, k, v, *, scale=None, causal=False, key_len=None, workspace=None):
    """Materialised three-pass baseline (S and P stored in device memory)."""
    import torch
    B, H, N, d, scale, kl = _prepare(q, k, v, scale, key_len)
    dt = _dtype_code(q)
    need = fa_naive_workspace_bytes(B, H, N, dt)
    workspace, ws, wsb = _workspace(workspace, need, q.device)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    check(fa_naive_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), B, H, N, d, scale, int(bool(causal)), kl, dt,
                           ws, wsb, stream))
    return out, lse


def forward_split(q, k, v, *, scale=None, causal=False, key_len=None, num_splits=0,
                  workspace=None, out=None, lse=None):
    """O, LSE = fa_forward_split(...): q [B, H, Nq, d] against k, v [B, H, Nk, d]
    (query row i at key position i + Nk - Nq), keys split into ranges that are
    merged by their log-sum-exp.  num_splits = 0 lets the library choose."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[0] != k.shape[0] \
            or q.shape[3] != k.shape[3] or k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise FAError(-2, f"q [B, H, Nq, d] and k, v [B, Hkv, Nk, d] (Hkv dividing H) expected; "
                          f"got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise FAError(-4, "q, k, v must share one dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise FAError(-1, "q, k, v must be contiguous device tensors")
    _same_device(q.device, k, v, key_len)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl = 0
    if key_len is not None:
        if key_len.dtype != torch.int32 or not key_len.is_cuda or key_len.numel() != B or \
                not key_len.is_contiguous():
            raise FAError(-1, "key_len must be a contiguous device int32 tensor of B elements")
        kl = key_len.data_ptr()
    need = fa_split_workspace_bytes(B, H, Nq, Nk, d, num_splits)
    ws, wsb = 0, 0
    if workspace is not None or need > 0:
        workspace, ws, wsb = _workspace(workspace, need, q.device)
    out = _output(out, q.shape, q.dtype, q.device, "out")
    lse = _output(lse, (B, H, Nq), torch.float32, q.device, "lse")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    check(fa_forward_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                           kl, _dtype_code(q), int(num_splits), ws, wsb, stream))
    return out, lse


def naive_backward(q, k, v, o, lse, dout, *, scale=None, causal=False, key_len=None,
                   workspace=None, dq=None, dk=None, dv=None):
    """The stored-state backward (fa_naive_backward): same gradients as
    ``backward``, with the N x N matrices in the workspace."""
    return backward(q, k, v, o, lse, dout, scale=scale, causal=causal, key_len=key_len,
                    workspace=workspace, dq=dq, dk=dk, dv=dv, _naive=True)


def backward_dropout(q, k, v, o, lse, dout, *, p_drop, seed, offset=0, scale=None, causal=False,
                     key_len=None, workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV = fa_backward_dropout(...): gradients for the result (o, lse)
    of forward_dropout with the same p_drop, seed, offset and masks."""
    return backward(q, k, v, o, lse, dout, scale=scale, causal=causal, key_len=key_len,
                    workspace=workspace, dq=dq, dk=dk, dv=dv, _drop=(p_drop, seed, offset))


def backward_bias(q, k, v, o, lse, dout, bias, *, scale=None, causal=False, key_len=None,
                  workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV = fa_backward_bias(...): gradients for the result (o, lse) of
    forward_bias with the same mask (a device float32 tensor broadcastable to
    [B, H, N, N] as for forward_bias)."""
    return backward(q, k, v, o, lse, dout, scale=scale, causal=causal, key_len=key_len,
                    workspace=workspace, dq=dq, dk=dk, dv=dv, _bias=bias)


def backward(q, k, v, o, lse, dout, *, scale=None, causal=False, key_len=None, workspace=None,
             dq=None, dk=None, dv=None, _naive=False, _drop=None, _bias=None):
    """dQ, dK, dV = fa_backward(...): gradients of sum(dout * O) for the forward
    result (o, lse) of the same q, k, v, scale, causal and key_len."""
    import torch
    for t in (q, k, v, o, dout):
        if t.dim() != 4 or t.shape != q.shape or t.dtype != q.dtype:
            raise FAError(-2, "q, k, v, o, dout must share one [B, H, N, d] shape and dtype")
        if not t.is_cuda or not t.is_contiguous():
            raise FAError(-1, "q, k, v, o, dout must be contiguous device tensors")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_cuda or \
            not lse.is_contiguous():
        raise FAError(-2, "lse must be a contiguous device float32 tensor [B, H, N]")
    _same_device(q.device, k, v, o, lse, dout, key_len)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl = 0
    if key_len is not None:
        if key_len.dtype != torch.int32 or not key_len.is_cuda or key_len.numel() != B:
            raise FAError(-1, "key_len must be a device int32 tensor of B elements")
        kl = key_len.data_ptr()
    dt = _dtype_code(q)
    need = (fa_naive_workspace_bytes(B, H, N, dt) if _naive
            else fa_backward_workspace_bytes(B, H, N, d, dt))
    workspace, ws, wsb = _workspace(workspace, need, q.device)
    dq = _output(dq, q.shape, q.dtype, q.device, "dq")
    dk = _output(dk, k.shape, k.dtype, q.device, "dk")
    dv = _output(dv, v.shape, v.dtype, q.device, "dv")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
            float(scale), int(bool(causal)), kl, dt)
    tail = (ws, wsb, stream)
    if _drop is not None:
        check(fa_backward_dropout(*args, float(_drop[0]), int(_drop[1]), int(_drop[2]), *tail))
    elif _bias is not None:
        _same_device(q.device, _bias)
        ptr, sb, sh, ld = _bias_layout(_bias, B, H, N)
        check(fa_backward_bias(*args[:9], ptr, *args[9:], sb, sh, ld, *tail))
    else:
        fn = fa_naive_backward if _naive else fa_backward
        check(fn(*args, *tail))
    return dq, dk, dv


def backward_gqa(q, k, v, o, lse, dout, *, scale=None, causal=False, key_len=None,
                 workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV = fa_backward_gqa(...): gradients for the result (o, lse) of
    forward_split on q [B, H, Nq, d], k, v [B, Hkv, Nk, d] (rows at the end of
    the keys); dk, dv sum over the query heads that share a key/value head."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[0] != k.shape[0] \
            or q.shape[3] != k.shape[3] or k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise FAError(-2, "q [B, H, Nq, d] and k, v [B, Hkv, Nk, d] (Hkv dividing H) expected")
    for t in (o, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise FAError(-2, "o and dout must have the shape and dtype of q")
    for t in (q, k, v, o, dout):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise FAError(-1, "q, k, v, o, dout must be contiguous device tensors of one dtype")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_cuda or \
            not lse.is_contiguous():
        raise FAError(-2, "lse must be a contiguous device float32 tensor [B, H, Nq]")
    _same_device(q.device, k, v, o, lse, dout, key_len)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl = 0
    if key_len is not None:
        if key_len.dtype != torch.int32 or not key_len.is_cuda or key_len.numel() != B or \
                not key_len.is_contiguous():
            raise FAError(-1, "key_len must be a contiguous device int32 tensor of B elements")
        kl = key_len.data_ptr()
    dt = _dtype_code(q)
    workspace, ws, wsb = _workspace(workspace, fa_backward_workspace_bytes(B, H, Nq, d, dt),
                                    q.device)
    dq = _output(dq, q.shape, q.dtype, q.device, "dq")
    dk = _output(dk, k.shape, k.dtype, q.device, "dk")
    dv = _output(dv, v.shape, v.dtype, q.device, "dv")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    check(fa_backward_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv,
                          Nq, Nk, d, float(scale), int(bool(causal)), kl, dt, ws, wsb, stream))
    return dq, dk, dv


def backward_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, *, scale=None, causal=False, workspace=None, dq=None, dk=None,
                    dv=None):
    """dQ, dK, dV = fa_backward_varlen(...): gradients for the result (o, lse)
    of forward_varlen on the same packed batch (q, o, dout [Tq, H, d]; k, v
    [Tk, Hkv, d]; lse [Tq, H])."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[2] != k.shape[2] \
            or k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise FAError(-2, "q [Tq, H, d] and k, v [Tk, Hkv, d] (Hkv dividing H) expected")
    for t in (o, dout):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise FAError(-2, "o and dout must have the shape and dtype of q")
    for t in (q, k, v, o, dout, cu_seqlens_q, cu_seqlens_k):
        if not t.is_cuda or not t.is_contiguous():
            raise FAError(-1, "all tensors must be contiguous device tensors")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or \
            cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise FAError(-2, "cu_seqlens_q and cu_seqlens_k must be int32 [B + 1]")
    Tq, H, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    if lse.shape != (Tq, H) or lse.dtype != torch.float32 or not lse.is_cuda or \
            not lse.is_contiguous():
        raise FAError(-2, "lse must be a contiguous device float32 tensor [Tq, H]")
    _same_device(q.device, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k)
    B = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = _dtype_code(q)
    workspace, ws, wsb = _workspace(workspace, fa_backward_workspace_bytes(1, H, Tq, d, dt),
                                    q.device)
    dq = _output(dq, q.shape, q.dtype, q.device, "dq")
    dk = _output(dk, k.shape, k.dtype, q.device, "dk")
    dv = _output(dv, v.shape, v.dtype, q.device, "dv")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    check(fa_backward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B,
                             H, Hkv, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), d,
                             float(scale), int(bool(causal)), dt, ws, wsb, stream))
    return dq, dk, dv


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *,
                   scale=None, causal=False, out=None, lse=None):
    """O, LSE = fa_forward_varlen(...): packed q [Tq, H, d], k, v [Tk, Hkv, d],
    device int32 offsets [B + 1]; lse is [Tq, H]."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise FAError(-2, "q [Tq, H, d] and k, v [Tk, Hkv, d] expected")
    for t in (q, k, v, cu_seqlens_q, cu_seqlens_k):
        if not t.is_cuda or not t.is_contiguous():
            raise FAError(-1, "all tensors must be contiguous device tensors")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or \
            cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise FAError(-2, "cu_seqlens_q and cu_seqlens_k must be int32 [B + 1]")
    Tq, H, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    _same_device(q.device, k, v, cu_seqlens_q, cu_seqlens_k)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _output(out, q.shape, q.dtype, q.device, "out")
    lse = _output(lse, (Tq, H), torch.float32, q.device, "lse")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    check(fa_forward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H,
                            Hkv, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), d, float(scale),
                            int(bool(causal)), _dtype_code(q), stream))
    return out, lse


def forward_dropout(q, k, v, *, p_drop, seed, offset=0, scale=None, causal=False, key_len=None,
                    out=None, lse=None):
    """O, LSE = fa_forward_dropout(...): dropout with rate p_drop on the
    probabilities, mask from Philox4x32-10 keyed by seed, counter word 3 = offset."""
    import torch
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise FAError(-2, "q, k, v must share one [B, H, N, d] shape")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise FAError(-1, "q, k, v must be contiguous device tensors")
    B, H, N, d = q.shape
    _same_device(q.device, k, v, key_len)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl = 0
    if key_len is not None:
        if key_len.dtype != torch.int32 or not key_len.is_cuda or key_len.numel() != B or \
                not key_len.is_contiguous():
            raise FAError(-1, "key_len must be a contiguous device int32 tensor of B elements")
        kl = key_len.data_ptr()
    out = _output(out, q.shape, q.dtype, q.device, "out")
    lse = _output(lse, (B, H, N), torch.float32, q.device, "lse")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    check(fa_forward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)), kl,
                             _dtype_code(q), float(p_drop), int(seed), int(offset), stream))
    return out, lse


def _bias_layout(bias, B, H, N):
    """(pointer, batch stride, head stride, row stride) of a mask tensor whose
    last two dims are [N, ld >= N] and whose batch and head dims have size B
    or 1 and H or 1 (size 1 broadcasts: stride 0)."""
    import torch
    if bias.dtype != torch.float32 or not bias.is_cuda or bias.dim() != 4 or \
            bias.shape[2] != N or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, H) or \
            bias.stride(3) != 1:
        raise FAError(-2, "bias must be a device float32 [B|1, H|1, N, ld] tensor, unit column stride")
    sb = bias.stride(0) if bias.shape[0] == B and B > 1 else 0
    sh = bias.stride(1) if bias.shape[1] == H and H > 1 else 0
    return bias.data_ptr(), sb, sh, bias.stride(2)


def forward_bias(q, k, v, bias, *, scale=None, causal=False, key_len=None, out=None, lse=None):
    """O, LSE = fa_forward_bias(...): bias is a device float32 tensor whose last
    two dims are [N, ld >= N] (ld a multiple of 4), with batch and head dims of
    size B or 1 and H or 1 (size 1 broadcasts: stride 0)."""
    import torch
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise FAError(-2, "q, k, v must share one [B, H, N, d] shape")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise FAError(-1, "q, k, v must be contiguous device tensors")
    B, H, N, d = q.shape
    _same_device(q.device, k, v, bias, key_len)
    ptr, sb, sh, ld = _bias_layout(bias, B, H, N)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kl = 0
    if key_len is not None:
        if key_len.dtype != torch.int32 or not key_len.is_cuda or key_len.numel() != B or \
                not key_len.is_contiguous():
            raise FAError(-1, "key_len must be a contiguous device int32 tensor of B elements")
        kl = key_len.data_ptr()
    out = _output(out, q.shape, q.dtype, q.device, "out")
    lse = _output(lse, (B, H, N), torch.float32, q.device, "lse")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    check(fa_forward_bias(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          ptr, B, H, N, d, float(scale), int(bool(causal)), kl,
                          _dtype_code(q), sb, sh, ld, stream))
    return out, lse
