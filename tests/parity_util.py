"""Helpers shared by the GPU parity tests: run the HIP path on seeded host
inputs, run the oracle on the same exact values, and compare.

Tolerances (max / mean absolute error over the outputs of valid rows; LSE
absolute error over valid rows):
  bf16 inputs: O max 2e-2, O mean 2e-3, LSE 1e-3;
  fp32 inputs: O max 1e-5, LSE 1e-3 (fp32 LSE errors are ~1e-6 in practice).
Padding rows (query index >= the sequence's key length) must be exactly 0
with LSE exactly -inf.
"""
from __future__ import annotations

import numpy as np

import oracle
from io_aware_exact_forward_amd import workloads as W

TOL = {"bf16": dict(o_max=2e-2, o_mean=2e-3, lse=1e-3),
       "f32": dict(o_max=1e-5, o_mean=1e-5, lse=1e-3)}


def to_device(inp):
    import torch
    dev = torch.device("cuda:0")
    if inp.wl.dtype == "bf16":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    q, k, v = conv(inp.q), conv(inp.k), conv(inp.v)
    kl = None if inp.key_len is None else torch.from_numpy(inp.key_len.astype(np.int32)).to(dev)
    return q, k, v, kl


def from_device(o):
    import torch
    if o.dtype == torch.bfloat16:
        return W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)
    return o.cpu().numpy().astype(np.float64)


def run_hip(inp, causal, scale, naive=False):
    import torch
    import io_aware_exact_forward_amd as fa
    q, k, v, kl = to_device(inp)
    fn = fa.naive_forward if naive else fa.forward
    o, lse = fn(q, k, v, scale=scale, causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return from_device(o), lse.cpu().numpy().astype(np.float64)


def row_lengths(inp):
    B, N = inp.q.shape[0], inp.q.shape[2]
    if inp.key_len is None:
        return np.full(B, N)
    return np.clip(inp.key_len.astype(np.int64), 0, N)


def compare(inp, o_gpu, lse_gpu, causal, scale, rows=None, tol=None, label=""):
    """Oracle on the same exact inputs (all rows, or rows [H, R]) vs the GPU.

    Returns a dict of the error statistics; raises AssertionError on failure.
    """
    tol = tol or TOL[inp.wl.dtype]
    qx, kx, vx = inp.exact("q"), inp.exact("k"), inp.exact("v")
    o_ref, lse_ref = oracle.attention(qx, kx, vx, scale, causal=causal, key_len=inp.key_len, rows=rows)
    B, H, N, d = inp.q.shape
    if rows is None:
        og, lg = o_gpu, lse_gpu
        ridx = np.broadcast_to(np.arange(N), (B, H, N))
    else:
        r = np.asarray(rows)
        r = np.broadcast_to(r if r.ndim == 2 else r[None, :], (H, r.shape[-1]))
        og = np.stack([o_gpu[:, h, r[h]] for h in range(H)], axis=1)
        lg = np.stack([lse_gpu[:, h, r[h]] for h in range(H)], axis=1)
        ridx = np.broadcast_to(r[None], (B, H, r.shape[-1]))
    lens = row_lengths(inp)
    valid = ridx < lens[:, None, None]
    stats = {"label": label, "rows_checked": int(valid.sum())}
    if valid.any():
        err = np.abs(og - o_ref)[valid]
        lerr = np.abs(lg[valid] - lse_ref[valid])
        stats.update(o_max=float(err.max()), o_mean=float(err.mean()), lse_max=float(lerr.max()))
        assert np.all(np.isfinite(og[valid])), f"{label}: non-finite output"
        assert stats["o_max"] <= tol["o_max"], f"{label}: O max abs {stats['o_max']:.3g} > {tol['o_max']}"
        assert stats["o_mean"] <= tol["o_mean"], f"{label}: O mean abs {stats['o_mean']:.3g} > {tol['o_mean']}"
        assert stats["lse_max"] <= tol["lse"], f"{label}: LSE abs {stats['lse_max']:.3g} > {tol['lse']}"
    pad = ~valid
    if pad.any():
        assert np.all(og[pad] == 0.0), f"{label}: padding rows not exactly zero"
        assert np.all(lg[pad] == -np.inf), f"{label}: padding rows' LSE not -inf"
    return stats


def check_all_padding(inp, o_gpu, lse_gpu):
    """Every padding row of the full GPU output is exactly 0 / -inf."""
    lens = row_lengths(inp)
    N = inp.q.shape[2]
    for b, L in enumerate(lens):
        if L < N:
            assert np.all(o_gpu[b, :, L:] == 0.0)
            assert np.all(lse_gpu[b, :, L:] == -np.inf)
