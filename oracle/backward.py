"""fp64 CPU oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test
suite, the smoke check and the benchmark's CPU-baseline leg call it; it
imports nothing from the HIP package.

What it computes.  "IO-aware exact attention" (section "Backward
recomputation") states the backward's result: dQ, dK and dV of attention
for an upstream gradient dO, rebuilt from the inputs, the output and the
per-row log-sum-exp.  The pages give no formulas; the gradient is that of the
plain definition O = softmax(scale * Q K^T + M) V (the forward oracle in
attention.py), for the scalar loss sum(dO * O).  Written out by the chain
rule, per (batch, head), with P the masked softmax and rows of P that see
no key equal to zero:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij            (equals dO_i . O_i)
    dS_ij = P_ij (dP_ij - D_i)        (the softmax Jacobian
                                       dP_ij/ds_ik = P_ij (delta_jk - P_ik))
    dQ = scale * dS K
    dK = scale * dS^T Q

Masked pairs have P_ij = 0 and so contribute nothing; padding rows (and keys
at or beyond a sequence's length) get zero gradients.  Everything is
materialised in fp64, one (batch, head) at a time.

Pins (tests/test_oracle_backward.py): central finite differences of
sum(dO * O) through the forward oracle on tiny inputs, for every mask;
torch.autograd in float64 through an independently written forward; closed
forms for uniform scores; invariants (keys' gradients sum to zero, a
constant added to every value row changes no gradient, the query gradient
of a row with a single visible key is zero); and planted mistakes that must
fail a pin.  No function here is parity unpinned.
"""
from __future__ import annotations

import numpy as np

from .attention import NEG_INF, _clamped_length, visible_mask

__all__ = ["attention_backward"]


def attention_backward(q, k, v, do, scale, causal=False, key_len=None):
    """Gradients (dq, dk, dv) of sum(do * O) for O = attention(q, k, v, ...).

    q, k, v, do: float64 arrays [B, H, N, d] (square: Nq = Nk = N); the
    positions and masks are those of ``attention`` (query row i at key
    position i, keys j < L_b, padding rows i >= L_b).  Returns three arrays
    shaped like q, k and v, and D [B, H, N] (D_i = sum_j P_ij dP_ij).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.zeros((B, H, N))
    for b in range(B):
        L = _clamped_length(key_len, b, N)
        vis = visible_mask(np.arange(N), N, L, causal)
        live = vis.any(axis=1)
        for h in range(H):
            # P: the masked softmax of the scaled scores, materialised.
            s = np.where(vis, scale * (q[b, h] @ k[b, h].T), NEG_INF)
            m = np.where(live, s.max(axis=1, initial=NEG_INF), 0.0)
            w = np.where(vis, np.exp(s - m[:, None]), 0.0)
            ell = w.sum(axis=1)
            p = np.divide(w, ell[:, None], out=np.zeros_like(w), where=live[:, None])
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            dvec[b, h] = (p * dp).sum(axis=1)
            ds = p * (dp - dvec[b, h][:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv, dvec
