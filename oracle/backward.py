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

Grouped key/value heads and packed batches ("IO-aware exact attention",
section "Why implementations form a family", lists both among the variants
that change data access only): a key/value head read by several query heads
is one operand shared by their attentions, so by the chain rule its gradient
is the sum of the per-query-head gradients (grouped_attention_backward); a
packed batch is a set of independent sequences (varlen_attention_backward).
Rows sit at the positions of the forward oracle's end-aligned reading.

An additive mask M ("IO-aware exact attention", section "Move less data":
softmax(Q K^T / sqrt(d) + M)) is a constant of the loss: it enters S and so P,
and the chain rule above is unchanged (attention_backward(..., bias=M)).

Pins (tests/test_oracle_backward.py): central finite differences of
sum(dO * O) through the forward oracle on tiny inputs, for every mask, for
grouped heads with end-aligned rows, for packed batches and with an additive
mask (hidden pairs and a wholly hidden row); a per-row constant mask changes
nothing;
torch.autograd in float64 through an independently written forward; closed
forms for uniform scores; invariants (keys' gradients sum to zero, a
constant added to every value row changes no gradient, the query gradient
of a row with a single visible key is zero); and planted mistakes that must
fail a pin.  No function here is parity unpinned.
"""
from __future__ import annotations

import numpy as np

from .attention import NEG_INF, _clamped_length, visible_mask

__all__ = ["attention_backward", "grouped_attention_backward", "varlen_attention_backward",
           "kv_head_of"]


def attention_backward(q, k, v, do, scale, causal=False, key_len=None, bias=None):
    """Gradients (dq, dk, dv) of sum(do * O) for O = attention(q, k, v, ...).

    q, k, v, do: float64 arrays [B, H, N, d] (square: Nq = Nk = N); the
    positions and masks are those of ``attention`` (query row i at key
    position i, keys j < L_b, padding rows i >= L_b).  bias: None, or the
    additive mask M of ``attention`` (broadcastable to [B, H, N, N]), a
    constant of the loss: S = scale * Q K^T + M, and -inf entries hide their
    pair.  Returns three arrays shaped like q, k and v, and D [B, H, N]
    (D_i = sum_j P_ij dP_ij).
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
    if bias is not None:
        bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, H, N, N))
    for b in range(B):
        L = _clamped_length(key_len, b, N)
        vis0 = visible_mask(np.arange(N), N, L, causal)
        for h in range(H):
            # P: the masked softmax of the scaled scores, materialised.
            s = scale * (q[b, h] @ k[b, h].T)
            vis = vis0
            if bias is not None:
                s = s + bias[b, h]
                vis = vis0 & (s > NEG_INF)
            live = vis.any(axis=1)
            s = np.where(vis, s, NEG_INF)
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


def kv_head_of(h, H, Hkv):
    """Key/value head read by query head h: each of the Hkv heads serves
    H / Hkv consecutive query heads (the grouping of expand_kv_heads)."""
    return h // (H // Hkv)


def _head_gradients(q, k, v, do, scale, vis):
    """One query head against its key/value head: q, do [Nq, d]; k, v
    [Nk, d]; vis [Nq, Nk] the visible pairs.  The chain rule of the module
    notes with P the masked softmax; returns dq, dk, dv and D [Nq]."""
    s = np.where(vis, scale * (q @ k.T), NEG_INF)
    live = vis.any(axis=1)
    m = np.where(live, s.max(axis=1, initial=NEG_INF), 0.0)
    w = np.where(vis, np.exp(s - m[:, None]), 0.0)
    ell = w.sum(axis=1)
    p = np.divide(w, ell[:, None], out=np.zeros_like(w), where=live[:, None])
    dv = p.T @ do
    dp = do @ v.T
    dvec = (p * dp).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv, dvec


def grouped_attention_backward(q, k, v, do, scale, causal=False, key_len=None, end_aligned=True):
    """Gradients of sum(do * O) for O = attention(q, expand_kv_heads(k, H),
    expand_kv_heads(v, H), scale, causal, key_len, end_aligned=end_aligned).

    q, do: [B, H, Nq, d]; k, v: [B, Hkv, Nk, d] with Hkv dividing H.  Query
    row i of sequence b sits at key position i + L_b - Nq (end_aligned, the
    reading of the split forward) or i, L_b = clamp(key_len[b], 0, Nk).  The
    gradient of key/value head g is the sum over the query heads h with
    kv_head_of(h) = g.  Returns dq [B, H, Nq, d], dk and dv [B, Hkv, Nk, d],
    D [B, H, Nq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, Nq, _ = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of the key/value heads")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.zeros((B, H, Nq))
    for b in range(B):
        L = _clamped_length(key_len, b, Nk)
        vis = visible_mask(np.arange(Nq), Nk, L, causal, L - Nq if end_aligned else 0)
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            gq, gk, gv, dvec[b, h] = _head_gradients(q[b, h], k[b, g], v[b, g], do[b, h], scale, vis)
            dq[b, h] = gq
            dk[b, g] += gk
            dv[b, g] += gv
    return dq, dk, dv, dvec


def varlen_attention_backward(q, k, v, do, cu_q, cu_k, scale, causal=False):
    """Gradients of sum(do * O) for O = varlen_attention(q, k, v, cu_q, cu_k,
    scale, causal): packed q, do [Tq, H, d] and k, v [Tk, Hkv, d], sequence b
    at query rows cu_q[b] .. cu_q[b+1]-1 and keys cu_k[b] .. cu_k[b+1]-1,
    rows at the end of their sequence's keys.  Sequences are independent, so
    each is grouped_attention_backward on its own tokens.  Returns dq
    [Tq, H, d], dk and dv [Tk, Hkv, d], D [Tq, H]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.zeros(q.shape[:2])
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        seq = lambda x, a, z: x[a:z].transpose(1, 0, 2)[None]
        gq, gk, gv, dd = grouped_attention_backward(seq(q, q0, q1), seq(k, k0, k1), seq(v, k0, k1),
                                                    seq(do, q0, q1), scale, causal=causal,
                                                    end_aligned=True)
        dq[q0:q1] = gq[0].transpose(1, 0, 2)
        dk[k0:k1] = gk[0].transpose(1, 0, 2)
        dv[k0:k1] = gv[0].transpose(1, 0, 2)
        dvec[q0:q1] = dd[0].T
    return dq, dk, dv, dvec
