"""fp64 CPU oracle for attention with dropout on the probabilities.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The pages name dropout as a variant that changes the schedule ("IO-aware
exact attention", section "Why implementations form a family") without
fixing its random numbers.  The reading taken here:

  * dropout acts on the normalised probabilities: O = (P * Z / (1 - p)) V,
    where Z_ij is 1 (keep) or 0 (drop); the log-sum-exp is that of the
    undropped row (the softmax normaliser), as without dropout;
  * Z_ij comes from the counter-based generator Philox4x32-10 (J. K. Salmon,
    M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy
    as 1, 2, 3", SC 2011), keyed by the 64-bit seed (low word first), with
    the 128-bit counter (j // 4, i, b * H + h, offset); output word j % 4 is
    the draw u_ij of query row i and key j of head h in batch entry b;
  * Z_ij = 1 iff u_ij >= floor(p * 2^32), so the keep probability is
    1 - floor(p * 2^32) / 2^32; p is the binary64 rate the caller gives,
    and the floor is that of the real product p * 2^32 (keep_threshold).

The gradient (dropout_attention_backward) treats the mask Z as a constant of
the step (the same seed and offset regenerate it): with P the undropped
softmax and dO the upstream gradient of the loss sum(dO * O),

    dV = (P * Z)^T dO / (1 - p)
    dP = Z * (dO V^T) / (1 - p)
    D_i = sum_j P_ij dP_ij        (equals dO_i . O_i with the dropped O)
    dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.

Pins (tests/test_oracle_dropout.py): the generator against the published
known-answer vectors of Philox4x32-10 (tests/golden/philox4x32_10_kat.json);
p = 0 equals attention(); the kept fraction within a binomial bound; the
average over many offsets tends to the undropped output (dropout is unbiased);
a closed form with uniform scores; distinct masks per head, batch entry,
offset and seed.
"""
from __future__ import annotations

import numpy as np

from .attention import NEG_INF, _clamped_length, visible_mask

__all__ = ["philox4x32_10", "keep_threshold", "dropout_keep", "dropout_attention",
           "dropout_attention_backward"]

_M0, _M1 = 0xD2511F53, 0xCD9E8D57  # round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85  # key schedule (Weyl) increments
_MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds on arrays of counters.

    counter: four uint32 arrays (broadcastable), key: two uint32 values.
    Each round multiplies words 0 and 2 by the round constants (64-bit
    products split into high and low halves), permutes and mixes them with
    words 1 and 3 and the key; the key is advanced by the Weyl increments
    between rounds.  Returns four uint32 arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK for c in counter)
    k0, k1 = int(key[0]) & _MASK, int(key[1]) & _MASK
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = c0 * np.uint64(_M0)
        p1 = c2 * np.uint64(_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def keep_threshold(p):
    """floor(p * 2^32) for a rate p in [0, 1): a draw u is kept iff u is at
    least this.  p is taken as the binary64 number it is; multiplying by 2^32
    moves only its exponent, so the product and its floor are exact."""
    return min(int(float(p) * 2.0 ** 32), _MASK)


def dropout_keep(b, h, H, N, Nk, p, seed, offset):
    """Boolean [N, Nk]: Z_ij of query row i and key j of head h in batch b."""
    i = np.arange(N, dtype=np.uint64)[:, None]
    j = np.arange(Nk, dtype=np.uint64)[None, :]
    words = philox4x32_10((j >> np.uint64(2), i, np.uint64(b * H + h), np.uint64(offset)),
                          (seed & _MASK, (seed >> 32) & _MASK))
    jj = np.broadcast_to(j & np.uint64(3), (N, Nk))
    u = np.choose(jj.astype(np.int64), [np.broadcast_to(w, (N, Nk)) for w in words])
    return u >= np.uint32(keep_threshold(p))


def dropout_attention(q, k, v, scale, p, seed, offset=0, causal=False, key_len=None,
                      head_ids=None, H_all=None):
    """O = (P * Z / (1 - p)) V and the undropped LSE, square problems
    ([B, H, N, d], positions and masks as ``attention``).  fp64.

    head_ids / H_all: q, k, v hold heads head_ids[0..H-1] of an H_all-head
    problem (the mask depends on the head index); by default all heads."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, _ = q.shape
    ids = list(range(H)) if head_ids is None else [int(x) for x in head_ids]
    H_all = H if H_all is None else int(H_all)
    o = np.zeros((B, H, N, v.shape[-1]))
    lse = np.full((B, H, N), NEG_INF)
    for b in range(B):
        L = _clamped_length(key_len, b, N)
        vis = visible_mask(np.arange(N), N, L, causal)
        live = vis.any(axis=1)
        for h in range(H):
            s = np.where(vis, scale * (q[b, h] @ k[b, h].T), NEG_INF)
            m = np.where(live, s.max(axis=1, initial=NEG_INF), 0.0)
            w = np.where(vis, np.exp(s - m[:, None]), 0.0)
            ell = w.sum(axis=1)
            P = np.divide(w, ell[:, None], out=np.zeros_like(w), where=live[:, None])
            Z = dropout_keep(b, ids[h], H_all, N, N, p, seed, offset)
            o[b, h] = (P * Z) @ v[b, h] / (1.0 - p)
            with np.errstate(divide="ignore"):
                lse[b, h] = np.where(live, m + np.log(np.where(live, ell, 1.0)), NEG_INF)
    return o, lse


def dropout_attention_backward(q, k, v, do, scale, p, seed, offset=0, causal=False, key_len=None,
                               head_ids=None, H_all=None, batch_ids=None):
    """Gradients (dq, dk, dv, D) of sum(do * O) for O = dropout_attention(q, k,
    v, scale, p, seed, offset, causal, key_len): square problems [B, H, N, d],
    masks and positions as ``attention``; the keep mask of every head from
    ``dropout_keep``.  fp64, materialised per (batch, head).

    head_ids / H_all / batch_ids: q, k, v hold heads head_ids of batch
    entries batch_ids of an H_all-head problem (the mask depends on both
    indices); by default all of them.  key_len is indexed like q's batch."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, _ = q.shape
    hids = list(range(H)) if head_ids is None else [int(x) for x in head_ids]
    bids = list(range(B)) if batch_ids is None else [int(x) for x in batch_ids]
    H_all = H if H_all is None else int(H_all)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dvec = np.zeros((B, H, N))
    for b in range(B):
        L = _clamped_length(key_len, b, N)
        vis = visible_mask(np.arange(N), N, L, causal)
        live = vis.any(axis=1)
        for h in range(H):
            s = np.where(vis, scale * (q[b, h] @ k[b, h].T), NEG_INF)
            m = np.where(live, s.max(axis=1, initial=NEG_INF), 0.0)
            w = np.where(vis, np.exp(s - m[:, None]), 0.0)
            ell = w.sum(axis=1)
            P = np.divide(w, ell[:, None], out=np.zeros_like(w), where=live[:, None])
            Z = dropout_keep(bids[b], hids[h], H_all, N, N, p, seed, offset)
            dv[b, h] = (P * Z).T @ do[b, h] / (1.0 - p)
            dP = Z * (do[b, h] @ v[b, h].T) / (1.0 - p)
            dvec[b, h] = (P * dP).sum(axis=1)
            dS = P * (dP - dvec[b, h][:, None])
            dq[b, h] = scale * (dS @ k[b, h])
            dk[b, h] = scale * (dS.T @ q[b, h])
    return dq, dk, dv, dvec
