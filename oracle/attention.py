"""fp64 CPU oracle for exact (masked, scaled) attention and its online-softmax form.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plainly written checker for
the HIP attention forward.  Only the test suite, the smoke check in the repository's
graft entry point and the CPU-baseline leg of the benchmark may import or call
it; the product path never does, and this module imports nothing from the
HIP package.

Every function works in float64 on the exact values it is given (for bf16
device tensors the caller passes their exact fp64 widening).

Sources, cited by page title and section:
  [P1] "FlashAttention: Exact Attention as an IO-Aware Streaming Computation",
       sections "Problem setting", "Mathematical structure", "Why it can work".
  [P2] "IO-aware exact attention", sections "Traffic in the materialized
       implementation", "One tiled forward-pass iteration", "Tile order and
       on-chip capacity", "Backward recomputation".
  [P3] "FlashAttention" (glossary), sections "Move less data", "Why a tile can
       be discarded", "One row, checked two ways", "Practice: can you average
       block outputs?".
  [P4] "FlashAttention: IO-Aware Exact Attention", section "The idea: tiling +
       online softmax, kept in SRAM".

Readings taken where the pages are silent (each is also listed with the design
notes of the repository):
  * the scale multiplies Q K^T and the additive mask M is added after it [P3
    "Move less data"; P2 "One tiled forward-pass iteration" scales then masks];
  * causal: key j is visible to query i iff j <= i [P2 "Tile order and on-chip
    capacity": keys at or before the query position];
  * a per-sequence length L masks keys j >= L and marks queries i >= L as
    padding, whose output is 0; the length is clamped to [0, N];
  * a row with no visible key (only padding rows here) gets O = 0 and
    LSE = -inf, the log of an empty sum [P3 "Why a tile can be discarded"
    requires explicit handling of fully masked blocks];
  * LSE is the natural-log log-sum-exp of the row's scaled, masked scores,
    the "compact per-row normalization information" of P2 "Backward
    recomputation";
  * with Nq query rows against Nk keys (decode and chunked prefill, the
    serving regimes of P2 "Exercise" and "Common errors"), the keys are a
    cache holding L_b = clamp(key_len[b], 0, Nk) valid entries (Nk without a
    length) and the query rows, when end aligned, are that sequence's last
    Nq positions: row i sits at key position p = i + L_b - Nq.  Keys j >= L_b
    are hidden, causal also hides j > p, and no row is padding; a row that
    sees no key (L_b = 0, or p < 0 under causal) gets O = 0, LSE = -inf.
    Without a length and with Nq = Nk this is the square case unchanged.

Pins (tests/test_oracle.py): the two worked examples of P3 with every printed
intermediate value, closed forms (uniform scores, causal running means,
single visible key, dominant key), invariants (convex hull, shift and
permutation invariance), scipy's softmax on the unmasked case, pure-Python
brute force with exact summation on tiny inputs, and agreement between the
plain definition and the streamed recurrence.  The Nq != Nk reading is pinned
by brute force with positions on tiny inputs, by the last Nq rows of the
square problem (causal and padded) and by decode rows against scipy's
softmax over the visible keys.  Grouped key/value heads are pinned by a
closed form (value rows that name their head) and varlen batches by the
padded problem with per-sequence lengths and by brute force with a key
cache.  The additive mask (bias) is pinned by zero and row-constant biases,
-inf entries reproducing the causal mask, a closed form with log weights and
brute force.  No function here is parity unpinned.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "attention",
    "visible_mask",
    "block_summary",
    "merge_summaries",
    "finalize_summary",
    "streamed_attention",
    "split_attention",
    "expand_kv_heads",
    "varlen_attention",
]

NEG_INF = -np.inf


def _clamped_length(key_len, b: int, N: int) -> int:
    if key_len is None:
        return N
    return int(min(max(int(key_len[b]), 0), N))


def visible_mask(rows: np.ndarray, N: int, L: int, causal: bool, pos_off: int = 0) -> np.ndarray:
    """Boolean [R, N]: key j (of N keys) visible to query rows[r].

    The query row sits at key position p = rows[r] + pos_off.  Key j is
    visible iff j < L, p < L and (not causal or j <= p).  This is the support
    of the additive mask M of [P3 "Move less data"]: M = 0 where visible,
    -inf elsewhere.
    """
    p = np.asarray(rows, dtype=np.int64)[:, None] + int(pos_off)
    j = np.arange(N, dtype=np.int64)[None, :]
    vis = (j < L) & (p < L)
    if causal:
        vis &= j <= p
    return vis


def attention(q, k, v, scale, causal=False, key_len=None, rows=None, chunk_rows=256,
              end_aligned=False, bias=None):
    """Plain definition: O = softmax(scale * Q K^T + M) V, and per-row LSE.

    [P1 "Problem setting"] defines O = softmax(Q K^T / sqrt(d)) V; [P3 "Move
    less data"] adds the optional additive mask M and states that softmax runs
    across keys for each query.  The materialised dataflow of [P1 "Problem
    setting"] / [P2 "Traffic in the materialized implementation"] is followed
    literally: whole score rows S[R, :] are formed, then P = softmax(S) row by
    row, then O = P V.  The usual max shift inside softmax changes nothing
    mathematically (softmax is shift invariant, [P4]).

    q: float64 array [B, H, Nq, d]; k, v: [B, H, Nk, d] (v may have its own
    last dim).  Query row i sits at key position i, or with end_aligned at
    i + L_b - Nq, where no row is padding (see the module notes).
    rows: None (all rows), or int array [R], [H, R] or [B, H, R] of query rows.
    bias: None, or the additive mask M of [P3 "Move less data"] as an array
    broadcastable to [B, H, Nq, Nk], added to the scaled scores before the
    causal and length masks; -inf entries hide a pair, and a row whose every
    score is -inf gets O = 0, LSE = -inf.
    Returns (o [B, H, R, dv], lse [B, H, R]) with R = Nq when rows is None.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, _ = q.shape
    N = k.shape[2]  # keys
    dv = v.shape[-1]
    if rows is None:
        rows_bh = np.broadcast_to(np.arange(Nq, dtype=np.int64), (B, H, Nq))
    else:
        r = np.asarray(rows, dtype=np.int64)
        if r.ndim == 1:
            r = r[None, None, :]
        elif r.ndim == 2:
            r = r[None, :, :]
        rows_bh = np.broadcast_to(r, (B, H, r.shape[-1]))
    R = rows_bh.shape[-1]
    if bias is not None:
        bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, H, Nq, N))
    o = np.zeros((B, H, R, dv), dtype=np.float64)
    lse = np.full((B, H, R), NEG_INF, dtype=np.float64)
    for b in range(B):
        L = _clamped_length(key_len, b, N)
        pos_off = L - Nq if end_aligned else 0
        for h in range(H):
            for r0 in range(0, R, chunk_rows):
                rr = rows_bh[b, h, r0:r0 + chunk_rows]
                # S = scale * Q K^T for whole rows (all N keys).
                s = scale * (q[b, h, rr, :] @ k[b, h].T)
                vis = visible_mask(rr, N, L, causal, pos_off)
                if bias is not None:
                    s = s + bias[b, h, rr, :]
                    vis = vis & (s > NEG_INF)  # an additive -inf hides the pair
                live = vis.any(axis=1)
                # Additive mask: -inf where not visible.
                s = np.where(vis, s, NEG_INF)
                # Row maximum over visible keys (0 for rows with none).
                m = np.where(live, s.max(axis=1, initial=NEG_INF), 0.0)
                w = np.where(vis, np.exp(s - m[:, None]), 0.0)
                ell = w.sum(axis=1)
                # P = softmax(S + M), materialised for these rows.
                p = np.divide(w, ell[:, None], out=np.zeros_like(w), where=live[:, None])
                o[b, h, r0:r0 + len(rr)] = p @ v[b, h]
                with np.errstate(divide="ignore"):
                    lse[b, h, r0:r0 + len(rr)] = np.where(live, m + np.log(np.where(live, ell, 1.0)), NEG_INF)
    return o, lse


# ---------------------------------------------------------------------------
# Block summaries [P3 "Why a tile can be discarded", "One row, checked two ways"]
# ---------------------------------------------------------------------------

def block_summary(scores, values):
    """Summary (m, l, u) of one query row over one block of keys.

    m = max of the block's scores, l = sum of exp(s - m), u = sum of
    exp(s - m) * v (the value-weighted numerator).  This is the row state
    (m, l, a) of [P1 "Mathematical structure"] restricted to one block.  A
    block whose scores are all -inf (fully masked) is handled explicitly and
    summarised as (-inf, 0, 0) instead of evaluating -inf - (-inf).
    """
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    vals = np.asarray(values, dtype=np.float64)
    vals = vals.reshape(len(s), -1)
    if s.size == 0 or np.all(s == NEG_INF):
        return NEG_INF, 0.0, np.zeros(vals.shape[1])
    m = float(np.max(s))
    w = np.exp(s - m)
    return m, float(w.sum()), w @ vals


def merge_summaries(a, b):
    """Merge the summaries of two disjoint key blocks of the same query row.

    Both are first expressed relative to the common maximum max(m_a, m_b):
    each block's l and u are multiplied by exp(m_block - m_common), then the
    two are added [P3 "Why a tile can be discarded"; worked in "One row,
    checked two ways" and "Practice"].  A fully masked side contributes zero.
    """
    ma, la, ua = a
    mb, lb, ub = b
    ua = np.asarray(ua, dtype=np.float64)
    ub = np.asarray(ub, dtype=np.float64)
    m = max(ma, mb)
    if m == NEG_INF:
        return NEG_INF, 0.0, np.zeros_like(ua)
    fa = 0.0 if ma == NEG_INF else float(np.exp(ma - m))
    fb = 0.0 if mb == NEG_INF else float(np.exp(mb - m))
    return m, fa * la + fb * lb, fa * ua + fb * ub


def finalize_summary(summary):
    """Output o = u / l of a row summary [P1 "Mathematical structure", final step].

    A row with l = 0 (no visible key) gives o = 0 and lse = -inf.
    Returns (o, lse).
    """
    m, ell, u = summary
    u = np.asarray(u, dtype=np.float64)
    if ell == 0.0:
        return np.zeros_like(u), NEG_INF
    return u / ell, m + float(np.log(ell))


# ---------------------------------------------------------------------------
# The streamed recurrence [P1 "Mathematical structure"; P2 "One tiled
# forward-pass iteration"]
# ---------------------------------------------------------------------------

def streamed_attention(q, k, v, scale, causal=False, key_len=None,
                       block_q=64, block_k=64, trace=None):
    """Tile-by-tile forward with running (m, l, a) per query row, in fp64.

    For each block of block_q query rows: start from m = -inf, l = 0, a = 0;
    for every block of block_k keys, in order, form the score tile
    scale * Q_tile K_tile^T, apply the mask, take the block's row maximum,
    raise the running maximum to it, rescale the old l and a by
    exp(m_old - m_new), add the block's exp(s - m_new) and exp(s - m_new) V,
    and drop the score tile.  After the last block, o = a / l.  Every key
    block is visited (including those wholly masked), so the explicit
    handling of fully masked blocks is exercised: where the running maximum
    is still -inf nothing is rescaled and nothing is added.

    ``trace``, if a list, receives (q_block, k_block, m, l, a) copies after
    every block update.

    Returns (o [B, H, N, dv], lse [B, H, N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, _ = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, N, dv))
    lse = np.full((B, H, N), NEG_INF)
    for b in range(B):
        L = _clamped_length(key_len, b, N)
        for h in range(H):
            for qi, q0 in enumerate(range(0, N, block_q)):
                rows = np.arange(q0, min(q0 + block_q, N))
                m = np.full(len(rows), NEG_INF)
                ell = np.zeros(len(rows))
                a = np.zeros((len(rows), dv))
                for kj, k0 in enumerate(range(0, N, block_k)):
                    cols = np.arange(k0, min(k0 + block_k, N))
                    s = scale * (q[b, h, rows] @ k[b, h, cols].T)
                    vis = visible_mask(rows, N, L, causal)[:, cols]
                    s = np.where(vis, s, NEG_INF)
                    m_blk = s.max(axis=1)
                    m_new = np.maximum(m, m_blk)
                    # Reference maximum; 0 stands in for rows that have seen
                    # no visible key yet, so -inf - (-inf) never occurs.
                    m_ref = np.where(m_new > NEG_INF, m_new, 0.0)
                    seen = m > NEG_INF
                    # exp(m_old - m_new) for rows with earlier state; rows
                    # without any (l = 0, a = 0) need no rescale.
                    alpha = np.where(seen, np.exp(np.where(seen, m, 0.0) - m_ref), 0.0)
                    w = np.where(vis, np.exp(s - m_ref[:, None]), 0.0)
                    ell = alpha * ell + w.sum(axis=1)
                    a = alpha[:, None] * a + w @ v[b, h, cols]
                    m = m_new
                    if trace is not None:
                        trace.append((qi, kj, m.copy(), ell.copy(), a.copy()))
                pos = ell > 0
                o[b, h, rows] = np.divide(a, ell[:, None], out=np.zeros_like(a), where=pos[:, None])
                with np.errstate(divide="ignore"):
                    lse[b, h, rows] = np.where(pos, m + np.log(np.where(pos, ell, 1.0)), NEG_INF)
    return o, lse


# ---------------------------------------------------------------------------
# Key ranges merged by their summaries [P3 "Why a tile can be discarded",
# "One row, checked two ways", "Practice: can you average block outputs?"]
# ---------------------------------------------------------------------------

def split_attention(q, k, v, scale, causal=False, key_len=None, split_keys=128,
                    end_aligned=True):
    """Each query row's keys cut into consecutive ranges of split_keys keys;
    every range is summarised on its own (block_summary over the row's masked
    scores in that range), the summaries are merged left to right with
    merge_summaries, and the merged summary is finalised.  Row by row, for
    small inputs.  Positions and masks are those of ``attention`` (end
    aligned by default, the decode convention).

    Returns (o [B, H, Nq, dv], lse [B, H, Nq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, _ = q.shape
    N = k.shape[2]
    dv = v.shape[-1]
    o = np.zeros((B, H, Nq, dv))
    lse = np.full((B, H, Nq), NEG_INF)
    for b in range(B):
        L = _clamped_length(key_len, b, N)
        pos_off = L - Nq if end_aligned else 0
        for h in range(H):
            vis = visible_mask(np.arange(Nq), N, L, causal, pos_off)
            s_all = scale * (q[b, h] @ k[b, h].T)
            for i in range(Nq):
                s_row = np.where(vis[i], s_all[i], NEG_INF)
                acc = (NEG_INF, 0.0, np.zeros(dv))
                for k0 in range(0, N, split_keys):
                    part = block_summary(s_row[k0:k0 + split_keys], v[b, h, k0:k0 + split_keys])
                    acc = merge_summaries(acc, part)
                o[b, h, i], lse[b, h, i] = finalize_summary(acc)
    return o, lse


# ---------------------------------------------------------------------------
# Shared key/value heads and packed variable-length batches ("IO-aware exact
# attention", section "Why implementations form a family": grouped heads and
# variable-length packing change the data access, not the result)
# ---------------------------------------------------------------------------

def expand_kv_heads(x, H):
    """[B, Hkv, N, d] -> [B, H, N, d]: query head h reads key/value head
    h // (H / Hkv), i.e. each key/value head serves H / Hkv consecutive query
    heads (grouped-query attention; Hkv = 1 is multi-query attention)."""
    x = np.asarray(x, dtype=np.float64)
    Hkv = x.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of the key/value heads")
    return np.repeat(x, H // Hkv, axis=1)


def varlen_attention(q, k, v, cu_q, cu_k, scale, causal=False):
    """Packed batch: q [Tq, H, d], k and v [Tk, Hkv, d]; sequence b holds
    query tokens cu_q[b] .. cu_q[b+1]-1 and keys cu_k[b] .. cu_k[b+1]-1.
    Each sequence is attention on its own tokens with its query rows at the
    end of its keys (end aligned, as ``attention``), heads grouped as
    ``expand_kv_heads``.  Returns (o [Tq, H, dv], lse [Tq, H])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, H, _ = q.shape
    o = np.zeros((Tq, H, v.shape[-1]))
    lse = np.full((Tq, H), NEG_INF)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        qb = q[q0:q1].transpose(1, 0, 2)[None]
        kb = expand_kv_heads(k[k0:k1].transpose(1, 0, 2)[None], H)
        vb = expand_kv_heads(v[k0:k1].transpose(1, 0, 2)[None], H)
        ob, lb = attention(qb, kb, vb, scale, causal=causal, end_aligned=True)
        o[q0:q1] = ob[0].transpose(1, 0, 2)
        lse[q0:q1] = lb[0].T
    return o, lse
