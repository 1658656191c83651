"""Pins for the fp64 gradient oracle (oracle.attention_backward).

The gradients are checked against things other than their own formulas:
central finite differences of the loss sum(dO * O) through the pinned
forward oracle, torch.autograd in float64 through a forward written here
with torch operations, closed forms for uniform scores, and invariants.
The last block plants plausible mistakes in a wrapped copy of the oracle
(dropped D term, missing scale, transposed score gradient, value gradient
from the wrong operand, D from the wrong axis) and checks that a pin fails.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def loss(q, k, v, do, scale, causal, key_len):
    o, _ = oracle.attention(q, k, v, scale, causal=causal, key_len=key_len)
    return float((do * o).sum())


def finite_difference(q, k, v, do, scale, causal, key_len, eps=1e-6):
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = loss(q, k, v, do, scale, causal, key_len)
            x[idx] = old - eps
            lm = loss(q, k, v, do, scale, causal, key_len)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal,L", list(itertools.product((False, True), (6, 4, 1, 0))))
def test_finite_differences(causal, L):
    B, H, N, d = 1, 2, 6, 3
    q, k, v, do = (rand((B, H, N, d), s) for s in (801, 802, 803, 804))
    key_len = np.array([L])
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.7, causal=causal, key_len=key_len)
    fq, fk, fv = finite_difference(q, k, v, do, 0.7, causal, key_len)
    for a, b, name in ((dq, fq, "dq"), (dk, fk, "dk"), (dv, fv, "dv")):
        assert np.allclose(a, b, atol=1e-8, rtol=0), (name, np.abs(a - b).max())


def torch_forward(q, k, v, scale, causal, key_len):
    """Masked attention written with torch operations (rows without a visible
    key give 0), for autograd."""
    B, H, N, d = q.shape
    s = scale * q @ k.transpose(-1, -2)
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    outs = []
    for b in range(B):
        L = N if key_len is None else max(0, min(int(key_len[b]), N))
        vis = (j < L) & (i < L)
        if causal:
            vis = vis & (j <= i)
        sb = s[b].masked_fill(~vis, float("-inf"))
        live = vis.any(dim=1)
        sb = torch.where(live[:, None], sb, torch.zeros_like(sb))
        p = torch.softmax(sb, dim=-1) * vis
        outs.append(p @ v[b])
    return torch.stack(outs)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_float64(causal):
    B, H, N, d = 3, 2, 33, 8
    q, k, v, do = (rand((B, H, N, d), s, 1.5) for s in (811, 812, 813, 814))
    key_len = np.array([33, 20, 0])
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch_forward(tq, tk, tv, 0.4, causal, key_len)
    (out * torch.tensor(do)).sum().backward()
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.4, causal=causal, key_len=key_len)
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_uniform_scores_closed_form():
    """q = 0: every visible key has weight 1/n_i.  Then dV_j = sum over rows
    that see j of dO_i / n_i, dK = 0, and dQ_i = scale/n_i * sum_j
    (dO_i . (v_j - mean_i v)) k_j."""
    B, H, N, d = 1, 1, 9, 4
    q = np.zeros((B, H, N, d))
    k, v, do = (rand((B, H, N, d), s) for s in (821, 822, 823))
    for causal in (False, True):
        dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.9, causal=causal)
        ev = np.zeros((N, d))
        eq = np.zeros((N, d))
        for i in range(N):
            keys = list(range(i + 1)) if causal else list(range(N))
            n = len(keys)
            vbar = v[0, 0, keys].mean(axis=0)
            for j in keys:
                ev[j] += do[0, 0, i] / n
                eq[i] += 0.9 / n * (do[0, 0, i] @ (v[0, 0, j] - vbar)) * k[0, 0, j]
        assert np.allclose(dv[0, 0], ev, atol=1e-14)
        assert np.allclose(dq[0, 0], eq, atol=1e-14)
        assert np.all(dk == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    B, H, N, d = 2, 3, 21, 5
    q, k, v, do = (rand((B, H, N, d), s, 2.0) for s in (831, 832, 833, 834))
    key_len = np.array([21, 9])
    dq, dk, dv, dvec = oracle.attention_backward(q, k, v, do, 0.5, causal=causal, key_len=key_len)
    # the scores of a row are unchanged by a common shift of the keys: the
    # key gradients of each (batch, head) sum to zero
    assert np.allclose(dk.sum(axis=2), 0, atol=1e-12)
    # a constant added to every value row changes no gradient
    c = rand((1, 1, 1, d), 835)
    dq2, dk2, dv2, _ = oracle.attention_backward(q, k, v + c, do, 0.5, causal=causal, key_len=key_len)
    assert np.allclose(dq, dq2, atol=1e-12) and np.allclose(dk, dk2, atol=1e-12)
    assert np.allclose(dv, dv2, atol=1e-12)
    # D_i = dO_i . O_i
    o, _ = oracle.attention(q, k, v, 0.5, causal=causal, key_len=key_len)
    assert np.allclose(dvec, (do * o).sum(axis=-1), atol=1e-12)
    # padding rows and keys past the length have zero gradients
    assert np.all(dq[1, :, 9:] == 0) and np.all(dk[1, :, 9:] == 0) and np.all(dv[1, :, 9:] == 0)
    if causal:
        # row 0 sees one key: its weight is 1 whatever the score, so dQ_0 = 0
        assert np.allclose(dq[:, :, 0], 0, atol=1e-15)


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------

def _mistaken_backward(mistake):
    def f(q, k, v, do, scale, causal=False, key_len=None):
        dq, dk, dv, dvec = oracle.attention_backward(q, k, v, do, scale, causal, key_len)
        if mistake == "dk_missing_scale":
            return dq, dk / scale, dv, dvec
        B, H, N, _ = q.shape
        o_dq, o_dk, o_dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            L = N if key_len is None else int(key_len[b])
            vis = oracle.visible_mask(np.arange(N), N, L, causal)
            for h in range(H):
                s = np.where(vis, scale * q[b, h] @ k[b, h].T, -np.inf)
                live = vis.any(axis=1)
                s = np.where(live[:, None], s, 0.0)
                w = np.where(vis, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
                p = w / np.where(live, w.sum(axis=1), 1.0)[:, None]
                dp = do[b, h] @ v[b, h].T
                D = (p * dp).sum(axis=1)
                if mistake == "no_d_term":
                    ds = p * dp
                elif mistake == "d_from_wrong_axis":
                    ds = p * (dp - (p * dp).sum(axis=0)[None, :])
                else:
                    ds = p * (dp - D[:, None])
                if mistake == "transposed_ds":
                    ds = ds.T
                o_dq[b, h] = scale * ds @ k[b, h]
                o_dk[b, h] = scale * ds.T @ q[b, h]
                o_dv[b, h] = (dp.T @ do[b, h]) if mistake == "dv_from_dp" else p.T @ do[b, h]
        return o_dq, o_dk, o_dv, dvec
    return f


def _pins_fail(bwd):
    B, H, N, d = 1, 1, 5, 3
    q, k, v, do = (rand((B, H, N, d), s) for s in (841, 842, 843, 844))
    for causal in (False, True):
        dq, dk, dv, _ = bwd(q, k, v, do, 0.8, causal=causal, key_len=np.array([N]))
        fq, fk, fv = finite_difference(q, k, v, do, 0.8, causal, np.array([N]))
        if not (np.allclose(dq, fq, atol=1e-7) and np.allclose(dk, fk, atol=1e-7)
                and np.allclose(dv, fv, atol=1e-7)):
            return True
    return False


def test_pins_pass_on_oracle():
    assert not _pins_fail(oracle.attention_backward)
    assert not _pins_fail(_mistaken_backward("none"))


@pytest.mark.parametrize("mistake", ["no_d_term", "dk_missing_scale", "transposed_ds",
                                     "dv_from_dp", "d_from_wrong_axis"])
def test_planted_mistakes_are_caught(mistake):
    assert _pins_fail(_mistaken_backward(mistake))


# ---------------------------------------------------------------------------
# Grouped key/value heads, end-aligned rows, packed batches
# ---------------------------------------------------------------------------

def _fd(params, loss_fn, eps=1e-6):
    """Central differences of loss_fn() with respect to every entry of the
    arrays in params (changed in place and restored)."""
    grads = []
    for x in params:
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = loss_fn()
            x[idx] = old - eps
            lm = loss_fn()
            x[idx] = old
            g[idx] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


def grouped_loss(q, k, v, do, scale, causal, key_len, end_aligned):
    H = q.shape[1]
    o, _ = oracle.attention(q, oracle.expand_kv_heads(k, H), oracle.expand_kv_heads(v, H), scale,
                            causal=causal, key_len=key_len, end_aligned=end_aligned)
    return float((do * o).sum())


GROUPED_SHAPES = [
    # (B, H, Hkv, Nq, Nk, key_len)
    (1, 4, 2, 3, 5, None),      # fewer rows than keys: positions 2..4
    (2, 4, 1, 4, 3, [3, 1]),    # more rows than keys: causal rows before key 0 see nothing
    (1, 2, 2, 4, 4, [2]),       # ungrouped, a length below Nk
    (1, 3, 1, 2, 4, [0]),       # no key at all
]


@pytest.mark.parametrize("shape", GROUPED_SHAPES, ids=lambda s: f"h{s[1]}kv{s[2]}q{s[3]}k{s[4]}")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("end_aligned", [True, False])
def test_grouped_finite_differences(shape, causal, end_aligned):
    B, H, Hkv, Nq, Nk, kl = shape
    key_len = None if kl is None else np.array(kl)
    q, do = (rand((B, H, Nq, 2), s) for s in (851, 852))
    k, v = (rand((B, Hkv, Nk, 2), s) for s in (853, 854))
    dq, dk, dv, _ = oracle.grouped_attention_backward(q, k, v, do, 0.9, causal=causal,
                                                      key_len=key_len, end_aligned=end_aligned)
    fq, fk, fv = _fd((q, k, v), lambda: grouped_loss(q, k, v, do, 0.9, causal, key_len, end_aligned))
    for a, b, name in ((dq, fq, "dq"), (dk, fk, "dk"), (dv, fv, "dv")):
        assert np.allclose(a, b, atol=1e-8, rtol=0), (name, np.abs(a - b).max())


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_reduces_to_square(causal):
    """Hkv = H, Nq = Nk and rows at their own positions: the pinned square
    backward."""
    B, H, N, d = 2, 3, 11, 4
    q, k, v, do = (rand((B, H, N, d), s, 1.5) for s in (861, 862, 863, 864))
    key_len = np.array([11, 6])
    want = oracle.attention_backward(q, k, v, do, 0.6, causal=causal, key_len=key_len)
    got = oracle.grouped_attention_backward(q, k, v, do, 0.6, causal=causal, key_len=key_len,
                                            end_aligned=False)
    for a, b in zip(got, want):
        assert np.allclose(a, b, atol=1e-13)


def test_grouped_wrong_head_mapping_is_caught(monkeypatch):
    """Planted: query head h reading key/value head h % Hkv (interleaved)
    instead of h // (H / Hkv) fails the finite-difference pin."""
    B, H, Hkv, Nq, Nk = 1, 4, 2, 3, 4
    q, do = (rand((B, H, Nq, 2), s) for s in (871, 872))
    k, v = (rand((B, Hkv, Nk, 2), s) for s in (873, 874))
    fq, fk, fv = _fd((q, k, v), lambda: grouped_loss(q, k, v, do, 0.9, True, None, True))
    monkeypatch.setattr("oracle.backward.kv_head_of", lambda h, H, Hkv: h % Hkv)
    dq, dk, dv, _ = oracle.grouped_attention_backward(q, k, v, do, 0.9, causal=True)
    assert not (np.allclose(dk, fk, atol=1e-7) and np.allclose(dv, fv, atol=1e-7)
                and np.allclose(dq, fq, atol=1e-7))


def test_grouped_rows_not_end_aligned_is_caught():
    """Planted: rows taken at their own positions when the forward puts them
    at the end of the keys fails the finite-difference pin."""
    B, H, Hkv, Nq, Nk = 1, 2, 1, 3, 6
    q, do = (rand((B, H, Nq, 2), s) for s in (881, 882))
    k, v = (rand((B, Hkv, Nk, 2), s) for s in (883, 884))
    fq, fk, fv = _fd((q, k, v), lambda: grouped_loss(q, k, v, do, 0.9, True, None, True))
    dq, dk, dv, _ = oracle.grouped_attention_backward(q, k, v, do, 0.9, causal=True,
                                                      end_aligned=False)
    assert not np.allclose(dk, fk, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_finite_differences(causal):
    """Packed batch with an empty query range, more rows than keys and a
    sequence without keys, through the packed forward oracle."""
    cu_q = np.array([0, 2, 2, 6, 7])
    cu_k = np.array([0, 3, 5, 7, 7])
    H, Hkv, d = 2, 1, 2
    q, do = (rand((cu_q[-1], H, d), s) for s in (891, 892))
    k, v = (rand((cu_k[-1], Hkv, d), s) for s in (893, 894))

    def loss_fn():
        o, _ = oracle.varlen_attention(q, k, v, cu_q, cu_k, 0.8, causal=causal)
        return float((do * o).sum())

    dq, dk, dv, dvec = oracle.varlen_attention_backward(q, k, v, do, cu_q, cu_k, 0.8, causal=causal)
    fq, fk, fv = _fd((q, k, v), loss_fn)
    for a, b, name in ((dq, fq, "dq"), (dk, fk, "dk"), (dv, fv, "dv")):
        assert np.allclose(a, b, atol=1e-8, rtol=0), (name, np.abs(a - b).max())
    # keys of the sequence without queries, and rows of the one without keys
    assert np.all(dk[3:5] == 0) and np.all(dv[3:5] == 0) and np.all(dq[6:7] == 0)
    # D_i = dO_i . O_i
    o, _ = oracle.varlen_attention(q, k, v, cu_q, cu_k, 0.8, causal=causal)
    assert np.allclose(dvec, (do * o).sum(axis=-1), atol=1e-12)


# ---------------------------------------------------------------------------
# Additive mask M (a constant of the loss)
# ---------------------------------------------------------------------------

def bias_loss(q, k, v, do, scale, causal, key_len, bias):
    o, _ = oracle.attention(q, k, v, scale, causal=causal, key_len=key_len, bias=bias)
    return float((do * o).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_bias_finite_differences(causal):
    B, H, N, d = 1, 2, 6, 3
    q, k, v, do = (rand((B, H, N, d), s) for s in (1101, 1102, 1103, 1104))
    bias = rand((1, H, N, N), 1105, 1.5)
    bias[0, 1, 2, :] = -np.inf            # a row hidden entirely by the mask
    bias[0, 0, 3, [0, 4]] = -np.inf       # two hidden pairs
    key_len = np.array([5])
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.7, causal=causal, key_len=key_len,
                                              bias=bias)
    fq, fk, fv = _fd((q, k, v), lambda: bias_loss(q, k, v, do, 0.7, causal, key_len, bias))
    for a, b, name in ((dq, fq, "dq"), (dk, fk, "dk"), (dv, fv, "dv")):
        assert np.allclose(a, b, atol=1e-8, rtol=0), (name, np.abs(a - b).max())
    assert np.all(dq[0, 1, 2] == 0)       # the hidden row has no gradient


def test_bias_invariants():
    B, H, N, d = 2, 2, 9, 4
    q, k, v, do = (rand((B, H, N, d), s) for s in (1111, 1112, 1113, 1114))
    plain = oracle.attention_backward(q, k, v, do, 0.5, causal=True)
    zero = oracle.attention_backward(q, k, v, do, 0.5, causal=True, bias=np.zeros((N, N)))
    # a constant per query row shifts every score of the row: nothing changes
    row_const = oracle.attention_backward(q, k, v, do, 0.5, causal=True,
                                          bias=rand((B, H, N, 1), 1115, 3.0))
    for a, b, c in zip(plain, zero, row_const):
        assert np.allclose(a, b, atol=1e-14) and np.allclose(a, c, atol=1e-12)


def test_bias_planted_mistake_is_caught():
    """Planted: the mask multiplying the weights instead of adding to the
    scores fails the finite-difference pin."""
    B, H, N, d = 1, 1, 5, 3
    q, k, v, do = (rand((B, H, N, d), s) for s in (1121, 1122, 1123, 1124))
    bias = rand((N, N), 1125)
    fq, fk, fv = _fd((q, k, v), lambda: bias_loss(q, k, v, do, 0.8, False, None, bias))
    wrong = oracle.attention_backward(q, k, v, do, 0.8, bias=np.log(np.abs(bias)))
    assert not np.allclose(wrong[0], fq, atol=1e-6)
