"""Pins for the dropout oracle (oracle/dropout.py).

The generator is pinned to the published known-answer vectors of
Philox4x32-10 (tests/golden/philox4x32_10_kat.json).  The attention with
dropout is pinned by p = 0 (the plain definition), the kept fraction (a
binomial bound), unbiasedness (the average over many offsets approaches the
undropped output), a closed form with uniform scores, and the mask's
distinct masks per head, batch entry, offset and seed.  Planted mistakes
(key words swapped, counter words swapped, the 1/(1-p) scale dropped) must
fail a pin.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import dropout as D

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")))


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def kat_fails(gen):
    for vec in GOLD["vectors"]:
        c = [np.uint64(int(x, 16)) for x in vec["counter"]]
        k = [int(x, 16) for x in vec["key"]]
        out = [int(x) for x in gen(c, k)]
        if out != [int(x, 16) for x in vec["output"]]:
            return True
    return False


def test_philox_known_answers():
    assert not kat_fails(D.philox4x32_10)


def test_philox_planted_mistakes():
    assert kat_fails(lambda c, k: D.philox4x32_10(c, (k[1], k[0])) if k[0] != k[1] else (0, 0, 0, 0))
    assert kat_fails(lambda c, k: D.philox4x32_10((c[1], c[0], c[2], c[3]), k))


def test_zero_rate_is_plain_attention():
    B, H, N, d = 2, 2, 37, 8
    q, k, v = rand((B, H, N, d), 1000), rand((B, H, N, d), 1001), rand((B, H, N, d), 1002)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, 0.3, causal=causal, key_len=np.array([37, 20]))
        o2, l2 = oracle.dropout_attention(q, k, v, 0.3, 0.0, seed=7, causal=causal,
                                          key_len=np.array([37, 20]))
        assert np.allclose(o1, o2, atol=1e-14) and np.array_equal(l1, l2)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_kept_fraction(p):
    keep = np.concatenate([D.dropout_keep(b, h, 4, 300, 300, p, 12345, 0).ravel()
                           for b in range(2) for h in range(4)])
    n = keep.size
    expect = 1.0 - math.floor(p * 2 ** 32) / 2 ** 32
    sd = math.sqrt(n * expect * (1 - expect))
    assert abs(keep.sum() - n * expect) < 5 * sd
    # different heads, batches, offsets and seeds give different masks
    a = D.dropout_keep(0, 0, 4, 64, 64, p, 1, 0)
    assert not np.array_equal(a, D.dropout_keep(0, 1, 4, 64, 64, p, 1, 0))
    assert not np.array_equal(a, D.dropout_keep(1, 0, 4, 64, 64, p, 1, 0))
    assert not np.array_equal(a, D.dropout_keep(0, 0, 4, 64, 64, p, 1, 1))
    assert not np.array_equal(a, D.dropout_keep(0, 0, 4, 64, 64, p, 2, 0))


def test_unbiased_over_offsets():
    """E[Z / (1 - p)] = 1: averaging over 2000 offsets approaches the
    undropped output, within a bound from the per-offset spread."""
    B, H, N, d = 1, 1, 12, 4
    q, k, v = rand((B, H, N, d), 1010), rand((B, H, N, d), 1011), rand((B, H, N, d), 1012)
    o_ref, _ = oracle.attention(q, k, v, 0.5, causal=True)
    outs = np.stack([oracle.dropout_attention(q, k, v, 0.5, 0.3, seed=99, offset=t, causal=True)[0]
                     for t in range(2000)])
    mean, sd = outs.mean(axis=0), outs.std(axis=0)
    assert np.all(np.abs(mean - o_ref) <= 5 * sd / math.sqrt(2000) + 1e-12)


def test_uniform_scores_closed_form():
    """q = 0: P_ij = 1/n_i over visible keys, so O_i = sum of the kept v_j
    divided by n_i (1 - p)."""
    B, H, N, d = 1, 2, 20, 3
    q = np.zeros((B, H, N, d))
    k, v = rand((B, H, N, d), 1020), rand((B, H, N, d), 1021)
    p, seed = 0.25, 2024
    o, _ = oracle.dropout_attention(q, k, v, 1.0, p, seed=seed, offset=5, causal=True)
    for h in range(H):
        Z = D.dropout_keep(0, h, H, N, N, p, seed, 5)
        for i in range(N):
            keys = [j for j in range(i + 1) if Z[i, j]]
            expect = v[0, h, keys].sum(axis=0) / ((i + 1) * (1 - p)) if keys else np.zeros(d)
            assert np.allclose(o[0, h, i], expect, atol=1e-14)


def test_planted_scale_mistake():
    B, H, N, d = 1, 1, 30, 4
    q, k, v = rand((B, H, N, d), 1030), rand((B, H, N, d), 1031), rand((B, H, N, d), 1032)
    o_ref, _ = oracle.attention(q, k, v, 0.5)
    outs = np.stack([oracle.dropout_attention(q, k, v, 0.5, 0.5, seed=3, offset=t)[0] * 0.5
                     for t in range(400)])  # 1/(1-p) dropped
    assert np.abs(outs.mean(axis=0) - o_ref).max() > 0.1


def test_head_selection_matches_full_problem():
    B, H, N, d = 2, 5, 16, 4
    q, k, v = rand((B, H, N, d), 1040), rand((B, H, N, d), 1041), rand((B, H, N, d), 1042)
    full, _ = oracle.dropout_attention(q, k, v, 0.5, 0.4, seed=8, offset=2, causal=True)
    part, _ = oracle.dropout_attention(q[:, [3, 1]], k[:, [3, 1]], v[:, [3, 1]], 0.5, 0.4, seed=8,
                                       offset=2, causal=True, head_ids=[3, 1], H_all=H)
    assert np.array_equal(part, full[:, [3, 1]])


# ---------------------------------------------------------------------------
# The gradient with dropout
# ---------------------------------------------------------------------------

def _fd_dropout(q, k, v, do, scale, p, seed, offset, causal, key_len, eps=1e-6):
    def loss():
        o, _ = oracle.dropout_attention(q, k, v, scale, p, seed, offset, causal=causal,
                                        key_len=key_len)
        return float((do * o).sum())
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = loss()
            x[idx] = old - eps
            lm = loss()
            x[idx] = old
            g[idx] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal,L", [(False, 7), (True, 7), (True, 4), (False, 0)])
def test_dropout_gradient_finite_differences(causal, L):
    B, H, N, d = 1, 2, 7, 3
    q, k, v, do = (rand((B, H, N, d), s) for s in (951, 952, 953, 954))
    key_len = np.array([L])
    dq, dk, dv, _ = oracle.dropout_attention_backward(q, k, v, do, 0.8, 0.3, 77, 5, causal=causal,
                                                      key_len=key_len)
    fq, fk, fv = _fd_dropout(q, k, v, do, 0.8, 0.3, 77, 5, causal, key_len)
    for a, b, name in ((dq, fq, "dq"), (dk, fk, "dk"), (dv, fv, "dv")):
        assert np.allclose(a, b, atol=1e-8, rtol=0), (name, np.abs(a - b).max())


def test_dropout_gradient_zero_rate_is_plain_gradient():
    B, H, N, d = 2, 2, 9, 4
    q, k, v, do = (rand((B, H, N, d), s) for s in (961, 962, 963, 964))
    key_len = np.array([9, 5])
    for causal in (False, True):
        got = oracle.dropout_attention_backward(q, k, v, do, 0.5, 0.0, 3, 0, causal=causal,
                                                key_len=key_len)
        want = oracle.attention_backward(q, k, v, do, 0.5, causal=causal, key_len=key_len)
        for a, b in zip(got, want):
            assert np.allclose(a, b, atol=1e-13)


def test_dropout_gradient_d_is_do_dot_o():
    B, H, N, d = 1, 3, 11, 4
    q, k, v, do = (rand((B, H, N, d), s) for s in (971, 972, 973, 974))
    _, _, _, dvec = oracle.dropout_attention_backward(q, k, v, do, 0.6, 0.25, 9, 2, causal=True)
    o, _ = oracle.dropout_attention(q, k, v, 0.6, 0.25, 9, 2, causal=True)
    assert np.allclose(dvec, (do * o).sum(axis=-1), atol=1e-12)


def test_dropout_gradient_planted_mistakes():
    """Plausible mistakes fail the finite-difference pin: the mask or the
    1/(1-p) factor left out of dP (the value gradient alone is still right)."""
    B, H, N, d = 1, 1, 6, 3
    q, k, v, do = (rand((B, H, N, d), s) for s in (981, 982, 983, 984))
    fq, fk, fv = _fd_dropout(q, k, v, do, 0.8, 0.3, 11, 0, False, None)
    # dP without the mask: the undropped gradient scaled by 1/(1-p)
    wrong_q = oracle.attention_backward(q, k, v, do / 0.7, 0.8)[0]
    assert not np.allclose(wrong_q, fq, atol=1e-6)
    # dP masked but not rescaled: reproduce by scaling dO for dP only
    Z = D.dropout_keep(0, 0, 1, N, N, 0.3, 11, 0)
    s = 0.8 * q[0, 0] @ k[0, 0].T
    P = np.exp(s - s.max(axis=1, keepdims=True)); P /= P.sum(axis=1, keepdims=True)
    dP = Z * (do[0, 0] @ v[0, 0].T)
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    assert not np.allclose(0.8 * dS @ k[0, 0], fq[0, 0], atol=1e-6)
    got = oracle.dropout_attention_backward(q, k, v, do, 0.8, 0.3, 11, 0)
    assert np.allclose(got[0], fq, atol=1e-8)


def test_dropout_gradient_head_selection_matches_full_problem():
    B, H, N, d = 2, 3, 8, 3
    q, k, v, do = (rand((B, H, N, d), s) for s in (991, 992, 993, 994))
    full = oracle.dropout_attention_backward(q, k, v, do, 0.7, 0.4, 21, 3, causal=True)
    for b, h in ((1, 2), (0, 1)):
        sl = lambda x: x[b:b + 1, h:h + 1]
        part = oracle.dropout_attention_backward(sl(q), sl(k), sl(v), sl(do), 0.7, 0.4, 21, 3,
                                                 causal=True, head_ids=[h], H_all=H, batch_ids=[b])
        for a, c in zip(part, full):
            assert np.allclose(a[0, 0], c[b, h], atol=1e-14)


# ---- the keep threshold: one definition, pinned by exact rational arithmetic ----

GAP = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dropout_gap_draws.json")))


@pytest.mark.parametrize("p", [0.0, 0.1, 0.2, 0.3, 0.5, 0.9, 0.123456789, 1.0 - 2.0 ** -53])
def test_keep_threshold_is_floor_of_exact_product(p):
    """floor(p * 2^32) of the binary64 rate, computed here with Fractions
    (exact rationals), equals the oracle's threshold."""
    assert D.keep_threshold(p) == math.floor(Fraction(p) * 2 ** 32)


def test_keep_threshold_values():
    """Hand-derived values: 0.3 is 0.29999999999999998889776975... in
    binary64, times 2^32 is 1288490188.79..., so the threshold is
    1288490188; rounded to binary32 first the rate would be
    0.300000011920928955078125, giving exactly 1288490240 (a planted
    misreading that the pin rejects)."""
    assert D.keep_threshold(0.0) == 0
    assert D.keep_threshold(0.5) == 2 ** 31
    assert D.keep_threshold(0.1) == 429496729
    assert D.keep_threshold(0.3) == 1288490188
    assert D.keep_threshold(0.9) == 3865470566
    assert D.keep_threshold(float(np.float32(0.3))) == 1288490240 != D.keep_threshold(0.3)
    assert D.keep_threshold(float(np.float32(0.9))) == 3865470464 != D.keep_threshold(0.9)


@pytest.mark.parametrize("case", GAP["cases"], ids=lambda c: f"p{c['p']}")
def test_gap_draws(case):
    """The stored draws (tests/golden/make_dropout_gap_draws.py) lie between
    the two readings' thresholds, and dropout_keep decides them by the
    binary64 rate: the GPU test on them fails if the library rounds the rate
    to binary32."""
    p, n, seed = case["p"], case["n"], case["seed"]
    i, j, off = case["row"], case["key"], case["offset"]
    words = D.philox4x32_10((j // 4, i, 0, off), (seed & 0xFFFFFFFF, seed >> 32))
    u = int(words[j % 4])
    assert u == case["draw"]
    t64, t32 = D.keep_threshold(p), D.keep_threshold(float(np.float32(p)))
    assert min(t64, t32) <= u < max(t64, t32)
    keep = D.dropout_keep(0, 0, 1, n, n, p, seed, off)
    assert bool(keep[i, j]) == (u >= t64) == case["kept"]
