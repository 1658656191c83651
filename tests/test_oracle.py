"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Nothing here compares the oracle with itself.  The pins are: the glossary
page's two worked examples with every printed intermediate (tests/golden),
closed forms (uniform scores, causal running means, single visible key,
dominant key), invariants (convex hull, shift and permutation invariance),
scipy's softmax on the unmasked case, pure-Python brute force with exact
summation and no max shift on tiny inputs, and equality of the plain
definition with the streamed (m, l, a) recurrence.  The last block plants
plausible mistakes (dropped scale, transposed operand, flipped causal
direction, unmasked padding, wrong value operand, query rows of a key cache
placed at the wrong positions) and checks that a pin fails.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def frac(x):
    return x[0] / x[1]


def logs(spec):
    return [math.log(t) for t in spec["log_of"]]


def as_bhnd(x):
    """1-D sequence of scalars -> [1, 1, n, 1] fp64."""
    return np.asarray(x, dtype=np.float64).reshape(1, 1, -1, 1)


def scalar_row(scores, values, causal=False):
    """One query whose scores are exactly `scores`: q = [1], k_j = s_j, scale 1."""
    q = np.ones((1, 1, 1, 1))
    k = as_bhnd(scores)
    v = as_bhnd(values)
    # a single query row against n keys: pad the query side to n rows and
    # look at the last row (sees every key, also under the causal mask)
    n = k.shape[2]
    qq = np.ones((1, 1, n, 1))
    o, lse = oracle.attention(qq, k, v, 1.0, causal=causal)
    return o[0, 0, -1, 0], lse[0, 0, -1]


# ---------------------------------------------------------------------------
# Worked examples printed by the glossary page
# ---------------------------------------------------------------------------

def test_two_ways_direct_softmax():
    ex = GOLD["example_two_ways"]
    o, lse = scalar_row(logs(ex["scores"]), ex["values"])
    assert o == pytest.approx(frac(ex["output"]), abs=1e-13)
    assert lse == pytest.approx(math.log(ex["lse"]["log_of"]), abs=1e-13)
    # weights (1, 2, 3) / 6
    s = np.array(logs(ex["scores"]))
    w = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    assert np.allclose(w, [frac(x) for x in ex["softmax_weights"]], atol=1e-15)


def test_two_ways_block_summaries_and_merge():
    ex = GOLD["example_two_ways"]
    s = logs(ex["scores"])
    vals = ex["values"]
    c = ex["split_after"]
    A = oracle.block_summary(s[:c], vals[:c])
    B = oracle.block_summary(s[c:], vals[c:])
    assert A[0] == pytest.approx(math.log(ex["block_a"]["m"]["log_of"]), abs=1e-15)
    assert A[1] == pytest.approx(frac(ex["block_a"]["l"]), abs=1e-15)
    assert A[2][0] == pytest.approx(frac(ex["block_a"]["u"]), abs=1e-15)
    assert B[0] == pytest.approx(math.log(ex["block_b"]["m"]["log_of"]), abs=1e-15)
    assert B[1] == pytest.approx(frac(ex["block_b"]["l"]), abs=1e-15)
    assert B[2][0] == pytest.approx(frac(ex["block_b"]["u"]), abs=1e-15)
    # raising A's reference maximum to ln 3 multiplies its sums by 2/3
    assert math.exp(A[0] - B[0]) == pytest.approx(frac(ex["rescale_a_to_common_max"]), abs=1e-15)
    M = oracle.merge_summaries(A, B)
    assert M[0] == pytest.approx(math.log(ex["merged"]["m"]["log_of"]), abs=1e-15)
    assert M[1] == pytest.approx(frac(ex["merged"]["l"]), abs=1e-14)
    assert M[2][0] == pytest.approx(frac(ex["merged"]["u"]), abs=1e-14)
    o, lse = oracle.finalize_summary(M)
    assert o[0] == pytest.approx(frac(ex["merged"]["o"]), abs=1e-14)
    assert lse == pytest.approx(math.log(6.0), abs=1e-14)
    # merge order does not matter
    M2 = oracle.merge_summaries(B, A)
    assert oracle.finalize_summary(M2)[0][0] == pytest.approx(17 / 6, abs=1e-14)
    # adding the sums without the rescale gives the page's wrong 2.6
    wrong = (A[2][0] + B[2][0]) / (A[1] + B[1])
    assert wrong == pytest.approx(frac(ex["unrescaled_merge_wrong"]), abs=1e-14)
    assert abs(wrong - 17 / 6) > 0.2


def test_practice_example():
    ex = GOLD["example_practice"]
    s = logs(ex["scores"])
    vals = ex["values"]
    o, lse = scalar_row(s, vals)
    assert o == pytest.approx(frac(ex["output"]), abs=1e-13)
    assert lse == pytest.approx(math.log(ex["lse"]["log_of"]), abs=1e-13)
    c = ex["split_after"]
    A = oracle.block_summary(s[:c], vals[:c])
    B = oracle.block_summary(s[c:], vals[c:])
    oa, _ = oracle.finalize_summary(A)
    ob, _ = oracle.finalize_summary(B)
    assert oa[0] == pytest.approx(frac(ex["block_outputs"][0]), abs=1e-14)
    assert ob[0] == pytest.approx(frac(ex["block_outputs"][1]), abs=1e-14)
    # masses relative to the unshifted exponentials: l * exp(m)
    assert A[1] * math.exp(A[0]) == pytest.approx(frac(ex["block_masses_unshifted"][0]), abs=1e-13)
    assert B[1] * math.exp(B[0]) == pytest.approx(frac(ex["block_masses_unshifted"][1]), abs=1e-13)
    M = oracle.merge_summaries(A, B)
    assert M[0] == pytest.approx(math.log(3), abs=1e-15)
    assert M[1] == pytest.approx(frac(ex["merged_at_common_max"]["l"]), abs=1e-14)
    assert M[2][0] == pytest.approx(frac(ex["merged_at_common_max"]["u"]), abs=1e-13)
    assert oracle.finalize_summary(M)[0][0] == pytest.approx(20 / 3, abs=1e-13)
    avg = (oa[0] + ob[0]) / 2
    assert avg == pytest.approx(frac(ex["simple_average_wrong"]), abs=1e-14)
    assert abs(avg - 20 / 3) > 0.5


def test_worked_examples_through_streamed_recurrence():
    """The streamed recurrence, split after the second score, passes through
    exactly the printed intermediate state and ends at 17/6."""
    ex = GOLD["example_two_ways"]
    s = logs(ex["scores"])
    n = len(s)
    q = np.ones((1, 1, n, 1))
    trace = []
    o, lse = oracle.streamed_attention(q, as_bhnd(s), as_bhnd(ex["values"]), 1.0,
                                       block_q=n, block_k=ex["split_after"], trace=trace)
    assert o[0, 0, -1, 0] == pytest.approx(17 / 6, abs=1e-14)
    # after block A (last query row sees both of its keys)
    _, _, m, ell, a = trace[0]
    assert m[-1] == pytest.approx(math.log(2), abs=1e-15)
    assert ell[-1] == pytest.approx(1.5, abs=1e-15)
    assert a[-1, 0] == pytest.approx(2.5, abs=1e-15)
    _, _, m, ell, a = trace[1]
    assert m[-1] == pytest.approx(math.log(3), abs=1e-15)
    assert ell[-1] == pytest.approx(2.0, abs=1e-14)
    assert a[-1, 0] == pytest.approx(17 / 3, abs=1e-14)
    ex2 = GOLD["example_practice"]
    o2, _ = oracle.streamed_attention(q, as_bhnd(logs(ex2["scores"])), as_bhnd(ex2["values"]), 1.0,
                                      block_q=n, block_k=2)
    assert o2[0, 0, -1, 0] == pytest.approx(20 / 3, abs=1e-13)


def test_score_tile_size_arithmetic():
    g = GOLD["score_tile_size"]
    assert g["block_q"] * g["block_k"] == g["entries"]
    g = GOLD["materialised_score_matrix"]
    pairs = g["B"] * g["H"] * g["N"] ** 2
    assert abs(pairs - g["approx_pairs"]) / g["approx_pairs"] < 0.05
    assert pairs * g["bytes_per_element"] / 2 ** 30 == pytest.approx(g["approx_gib"])


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_uniform_scores_give_mean_of_values():
    B, H, N, d = 2, 3, 17, 5
    q = np.zeros((B, H, N, d))
    k = rand((B, H, N, d), 1)
    v = rand((B, H, N, d), 2)
    o, lse = oracle.attention(q, k, v, 0.3)
    assert np.allclose(o, v.mean(axis=2, keepdims=True), atol=1e-14)
    assert np.allclose(lse, math.log(N), atol=1e-14)


def test_uniform_scores_causal_running_mean():
    B, H, N, d = 1, 2, 23, 4
    q = np.zeros((B, H, N, d))
    k = rand((B, H, N, d), 3)
    v = rand((B, H, N, d), 4)
    o, lse = oracle.attention(q, k, v, 0.125, causal=True)
    run = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    assert np.allclose(o, run, atol=1e-13)
    assert np.allclose(lse, np.log(np.arange(1, N + 1))[None, None], atol=1e-13)


def test_uniform_scores_key_length():
    B, H, N, d = 4, 2, 19, 3
    q = np.zeros((B, H, N, d))
    k = rand((B, H, N, d), 5)
    v = rand((B, H, N, d), 6)
    key_len = np.array([0, 1, 7, 40], dtype=np.int32)  # 40 clamps to N
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.5, causal=causal, key_len=key_len)
        for b, L in enumerate(key_len):
            L = min(int(L), N)
            for i in range(N):
                if i >= L:
                    assert np.all(o[b, :, i] == 0.0)
                    assert np.all(lse[b, :, i] == -np.inf)
                    continue
                hi = i + 1 if causal else L
                assert np.allclose(o[b, :, i], v[b, :, :hi].mean(axis=1), atol=1e-13)
                assert np.allclose(lse[b, :, i], math.log(hi), atol=1e-13)


def test_single_visible_key():
    B, H, N, d = 1, 2, 9, 6
    q, k, v = rand((B, H, N, d), 7), rand((B, H, N, d), 8), rand((B, H, N, d), 9)
    scale = 0.37
    o, lse = oracle.attention(q, k, v, scale, causal=True)
    # causal row 0 sees only key 0
    assert np.allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)
    assert np.allclose(lse[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-14)
    # key length 1: row 0 sees key 0, every other row is padding
    o, lse = oracle.attention(q, k, v, scale, key_len=np.array([1]))
    assert np.allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)
    assert np.all(o[:, :, 1:] == 0) and np.all(lse[:, :, 1:] == -np.inf)
    # N = 1
    o, lse = oracle.attention(q[:, :, :1], k[:, :, :1], v[:, :, :1], scale)
    assert np.allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)


def test_dominant_key_selects_its_value():
    """One score 60 above all others: O is that key's value to fp64 precision."""
    B, H, N, d = 1, 2, 31, 4
    rng = np.random.default_rng(10)
    e = np.zeros(d)
    e[1] = 1.0
    q = np.broadcast_to(e, (B, H, N, d)).copy()
    k = rng.standard_normal((B, H, N, d)) * 0.01
    v = rng.standard_normal((B, H, N, d))
    j = 29
    k[:, :, j] = 60.0 * e
    o, lse = oracle.attention(q, k, v, 1.0)
    assert np.allclose(o, v[:, :, j:j + 1], atol=1e-15, rtol=0)
    # exp(-59.9) corrections are far below fp64 resolution of 60
    assert np.allclose(lse, 60.0, atol=1e-14, rtol=0)


def test_large_scores_no_overflow():
    """Scores of order 1e4 would overflow exp without the max shift."""
    B, H, N, d = 1, 1, 16, 8
    q = rand((B, H, N, d), 11, 100.0)
    k = rand((B, H, N, d), 12, 100.0)
    v = rand((B, H, N, d), 13)
    o, lse = oracle.attention(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    s = q[0, 0] @ k[0, 0].T
    assert np.allclose(lse[0, 0], s.max(axis=1) + np.log(np.exp(s - s.max(axis=1, keepdims=True)).sum(1)),
                       rtol=1e-15, atol=1e-9)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_convex_hull(causal):
    B, H, N, d = 2, 2, 40, 8
    q, k, v = rand((B, H, N, d), 14, 2.0), rand((B, H, N, d), 15), rand((B, H, N, d), 16)
    key_len = np.array([40, 13])
    o, _ = oracle.attention(q, k, v, 0.5, causal=causal, key_len=key_len)
    for b in range(B):
        L = int(key_len[b])
        for i in range(L):
            hi = i + 1 if causal else L
            lo_v = v[b, :, :hi].min(axis=1)
            hi_v = v[b, :, :hi].max(axis=1)
            assert np.all(o[b, :, i] >= lo_v - 1e-13) and np.all(o[b, :, i] <= hi_v + 1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    """K' = K + 1 w^T adds scale * (q_i . w) to every score of row i:
    O is unchanged and LSE moves by that amount."""
    B, H, N, d = 1, 2, 33, 8
    q, k, v = rand((B, H, N, d), 17), rand((B, H, N, d), 18), rand((B, H, N, d), 19)
    w = rand((d,), 20)
    scale = 0.4
    o1, l1 = oracle.attention(q, k, v, scale, causal=causal)
    o2, l2 = oracle.attention(q, k + w, v, scale, causal=causal)
    assert np.allclose(o1, o2, atol=1e-12)
    assert np.allclose(l2 - l1, scale * (q @ w), atol=1e-12)


def test_key_value_permutation_invariance():
    B, H, N, d = 1, 2, 29, 6
    q, k, v = rand((B, H, N, d), 21), rand((B, H, N, d), 22), rand((B, H, N, d), 23)
    perm = np.random.default_rng(24).permutation(N)
    o1, l1 = oracle.attention(q, k, v, 0.3)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.3)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_rows_argument_matches_full():
    B, H, N, d = 2, 3, 50, 4
    q, k, v = rand((B, H, N, d), 25), rand((B, H, N, d), 26), rand((B, H, N, d), 27)
    key_len = np.array([50, 21])
    o, lse = oracle.attention(q, k, v, 0.2, causal=True, key_len=key_len)
    rows = np.stack([np.sort(np.random.default_rng(28 + h).choice(N, 7, replace=False)) for h in range(H)])
    o2, l2 = oracle.attention(q, k, v, 0.2, causal=True, key_len=key_len, rows=rows)
    for h in range(H):
        assert np.array_equal(o2[:, h], o[:, h, rows[h]])
        assert np.array_equal(l2[:, h], lse[:, h, rows[h]])


# ---------------------------------------------------------------------------
# Library routine and brute force
# ---------------------------------------------------------------------------

def test_matches_scipy_softmax_unmasked():
    B, H, N, d = 2, 2, 37, 16
    q, k, v = rand((B, H, N, d), 29), rand((B, H, N, d), 30), rand((B, H, N, d), 31)
    scale = 1 / 4
    o, lse = oracle.attention(q, k, v, scale)
    s = scale * q @ np.swapaxes(k, -1, -2)
    ref = scipy.special.softmax(s, axis=-1) @ v
    assert np.allclose(o, ref, atol=1e-14)
    assert np.allclose(lse, scipy.special.logsumexp(s, axis=-1), atol=1e-13)


def brute(q, k, v, scale, causal, L, end_aligned=False):
    """Direct definition with exact summation and no max shift, pure Python.

    q: nested list [Nq][d]; k, v: [Nk][d].  Query row i sits at key position
    p = i, or p = i + L - Nq when end_aligned; key j is visible iff j < L,
    p < L and (not causal or j <= p).  Returns (o [Nq][dv], lse [Nq]).
    """
    Nq, Nk = len(q), len(k)
    d = len(q[0])
    dv = len(v[0]) if Nk else 1
    O, LSE = [], []
    for i in range(Nq):
        p = i + (L - Nq if end_aligned else 0)
        keys = [j for j in range(Nk) if j < L and p < L and (not causal or j <= p)]
        if not keys:
            O.append([0.0] * dv)
            LSE.append(-math.inf)
            continue
        e = {j: math.exp(scale * math.fsum(q[i][c] * k[j][c] for c in range(d))) for j in keys}
        den = math.fsum(e.values())
        O.append([math.fsum(e[j] * v[j][c] for j in keys) / den for c in range(dv)])
        LSE.append(math.log(den))
    return O, LSE


@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 2), (8, 4), (7, 3)])
def test_brute_force_all_masks(N, d):
    rng = np.random.default_rng(100 + N * 10 + d)
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d + 1))  # value width differs from d
    scale = 0.7
    for causal, L in itertools.product((False, True), range(0, N + 2)):
        o, lse = oracle.attention(q, k, v, scale, causal=causal, key_len=np.array([L]))
        O, LSE = brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale, causal, min(L, N))
        assert np.allclose(o[0, 0], np.array(O), atol=1e-13, rtol=0)
        for a, b in zip(lse[0, 0], LSE):
            if b == -math.inf:
                assert a == -math.inf
            else:
                assert abs(a - b) < 1e-13


def test_brute_force_exact_rationals():
    """With scores ln(n) the weights are rational: check O exactly in Fractions."""
    # q = 1 (d = 1), k_j = ln(w_j): weights proportional to w_j
    wts = [1, 4, 2, 7, 3]
    vals = [3, -1, 5, 2, 8]
    N = len(wts)
    q = np.ones((1, 1, N, 1))
    k = as_bhnd([math.log(w) for w in wts])
    v = as_bhnd(vals)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 1.0, causal=causal)
        for i in range(N):
            hi = i + 1 if causal else N
            exact = Fraction(sum(w * x for w, x in zip(wts[:hi], vals[:hi])), sum(wts[:hi]))
            assert o[0, 0, i, 0] == pytest.approx(float(exact), abs=1e-14)
            assert lse[0, 0, i] == pytest.approx(math.log(sum(wts[:hi])), abs=1e-14)


# ---------------------------------------------------------------------------
# Query rows at the end of a longer key cache (decode, chunked prefill)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Nq,Nk,d", [(1, 1, 2), (1, 6, 3), (3, 7, 2), (6, 3, 2), (4, 4, 3), (2, 0, 2)])
def test_brute_force_end_aligned(Nq, Nk, d):
    rng = np.random.default_rng(700 + 10 * Nq + Nk)
    q = rng.standard_normal((1, 1, Nq, d))
    k = rng.standard_normal((1, 1, Nk, d))
    v = rng.standard_normal((1, 1, Nk, d + 1))
    for causal, L in itertools.product((False, True), range(0, Nk + 2)):
        o, lse = oracle.attention(q, k, v, 0.8, causal=causal, key_len=np.array([L]), end_aligned=True)
        O, LSE = brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.8, causal,
                       min(L, Nk), end_aligned=True)
        assert np.allclose(o[0, 0], np.array(O).reshape(Nq, -1)[:, :d + 1], atol=1e-13), (causal, L)
        for a, b in zip(lse[0, 0], LSE):
            assert (a == b == -math.inf) or abs(a - b) < 1e-13, (causal, L)


@pytest.mark.parametrize("causal", [False, True])
def test_end_aligned_without_length_is_square_when_nq_equals_nk(causal):
    B, H, N, d = 2, 2, 33, 5
    q, k, v = rand((B, H, N, d), 710), rand((B, H, N, d), 711), rand((B, H, N, d), 712)
    o1, l1 = oracle.attention(q, k, v, 0.3, causal=causal)
    o2, l2 = oracle.attention(q, k, v, 0.3, causal=causal, end_aligned=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_rows_are_softmax_over_cached_keys():
    """Nq = 1 at position L - 1 sees exactly the first L keys, causal or not:
    scipy's softmax and logsumexp over those scores."""
    B, H, Nk, d = 4, 3, 50, 8
    q, k, v = rand((B, H, 1, d), 720), rand((B, H, Nk, d), 721), rand((B, H, Nk, d), 722)
    key_len = np.array([50, 1, 0, 17])
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.4, causal=causal, key_len=key_len, end_aligned=True)
        for b, L in enumerate(key_len):
            for h in range(H):
                if L == 0:
                    assert np.all(o[b, h] == 0) and lse[b, h, 0] == -math.inf
                    continue
                s = 0.4 * k[b, h, :L] @ q[b, h, 0]
                assert np.allclose(o[b, h, 0], scipy.special.softmax(s) @ v[b, h, :L], atol=1e-14)
                assert abs(lse[b, h, 0] - scipy.special.logsumexp(s)) < 1e-13


@pytest.mark.parametrize("Nq", [1, 6, 23, 40])
def test_end_aligned_rows_match_square_problem(Nq):
    """Causal: row i at p = i + L - Nq equals row p of the square causal
    problem over the first L keys (whose other query rows are arbitrary);
    rows with p < 0 see nothing.  Non-causal: every row is the softmax over
    the first L keys."""
    B, H, Nk, d = 3, 2, 30, 4
    q, k, v = rand((B, H, Nq, d), 730), rand((B, H, Nk, d), 731), rand((B, H, Nk, d), 732)
    key_len = np.array([30, 11, 0])
    oc, lc = oracle.attention(q, k, v, 0.5, causal=True, key_len=key_len, end_aligned=True)
    on, ln_ = oracle.attention(q, k, v, 0.5, causal=False, key_len=key_len, end_aligned=True)
    rng = np.random.default_rng(733)
    for b, L in enumerate(key_len):
        for h in range(H):
            for i in range(Nq):
                p = i + L - Nq
                if L == 0 or p < 0:
                    assert np.all(oc[b, h, i] == 0) and lc[b, h, i] == -math.inf
                    if L == 0:
                        assert np.all(on[b, h, i] == 0) and ln_[b, h, i] == -math.inf
                    continue
                qs = rng.standard_normal((1, 1, L, d))
                qs[0, 0, p] = q[b, h, i]
                o_sq, l_sq = oracle.attention(qs, k[b:b + 1, h:h + 1, :L], v[b:b + 1, h:h + 1, :L],
                                              0.5, causal=True)
                assert np.allclose(oc[b, h, i], o_sq[0, 0, p], atol=1e-14)
                assert abs(lc[b, h, i] - l_sq[0, 0, p]) < 1e-13
            for i in range(Nq):
                if L == 0:
                    continue
                s = 0.5 * k[b, h, :L] @ q[b, h, i]
                assert np.allclose(on[b, h, i], scipy.special.softmax(s) @ v[b, h, :L], atol=1e-14)


@pytest.mark.parametrize("split_keys", [1, 3, 8, 16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_split_ranges_merged_equal_definition(split_keys, causal):
    """Key ranges summarised separately and merged (including ranges that
    are wholly masked) give the plain definition."""
    B, H, Nq, Nk, d = 3, 2, 9, 37, 4
    q, k, v = rand((B, H, Nq, d), 740, 2.0), rand((B, H, Nk, d), 741), rand((B, H, Nk, d), 742)
    key_len = np.array([37, 5, 0])
    o1, l1 = oracle.attention(q, k, v, 0.6, causal=causal, key_len=key_len, end_aligned=True)
    o2, l2 = oracle.split_attention(q, k, v, 0.6, causal=causal, key_len=key_len,
                                    split_keys=split_keys)
    assert np.allclose(o1, o2, atol=1e-13, rtol=0)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    assert np.allclose(l1[fin], l2[fin], atol=1e-13)


def test_split_average_of_block_outputs_is_wrong():
    """Averaging the ranges' normalised outputs (the error the glossary page
    warns about) differs from the merged result."""
    rng = np.random.default_rng(750)
    q = rng.standard_normal((1, 1, 1, 4)) * 3
    k = rng.standard_normal((1, 1, 8, 4))
    v = rng.standard_normal((1, 1, 8, 2))
    o, _ = oracle.split_attention(q, k, v, 1.0, split_keys=4)
    parts = [oracle.attention(q, k[:, :, a:a + 4], v[:, :, a:a + 4], 1.0, end_aligned=True)[0]
             for a in (0, 4)]
    assert not np.allclose(o, 0.5 * (parts[0] + parts[1]), atol=1e-3)


# ---------------------------------------------------------------------------
# The streamed recurrence equals the plain definition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bq,bk", [(1, 1), (4, 3), (16, 16), (7, 64), (64, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_streamed_equals_definition(bq, bk, causal):
    B, H, N, d = 3, 2, 45, 8
    rng = np.random.default_rng(200 + bq * 7 + bk)
    q = rng.standard_normal((B, H, N, d)) * 3
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    key_len = np.array([45, 0, 11])  # full, empty, and ragged
    o1, l1 = oracle.attention(q, k, v, 0.35, causal=causal, key_len=key_len)
    o2, l2 = oracle.streamed_attention(q, k, v, 0.35, causal=causal, key_len=key_len,
                                       block_q=bq, block_k=bk)
    assert np.allclose(o1, o2, atol=1e-12, rtol=0)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    assert np.allclose(l1[fin], l2[fin], atol=1e-12)
    assert np.all(o2[~fin] == 0)


def test_streamed_dominant_key_in_last_block():
    """A much larger score arriving in the last block forces a large rescale."""
    B, H, N, d = 1, 1, 64, 4
    rng = np.random.default_rng(300)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    k[0, 0, N - 1] = 30.0 * q[0, 0].mean(axis=0) / np.linalg.norm(q[0, 0].mean(axis=0))
    o1, l1 = oracle.attention(q, k, v, 1.0)
    o2, l2 = oracle.streamed_attention(q, k, v, 1.0, block_q=16, block_k=8)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


def test_fully_masked_block_summary_merge():
    A = oracle.block_summary([-math.inf, -math.inf], [1.0, 2.0])
    assert A[0] == -math.inf and A[1] == 0.0 and A[2][0] == 0.0
    B = oracle.block_summary([0.0, math.log(3)], [2.0, 6.0])
    M = oracle.merge_summaries(A, B)
    assert oracle.finalize_summary(M)[0][0] == pytest.approx(5.0, abs=1e-14)
    E = oracle.merge_summaries(A, A)
    o, lse = oracle.finalize_summary(E)
    assert o[0] == 0.0 and lse == -math.inf


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible error in the oracle fails some pin above.
# The mistakes are planted by wrapping the oracle (never the HIP path).
# ---------------------------------------------------------------------------

def _pin_suite(attn):
    """Returns the names of the pins that `attn` (same signature as
    oracle.attention) fails."""
    failed = []
    ex = GOLD["example_two_ways"]
    s = logs(ex["scores"])
    n = len(s)
    o, _ = attn(np.ones((1, 1, n, 1)), as_bhnd(s), as_bhnd(ex["values"]), 1.0)
    if abs(o[0, 0, -1, 0] - 17 / 6) > 1e-12:
        failed.append("two_ways")
    B, H, N, d = 1, 1, 9, 3
    rng = np.random.default_rng(0)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    for causal, L in itertools.product((False, True), (N, 4)):
        o, lse = attn(q, k, v, 0.6, causal=causal, key_len=np.array([L]))
        O, LSE = brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.6, causal, L)
        if not np.allclose(o[0, 0], np.array(O), atol=1e-12):
            failed.append(f"brute_{causal}_{L}")
    # three query rows at the end of a nine-key cache holding 7 (then 2) keys
    qd = rng.standard_normal((B, H, 3, d))
    for causal, L in itertools.product((False, True), (7, 2)):
        try:
            o, lse = attn(qd, k, v, 0.6, causal=causal, key_len=np.array([L]), end_aligned=True)
            ok = o.shape == (1, 1, 3, d)
        except (ValueError, IndexError):
            ok = False
        if ok:
            O, LSE = brute(qd[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.6, causal, L,
                           end_aligned=True)
            ok = np.allclose(o[0, 0], np.array(O), atol=1e-12)
        if not ok:
            failed.append(f"brute_end_{causal}_{L}")
    return failed


def test_pins_pass_on_oracle():
    assert _pin_suite(oracle.attention) == []


@pytest.mark.parametrize("mistake", ["dropped_scale", "transposed_qk", "flipped_causal",
                                     "unmasked_padding_rows", "wrong_value_operand",
                                     "start_aligned_cache_rows", "rows_aligned_to_capacity"])
def test_planted_mistakes_are_caught(mistake):
    def attn(q, k, v, scale, causal=False, key_len=None, rows=None, end_aligned=False):
        ea = end_aligned
        if mistake == "dropped_scale":
            return oracle.attention(q, k, v, 1.0, causal, key_len, rows, end_aligned=ea)
        if mistake == "transposed_qk":
            return oracle.attention(k, q, v, scale, causal, key_len, rows, end_aligned=ea)
        if mistake == "flipped_causal":
            # j >= i instead of j <= i: reverse the sequence on both sides
            o, l = oracle.attention(q[:, :, ::-1], k[:, :, ::-1], v[:, :, ::-1], scale, causal,
                                    None if key_len is None else key_len, rows, end_aligned=ea)
            return o[:, :, ::-1], l[:, :, ::-1]
        if mistake == "unmasked_padding_rows":
            o, l = oracle.attention(q, k, v, scale, causal, key_len, rows, end_aligned=ea)
            # padding rows computed as if they were ordinary rows
            N = q.shape[2]
            o2, l2 = oracle.attention(q, k, v, scale, causal,
                                      None if key_len is None else np.full_like(key_len, N), rows,
                                      end_aligned=ea)
            L = N if key_len is None else int(key_len[0])
            o[:, :, L:] = o2[:, :, L:]
            return o, l
        if mistake == "wrong_value_operand":
            return oracle.attention(q, k, k, scale, causal, key_len, rows, end_aligned=ea)
        if mistake == "start_aligned_cache_rows":
            # query row i at position i whatever the cache holds
            return oracle.attention(q, k, v, scale, causal, key_len, rows)
        if mistake == "rows_aligned_to_capacity":
            # row i at i + Nk - Nq, ignoring the sequence's own length
            if not ea:
                return oracle.attention(q, k, v, scale, causal, key_len, rows)
            Nq, Nk = q.shape[2], k.shape[2]
            qp = np.zeros(q.shape[:2] + (Nk, q.shape[3]))
            qp[:, :, Nk - Nq:] = q
            return oracle.attention(qp, k, v, scale, causal, key_len, rows=np.arange(Nk - Nq, Nk))
        raise AssertionError(mistake)

    assert _pin_suite(attn) != []


# ---------------------------------------------------------------------------
# Grouped key/value heads and packed variable-length batches
# ---------------------------------------------------------------------------

def test_grouped_heads_read_their_group():
    """Value rows of key/value head g all equal g: every output row of query
    head h is exactly h // (H / Hkv), and with equal K/V heads the result is
    independent of the grouping."""
    B, H, Hkv, N, d = 2, 8, 2, 11, 4
    q = rand((B, H, N, d), 900)
    k = rand((B, Hkv, N, d), 901)
    v = np.broadcast_to(np.arange(Hkv, dtype=np.float64)[None, :, None, None], (B, Hkv, N, d))
    o, _ = oracle.attention(q, oracle.expand_kv_heads(k, H), oracle.expand_kv_heads(v, H), 0.5)
    for h in range(H):
        assert np.allclose(o[:, h], h // (H // Hkv), atol=1e-14)
    k1 = np.broadcast_to(k[:, :1], (B, Hkv, N, d))
    v1 = rand((B, 1, N, d), 902)
    a, _ = oracle.attention(q, oracle.expand_kv_heads(k1, H),
                            oracle.expand_kv_heads(np.broadcast_to(v1, (B, Hkv, N, d)), H), 0.5)
    b, _ = oracle.attention(q, oracle.expand_kv_heads(k1[:, :1], H), oracle.expand_kv_heads(v1, H), 0.5)
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.expand_kv_heads(k, 7)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_padded_batch(causal):
    """A packed batch with equal query and key lengths per sequence equals the
    padded [B, H, N, d] problem with per-sequence lengths."""
    H, Hkv, d = 4, 2, 6
    lens = [5, 0, 1, 13, 7]
    N = max(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = rand((T, H, d), 910), rand((T, Hkv, d), 911), rand((T, Hkv, d), 912)
    o, lse = oracle.varlen_attention(q, k, v, cu, cu, 0.4, causal)
    B = len(lens)
    qp = np.zeros((B, H, N, d)); kp = np.zeros((B, Hkv, N, d)); vp = np.zeros((B, Hkv, N, d))
    for b, L in enumerate(lens):
        qp[b, :, :L] = q[cu[b]:cu[b + 1]].transpose(1, 0, 2)
        kp[b, :, :L] = k[cu[b]:cu[b + 1]].transpose(1, 0, 2)
        vp[b, :, :L] = v[cu[b]:cu[b + 1]].transpose(1, 0, 2)
    op, lp = oracle.attention(qp, oracle.expand_kv_heads(kp, H), oracle.expand_kv_heads(vp, H), 0.4,
                              causal=causal, key_len=np.array(lens))
    for b, L in enumerate(lens):
        assert np.allclose(o[cu[b]:cu[b + 1]], op[b, :, :L].transpose(1, 0, 2), atol=1e-14)
        assert np.allclose(lse[cu[b]:cu[b + 1]], lp[b, :, :L].T, atol=1e-14)


def test_varlen_brute_force_with_cache():
    """Query chunks shorter than their key sequences: brute force per
    (sequence, head) with the end-aligned positions."""
    H, Hkv, d = 2, 1, 3
    lq, lk = [2, 3, 1], [5, 3, 4]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    q, k, v = rand((cq[-1], H, d), 920), rand((ck[-1], Hkv, d), 921), rand((ck[-1], Hkv, d), 922)
    for causal in (False, True):
        o, lse = oracle.varlen_attention(q, k, v, cq, ck, 0.9, causal)
        for b in range(3):
            for h in range(H):
                O, LSE = brute(q[cq[b]:cq[b + 1], h].tolist(), k[ck[b]:ck[b + 1], 0].tolist(),
                               v[ck[b]:ck[b + 1], 0].tolist(), 0.9, causal, lk[b], end_aligned=True)
                assert np.allclose(o[cq[b]:cq[b + 1], h], np.array(O), atol=1e-13)
                assert np.allclose(lse[cq[b]:cq[b + 1], h], np.array(LSE), atol=1e-13)


# ---------------------------------------------------------------------------
# Additive mask (bias)
# ---------------------------------------------------------------------------

def test_bias_zero_and_row_constant():
    B, H, N, d = 2, 2, 19, 5
    q, k, v = rand((B, H, N, d), 950), rand((B, H, N, d), 951), rand((B, H, N, d), 952)
    o0, l0 = oracle.attention(q, k, v, 0.5, causal=True)
    o1, l1 = oracle.attention(q, k, v, 0.5, causal=True, bias=np.zeros((N, N)))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # a constant per row shifts the LSE and leaves O unchanged
    c = rand((B, H, N, 1), 953)
    o2, l2 = oracle.attention(q, k, v, 0.5, causal=True, bias=np.broadcast_to(c, (B, H, N, N)))
    assert np.allclose(o2, o0, atol=1e-13) and np.allclose(l2, l0 + c[..., 0], atol=1e-13)


def test_bias_minus_inf_is_a_mask():
    """-inf above the diagonal reproduces the causal mask; a row of -inf gets 0 / -inf."""
    B, H, N, d = 1, 2, 13, 3
    q, k, v = rand((B, H, N, d), 960), rand((B, H, N, d), 961), rand((B, H, N, d), 962)
    tri = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], 0.0, -np.inf)
    oc, lc = oracle.attention(q, k, v, 0.7, causal=True)
    ob, lb = oracle.attention(q, k, v, 0.7, bias=tri)
    assert np.allclose(oc, ob, atol=1e-14) and np.allclose(lc, lb, atol=1e-14)
    m = np.zeros((N, N))
    m[4] = -np.inf
    o, l = oracle.attention(q, k, v, 0.7, bias=m)
    assert np.all(o[:, :, 4] == 0) and np.all(l[:, :, 4] == -np.inf)


def test_bias_log_weights_closed_form():
    """q = 0 and bias log w_j: O_i = sum_j w_j v_j / sum_j w_j, LSE = log sum w."""
    B, H, N, d = 1, 1, 9, 4
    q = np.zeros((B, H, N, d))
    k, v = rand((B, H, N, d), 970), rand((B, H, N, d), 971)
    w = np.random.default_rng(972).uniform(0.1, 3.0, size=(N, N))
    o, l = oracle.attention(q, k, v, 1.0, bias=np.log(w))
    assert np.allclose(o[0, 0], (w @ v[0, 0]) / w.sum(axis=1)[:, None], atol=1e-14)
    assert np.allclose(l[0, 0], np.log(w.sum(axis=1)), atol=1e-14)


def test_bias_brute_force():
    N, d = 6, 3
    q, k, v = rand((1, 1, N, d), 980), rand((1, 1, N, d), 981), rand((1, 1, N, d), 982)
    m = rand((N, N), 983)
    m[2, 3] = -np.inf
    for causal in (False, True):
        o, l = oracle.attention(q, k, v, 0.6, causal=causal, bias=m)
        for i in range(N):
            keys = [j for j in range(N) if (not causal or j <= i) and m[i, j] > -np.inf]
            e = {j: math.exp(0.6 * math.fsum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d)) + m[i, j])
                 for j in keys}
            den = math.fsum(e.values())
            ref = [math.fsum(e[j] * v[0, 0, j, c] for j in keys) / den for c in range(d)]
            assert np.allclose(o[0, 0, i], ref, atol=1e-13)
            assert abs(l[0, 0, i] - math.log(den)) < 1e-13
