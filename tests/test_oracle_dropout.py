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
