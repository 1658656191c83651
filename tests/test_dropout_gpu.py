"""GPU parity of the forward with dropout (fa_forward_dropout) against
oracle.dropout_attention, every element.

Both sides draw the keep mask from Philox4x32-10 with the same key and
counters; the mask decisions are integer comparisons, so they agree exactly,
and the outputs are compared with the bf16 forward tolerances.  Also: the LSE
is the undropped one, rate 0 gives the plain forward's result, and different
offsets and seeds give different outputs.

Tolerance: the forward's bf16 bounds (O max 2e-2, mean 2e-3, LSE 1e-3)
scaled by 1 / (1 - p) for O: the kept weights are amplified by that factor
(a row with few kept keys has |O| up to max|v| / (1 - p)), and the
roundings (bf16 weights, bf16 output) are relative, so absolute errors grow
by the same factor.  The LSE does not depend on the mask.
"""
import numpy as np
import pytest

import oracle
from io_aware_exact_forward_amd import workloads as W
from parity_util import TOL, run_hip, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_drop(inp, causal, scale, p, seed, offset):
    import torch
    import io_aware_exact_forward_amd as fa
    q, k, v, kl = to_device(inp)
    o, lse = fa.forward_dropout(q, k, v, p_drop=p, seed=seed, offset=offset, scale=scale,
                                causal=causal, key_len=kl)
    torch.cuda.synchronize()
    o = W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)
    return o, lse.cpu().numpy().astype(np.float64)


def check(inp, causal, scale, p, seed, offset, o, lse, label):
    tol = TOL["bf16"]
    o_ref, l_ref = oracle.dropout_attention(inp.exact("q"), inp.exact("k"), inp.exact("v"), scale,
                                            p, seed, offset, causal=causal, key_len=inp.key_len)
    live = np.isfinite(l_ref)
    err = np.abs(o - o_ref)[live]
    stats = dict(label=label, o_max=float(err.max()), o_mean=float(err.mean()),
                 lse_max=float(np.abs(lse[live] - l_ref[live]).max()))
    say(stats)
    amp = 1.0 / (1.0 - p)
    assert stats["o_max"] <= tol["o_max"] * amp and stats["o_mean"] <= tol["o_mean"] * amp, stats
    assert stats["lse_max"] <= tol["lse"], stats
    assert np.all(o[~live] == 0) and np.all(lse[~live] == -np.inf)


CASES = [
    # (B, H, N, d, key_len, p, seed, offset)
    (1, 2, 300, 64, None, 0.1, 1234, 0),
    (1, 2, 300, 128, None, 0.5, 99, 7),
    (2, 2, 513, 128, [513, 200], 0.2, 2 ** 63 + 5, 3),
    (1, 3, 129, 64, None, 0.9, 42, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"n{c[2]}d{c[3]}p{c[5]}")
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_against_oracle(case, causal):
    B, H, N, d, key_len, p, seed, offset = case
    inp = W.random_inputs(B, H, N, d, "bf16", 9950 + N, key_len=key_len)
    o, lse = run_drop(inp, causal, 1 / np.sqrt(d), p, seed, offset)
    check(inp, causal, 1 / np.sqrt(d), p, seed, offset, o, lse, f"{case} causal={causal}")


def test_dropout_rate_zero_and_lse():
    inp = W.random_inputs(1, 4, 700, 128, "bf16", 9960)
    for causal in (False, True):
        o0, l0 = run_drop(inp, causal, 1 / np.sqrt(128), 0.0, 5, 0)
        o1, l1 = run_hip(inp, causal, 1 / np.sqrt(128))
        assert np.abs(o0 - o1).max() <= TOL["bf16"]["o_max"]
        od, ld = run_drop(inp, causal, 1 / np.sqrt(128), 0.3, 5, 0)
        assert np.abs(ld - l1).max() <= TOL["bf16"]["lse"]   # the undropped normaliser


def test_dropout_offsets_and_seeds_differ():
    inp = W.random_inputs(1, 2, 256, 64, "bf16", 9961)
    a, _ = run_drop(inp, True, 0.125, 0.5, 11, 0)
    b, _ = run_drop(inp, True, 0.125, 0.5, 11, 1)
    c, _ = run_drop(inp, True, 0.125, 0.5, 12, 0)
    a2, _ = run_drop(inp, True, 0.125, 0.5, 11, 0)
    assert np.array_equal(a, a2)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_dropout_mid_size():
    """32 heads at N = 2048, causal, d = 128: every element of two heads."""
    inp = W.random_inputs(1, 32, 2048, 128, "bf16", 9962)
    o, lse = run_drop(inp, True, 1 / np.sqrt(128), 0.1, 777, 3)
    for h in (0, 31):
        o_ref, _ = oracle.dropout_attention(
            inp.exact("q")[:, h:h + 1], inp.exact("k")[:, h:h + 1], inp.exact("v")[:, h:h + 1],
            1 / np.sqrt(128), 0.1, 777, 3, causal=True, head_ids=[h], H_all=32)
        err = np.abs(o[:, h] - o_ref[:, 0])
        say("head", h, float(err.max()), float(err.mean()))
        amp = 1.0 / (1.0 - 0.1)
        assert err.max() <= TOL["bf16"]["o_max"] * amp and err.mean() <= TOL["bf16"]["o_mean"] * amp


GAP = __import__("json").load(open(__import__("os").path.join(
    __import__("os").path.dirname(__file__), "golden", "dropout_gap_draws.json")))


def gap_problem(case, d=64):
    """One head, n queries and keys, q = 0 (every weight 1/n), V rows one-hot
    (V[j] = e_j): O[i, j] = Z_ij / (n (1 - p)), so the stored draw's pair
    decides one output element by at least 0.15."""
    n = case["n"]
    q = np.zeros((1, 1, n, d), np.float32)
    k = np.random.default_rng(7).standard_normal((1, 1, n, d), dtype=np.float32)
    v = np.zeros((1, 1, n, d), np.float32)
    v[0, 0, np.arange(n), np.arange(n)] = 1.0
    return W.bf16_encode(q), W.bf16_encode(k), W.bf16_encode(v)


@pytest.mark.parametrize("case", GAP["cases"], ids=lambda c: f"p{c['p']}")
def test_dropout_rate_is_the_binary64_value(case):
    """The stored draw lies between floor(p * 2^32) and floor(f32(p) * 2^32)
    (tests/golden/make_dropout_gap_draws.py): the library must keep or drop
    that pair as the binary64 rate says.  Every element against the oracle;
    the values are multiples of 1 / (n (1 - p)) up to the bf16 rounding of O
    (relative 2^-9 of at most 0.18), so the tolerance is 1e-3."""
    import torch
    import io_aware_exact_forward_amd as fa
    p, n, seed, off = case["p"], case["n"], case["seed"], case["offset"]
    qb, kb, vb = gap_problem(case)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    say(f"gap draw p={p} n={n} offset={off} row={case['row']} key={case['key']}")
    o, lse = fa.forward_dropout(dev(qb), dev(kb), dev(vb), p_drop=p, seed=seed, offset=off,
                                scale=0.125)
    torch.cuda.synchronize()
    o = W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)
    ex = lambda b: W.bf16_decode(b, np.float64)
    o_ref, l_ref = oracle.dropout_attention(ex(qb), ex(kb), ex(vb), 0.125, p, seed, off)
    assert np.abs(o - o_ref).max() <= 1e-3
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= 1e-3
    want = 1.0 / (n * (1.0 - p)) if case["kept"] else 0.0
    assert abs(o[0, 0, case["row"], case["key"]] - want) <= 1e-3
