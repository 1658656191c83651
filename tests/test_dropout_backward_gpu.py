"""GPU parity of the backward with dropout (fa_backward_dropout) against
oracle.dropout_attention_backward, every element of dQ, dK and dV.

Each case runs the HIP forward with dropout (fa_forward_dropout) for O and
LSE, then the HIP backward with the same rate, seed and offset.  Both sides
draw the keep mask from Philox4x32-10 with the same key and counters and
decide it by integer comparison, so the masks agree exactly; the dK/dV
kernel, whose lanes hold keys rather than rows, exchanges the draws inside
groups of four lanes, which the cases with several key tiles and ragged
lengths exercise.

Tolerance: the backward's (tests/test_backward_gpu.py: per gradient tensor,
max error <= 1.2e-2 * max |ref|, mean error <= 1.2e-2 * mean |ref|).  Kept
terms are amplified by 1 / (1 - p), and so are their rounding errors, so the
errors stay in proportion to the gradients' own scale.  Keys past a length
and padding rows get exactly zero gradients.  Rate 0 reproduces
fa_backward.
"""
import numpy as np
import pytest

import oracle
from io_aware_exact_forward_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 1.2e-2, 1.2e-2


def say(*a):
    print(*a, flush=True)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def host(t):
    import torch
    return W.bf16_decode(t.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)


def run(inp, do_bits, causal, scale, p, seed, offset):
    import torch
    import io_aware_exact_forward_amd as fa
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(do_bits)
    kl = None if inp.key_len is None else torch.from_numpy(inp.key_len).to("cuda:0")
    o, lse = fa.forward_dropout(q, k, v, p_drop=p, seed=seed, offset=offset, scale=scale,
                                causal=causal, key_len=kl)
    dq, dk, dv = fa.backward_dropout(q, k, v, o, lse, do, p_drop=p, seed=seed, offset=offset,
                                     scale=scale, causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def check(inp, do_bits, causal, scale, p, seed, offset, got, label):
    ref = oracle.dropout_attention_backward(inp.exact("q"), inp.exact("k"), inp.exact("v"),
                                            W.bf16_decode(do_bits, np.float64), scale, p, seed,
                                            offset, causal=causal, key_len=inp.key_len)[:3]
    stats = {"label": label}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite"
        err = np.abs(g - r)
        smax, smean = float(np.abs(r).max()), float(np.abs(r).mean())
        stats[name] = (float(err.max()) / max(smax, 1e-30), float(err.mean()) / max(smean, 1e-30))
        if smax > 0:
            assert err.max() <= TOL_MAX * smax, f"{label} {name}: max err {err.max():.3g} vs {smax:.3g}"
            assert err.mean() <= TOL_MEAN * smean, f"{label} {name}: mean {err.mean():.3g} vs {smean:.3g}"
        else:
            assert np.all(g == 0), f"{label} {name}: expected zeros"
    if inp.key_len is not None:
        N = inp.exact("q").shape[2]
        for b, L in enumerate(np.clip(inp.key_len, 0, N)):
            for g in got:
                assert np.all(g[b, :, L:] == 0.0), f"{label}: nonzero gradient past the length"
    say(stats)


CASES = [
    # (B, H, N, d, key_len, p, seed, offset, data seed)
    (1, 2, 300, 64, None, 0.1, 1234, 0, 9801),
    (1, 2, 300, 128, None, 0.5, 99, 7, 9802),
    (2, 2, 513, 128, [513, 200], 0.2, 2 ** 63 + 5, 3, 9803),
    (2, 1, 129, 64, [129, 63], 0.9, 42, 1, 9804),
    (1, 2, 64, 128, None, 0.3, 7, 2, 9805),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"n{c[2]}d{c[3]}p{c[5]}")
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_against_oracle(case, causal):
    B, H, N, d, key_len, p, seed, offset, ds = case
    say("case", case, "causal", causal)
    inp, do = W.grad_inputs(B, H, N, d, ds, key_len=key_len)
    got = run(inp, do, causal, 1 / np.sqrt(d), p, seed, offset)
    check(inp, do, causal, 1 / np.sqrt(d), p, seed, offset, got, f"{case} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_dropout_backward_rate_zero_is_plain_backward(d):
    """At rate 0 every weight is kept and scaled by 1: at d = 128 the dropout
    kernels are the plain kernels' arithmetic, bit for bit; at d = 64 the
    plain dK/dV kernel runs four waves per workgroup and the dropout one
    eight (a wave pair splitting the rows, their sums added at the end), so
    dK and dV agree to rounding and dQ bit for bit."""
    import torch
    import io_aware_exact_forward_amd as fa
    inp, do_bits = W.grad_inputs(1, 2, 333, d, 9810)
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(do_bits)
    for causal in (False, True):
        o, lse = fa.forward(q, k, v, causal=causal)
        a = fa.backward(q, k, v, o, lse, do, causal=causal)
        b = fa.backward_dropout(q, k, v, o, lse, do, p_drop=0.0, seed=3, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0])
        for x, y in zip(a[1:], b[1:]):
            if d == 128:
                assert torch.equal(x, y)
            else:
                xf, yf = x.float(), y.float()
                assert (xf - yf).abs().max() <= 1e-2 * xf.abs().max()


def test_dropout_backward_full_size_heads():
    """The pages' backward workload (batch 2, 16 heads, N 4096, d 64) at rate
    0.1, causal: every element of two heads (each with its own mask stream)."""
    wl = W.BWD_WORKLOADS["bwd_b2_h16_n4096_d64_bf16"]
    inp, do = W.grad_inputs(wl.B, wl.H, wl.N, wl.d, wl.seed)
    say("full size", wl.name)
    got = run(inp, do, True, wl.scale, 0.1, 2024, 1)
    dox = W.bf16_decode(do, np.float64)
    for b, h in ((0, 0), (1, 15)):
        sl = lambda x: x[b:b + 1, h:h + 1]
        ref = oracle.dropout_attention_backward(
            sl(inp.exact("q")), sl(inp.exact("k")), sl(inp.exact("v")), sl(dox), wl.scale, 0.1,
            2024, 1, causal=True, head_ids=[h], H_all=wl.H, batch_ids=[b])[:3]
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            g, r = g[b, h], r[0, 0]
            err = np.abs(g - r)
            assert err.max() <= TOL_MAX * np.abs(r).max(), (b, h, name, err.max())
            assert err.mean() <= TOL_MEAN * np.abs(r).mean(), (b, h, name, err.mean())
        say({"head": (b, h), "ok": True})


GAP = __import__("json").load(open(__import__("os").path.join(
    __import__("os").path.dirname(__file__), "golden", "dropout_gap_draws.json")))


@pytest.mark.parametrize("case", GAP["cases"], ids=lambda c: f"p{c['p']}")
def test_dropout_backward_rate_is_the_binary64_value(case):
    """The backward regenerates the forward's mask from the binary64 rate:
    with q = 0 (weights 1/n), V and dO rows one-hot (dO_i = e_i),
    dV[j, i] = Z_ij / (n (1 - p)), so the stored gap draw
    (tests/golden/make_dropout_gap_draws.py) decides one element of dV by at
    least 0.15.  Every element of dQ, dK, dV against the oracle at this
    file's tolerance, and that element to 1e-3."""
    import torch
    import io_aware_exact_forward_amd as fa
    p, n, seed, off = case["p"], case["n"], case["seed"], case["offset"]
    d = 64
    q = np.zeros((1, 1, n, d), np.float32)
    k = np.random.default_rng(7).standard_normal((1, 1, n, d), dtype=np.float32)
    v = np.zeros((1, 1, n, d), np.float32)
    v[0, 0, np.arange(n), np.arange(n)] = 1.0
    qb, kb, vb, dob = (W.bf16_encode(x) for x in (q, k, v, v))
    say(f"gap draw backward p={p} n={n} offset={off} row={case['row']} key={case['key']}")
    tq, tk, tv, tdo = dev(qb), dev(kb), dev(vb), dev(dob)
    o, lse = fa.forward_dropout(tq, tk, tv, p_drop=p, seed=seed, offset=off, scale=0.125)
    dq, dk, dv = fa.backward_dropout(tq, tk, tv, o, lse, tdo, p_drop=p, seed=seed, offset=off,
                                     scale=0.125)
    torch.cuda.synchronize()
    got = host(dq), host(dk), host(dv)
    ex = lambda b: W.bf16_decode(b, np.float64)
    ref = oracle.dropout_attention_backward(ex(qb), ex(kb), ex(vb), ex(dob), 0.125, p, seed,
                                            off)[:3]
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        err = np.abs(g - r)
        scale_max = max(np.abs(r).max(), 1e-30)
        assert err.max() <= TOL_MAX * scale_max + 1e-6, (name, err.max())
    want = 1.0 / (n * (1.0 - p)) if case["kept"] else 0.0
    assert abs(got[2][0, 0, case["key"], case["row"]] - want) <= 1e-3
