"""GPU parity of the backward with an additive mask (fa_backward_bias)
against oracle.attention_backward(..., bias=M), every element of dQ, dK, dV.

Each case runs the HIP forward with the mask (fa_forward_bias) for O and LSE,
then the HIP backward with the same mask.  The tolerance is the backward's
(tests/test_backward_gpu.py: per gradient tensor, max error <= 1.2e-2 *
max |ref|, mean error <= 1.2e-2 * mean |ref|).  Cases: a full [B, H, N, ld]
mask with padded rows (N not a multiple of 4) and -inf entries, masks
broadcast over batch and over heads, d = 64 and 128, causal and not, with
per-sequence lengths, and rows hidden entirely by the mask (their gradients
are exactly zero); a zero mask reproduces fa_backward.
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


def make_bias(shape_bh, N, ld, seed, neg_inf_frac=0.05, hidden_rows=()):
    rng = np.random.default_rng(seed)
    m = np.zeros(shape_bh + (N, ld), dtype=np.float32)
    m[..., :N] = rng.standard_normal(shape_bh + (N, N)).astype(np.float32) * 2.0
    hide = rng.random(shape_bh + (N, N)) < neg_inf_frac
    m[..., :N][hide] = -np.inf
    for r in hidden_rows:
        m[..., r, :N] = -np.inf
    return m


def run(inp, do_bits, bias, causal, scale):
    import torch
    import io_aware_exact_forward_amd as fa
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(do_bits)
    kl = None if inp.key_len is None else torch.from_numpy(inp.key_len).to("cuda:0")
    bt = torch.from_numpy(bias).to("cuda:0")
    o, lse = fa.forward_bias(q, k, v, bt, scale=scale, causal=causal, key_len=kl)
    dq, dk, dv = fa.backward_bias(q, k, v, o, lse, do, bt, scale=scale, causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def check(inp, do_bits, bias, causal, scale, got, label, hidden_rows=()):
    N = inp.q.shape[2]
    ref = oracle.attention_backward(inp.exact("q"), inp.exact("k"), inp.exact("v"),
                                    W.bf16_decode(do_bits, np.float64), scale, causal=causal,
                                    key_len=inp.key_len, bias=bias[..., :N].astype(np.float64))[:3]
    stats = {"label": label}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite"
        err = np.abs(g - r)
        smax, smean = float(np.abs(r).max()), float(np.abs(r).mean())
        stats[name] = (float(err.max()) / smax, float(err.mean()) / smean)
        assert err.max() <= TOL_MAX * smax, f"{label} {name}: max err {err.max():.3g} vs {smax:.3g}"
        assert err.mean() <= TOL_MEAN * smean, f"{label} {name}: mean {err.mean():.3g} vs {smean:.3g}"
    for r in hidden_rows:
        assert np.all(got[0][:, :, r] == 0), f"{label}: gradient of a hidden row"
    if inp.key_len is not None:
        for b, L in enumerate(np.clip(inp.key_len, 0, N)):
            for g in got:
                assert np.all(g[b, :, L:] == 0.0), f"{label}: nonzero gradient past the length"
    say(stats)


CASES = [
    # (B, H, N, d, key_len, mask batch/head shape, ld, hidden rows, seed)
    (2, 2, 300, 64, None, (2, 2), 300, (), 9981),
    (2, 2, 301, 128, [301, 150], (2, 2), 304, (5, 140), 9982),
    (2, 3, 257, 128, None, (1, 3), 260, (), 9983),      # broadcast over batch
    (2, 3, 200, 64, [200, 77], (2, 1), 200, (3,), 9984),  # broadcast over heads
    (1, 2, 130, 128, None, (1, 1), 132, (), 9985),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"n{c[2]}d{c[3]}m{c[5][0]}{c[5][1]}")
@pytest.mark.parametrize("causal", [False, True])
def test_bias_backward_against_oracle(case, causal):
    B, H, N, d, key_len, mbh, ld, hidden, seed = case
    say("case", case, "causal", causal)
    inp, do = W.grad_inputs(B, H, N, d, seed, key_len=key_len)
    bias = make_bias(mbh, N, ld, seed + 1, hidden_rows=hidden)
    got = run(inp, do, bias, causal, 1 / np.sqrt(d))
    check(inp, do, bias, causal, 1 / np.sqrt(d), got, f"{case} causal={causal}", hidden)


def test_bias_backward_zero_mask_is_plain_backward():
    import torch
    import io_aware_exact_forward_amd as fa
    inp, do_bits = W.grad_inputs(1, 2, 333, 64, 9990)
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(do_bits)
    zero = torch.zeros((1, 1, 333, 336), dtype=torch.float32, device="cuda:0")
    for causal in (False, True):
        o, lse = fa.forward(q, k, v, causal=causal)
        a = fa.backward(q, k, v, o, lse, do, causal=causal)
        b = fa.backward_bias(q, k, v, o, lse, do, zero, causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            err = (x.float() - y.float()).abs().max().item()
            assert err <= TOL_MAX * x.float().abs().max().item(), err
