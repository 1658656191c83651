"""GPU parity of the forward with an additive mask (fa_forward_bias) against
oracle.attention(..., bias=M), every element, bf16 tolerances.

Cases: a full [B, H, N, ld] bias with padded rows and -inf entries, bias
broadcast over batch and over heads, d = 64 and 128, causal and not, with
per-sequence lengths, a -inf pattern that reproduces the causal mask, and
rows hidden entirely by the bias (O = 0, LSE = -inf).
"""
import numpy as np
import pytest

import oracle
from io_aware_exact_forward_amd import workloads as W
from parity_util import TOL, run_hip, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def make_bias(shape_bh, N, ld, seed, neg_inf_frac=0.05):
    rng = np.random.default_rng(seed)
    m = np.zeros(shape_bh + (N, ld), dtype=np.float32)
    m[..., :N] = rng.standard_normal(shape_bh + (N, N)).astype(np.float32) * 2.0
    hide = rng.random(shape_bh + (N, N)) < neg_inf_frac
    m[..., :N][hide] = -np.inf
    return m


def run_bias(inp, bias, causal, scale):
    import torch
    import io_aware_exact_forward_amd as fa
    q, k, v, kl = to_device(inp)
    bt = torch.from_numpy(bias).to("cuda:0")
    o, lse = fa.forward_bias(q, k, v, bt, scale=scale, causal=causal, key_len=kl)
    torch.cuda.synchronize()
    o = W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)
    return o, lse.cpu().numpy().astype(np.float64)


def check(inp, bias, causal, scale, o, lse, label):
    tol = TOL["bf16"]
    N = inp.q.shape[2]
    o_ref, l_ref = oracle.attention(inp.exact("q"), inp.exact("k"), inp.exact("v"), scale,
                                    causal=causal, key_len=inp.key_len,
                                    bias=bias[..., :N].astype(np.float64))
    live = np.isfinite(l_ref)
    stats = {"label": label, "rows": int(live.sum()), "empty": int((~live).sum())}
    if live.any():
        err = np.abs(o - o_ref)[live]
        stats.update(o_max=float(err.max()), o_mean=float(err.mean()),
                     lse_max=float(np.abs(lse[live] - l_ref[live]).max()))
        assert stats["o_max"] <= tol["o_max"] and stats["o_mean"] <= tol["o_mean"], stats
        assert stats["lse_max"] <= tol["lse"], stats
    assert np.all(o[~live] == 0) and np.all(lse[~live] == -np.inf), label
    say(stats)


CASES = [
    # (B, H, N, d, key_len, bias batch/head shape, ld, seed)
    (2, 2, 300, 64, None, (2, 2), 300, 9971),
    (2, 2, 301, 128, [301, 150], (2, 2), 304, 9972),
    (2, 3, 257, 128, None, (1, 3), 260, 9973),     # broadcast over batch
    (2, 3, 200, 64, [200, 77], (2, 1), 200, 9974),  # broadcast over heads
    (1, 2, 640, 128, None, (1, 1), 640, 9975),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"n{c[2]}d{c[3]}s{c[7]}")
@pytest.mark.parametrize("causal", [False, True])
def test_bias_against_oracle(case, causal):
    B, H, N, d, key_len, bshape, ld, seed = case
    inp = W.random_inputs(B, H, N, d, "bf16", seed, key_len=key_len)
    bias = make_bias(bshape, N, ld, seed + 1)
    o, lse = run_bias(inp, bias, causal, 1 / np.sqrt(d))
    check(inp, bias, causal, 1 / np.sqrt(d), o, lse, f"{case} causal={causal}")


def test_bias_causal_pattern_and_hidden_rows():
    N = 333
    inp = W.random_inputs(1, 2, N, 128, "bf16", 9976)
    tri = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], 0.0, -np.inf).astype(np.float32)
    bias = np.zeros((1, 1, N, 336), dtype=np.float32)
    bias[0, 0, :, :N] = tri
    o_b, l_b = run_bias(inp, bias, False, 1 / np.sqrt(128))
    o_c, l_c = run_hip(inp, True, 1 / np.sqrt(128))
    assert np.abs(o_b - o_c).max() <= TOL["bf16"]["o_max"]
    assert np.abs(l_b - l_c).max() <= TOL["bf16"]["lse"]
    bias[0, 0, 10, :] = -np.inf
    bias[0, 0, 200, :] = -np.inf
    o, lse = run_bias(inp, bias, False, 1 / np.sqrt(128))
    assert np.all(o[:, :, [10, 200]] == 0) and np.all(lse[:, :, [10, 200]] == -np.inf)
    check(inp, bias, False, 1 / np.sqrt(128), o, lse, "hidden rows")
