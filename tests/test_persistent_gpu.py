"""GPU parity of the persistent form of the 256-row forward kernel.

The library runs one workgroup per compute unit over a balanced list of
query tiles when the problem allows it (dense layout, Nk == N, no
per-sequence lengths, one key range, and B*H*ceil(N/256)/2 a multiple of the
compute-unit count, non-negative scale).  A negative scale is applied by
flipping the sign bits of Q, which is exact, and takes the one-tile-per-
workgroup launch of the same kernel: forward(q, scale=-s) and forward(-q,
scale=s) compute the same values, so the two launches must agree bit for bit
on every element.  Sampled rows are also compared with the fp64 oracle.
"""
import math

import numpy as np
import pytest

import oracle
from io_aware_exact_forward_amd import workloads as W
from parity_util import TOL, compare, from_device, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def heads_for_persistence(B, N):
    """Heads that make B*H*ceil(N/256)/2 a multiple of the compute units."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units_per_head = B * ((N + 255) // 256) // 2
    if cus % 8 or units_per_head == 0:
        pytest.skip(f"{cus} compute units: no persistent launch")
    h = cus // math.gcd(cus, units_per_head)
    while h < 16:
        h *= 2
    return h


def sampled_rows(N, H, seed):
    rng = np.random.default_rng(seed)
    extra = [0, 1, 255, 256, N - 1]
    out = []
    for _ in range(H):
        r = sorted(set(extra) | set(rng.choice(N, 12, replace=False).tolist()))
        out.append(r)
    R = min(len(x) for x in out)
    return np.array([x[:R] for x in out], dtype=np.int64)


@pytest.mark.parametrize("B,d,causal,N", [(1, 128, True, 4096), (1, 128, False, 4096),
                                          (1, 64, True, 4096), (1, 64, False, 2048),
                                          (1, 128, True, 4000), (1, 64, True, 4000),
                                          (1, 128, True, 8192), (1, 128, False, 8192),
                                          (1, 64, True, 8192),
                                          (2, 128, True, 4096), (2, 64, False, 4096)])
def test_persistent_matches_per_tile_launch(B, d, causal, N):
    import torch
    import io_aware_exact_forward_amd as fa
    H = heads_for_persistence(B, N)
    inp = W.random_inputs(B, H, N, d, "bf16", seed=400 + d + N + causal, key_len=None)
    scale = 1.0 / math.sqrt(d)
    say("case", f"B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v, _ = to_device(inp)
    o1, l1 = fa.forward(q, k, v, scale=-scale, causal=causal)   # one tile per workgroup
    o2, l2 = fa.forward(-q, k, v, scale=scale, causal=causal)   # persistent
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "O differs between launches"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "LSE differs between launches"
    rows = sampled_rows(N, H, 5)
    st = compare(inp, from_device(o2), l2.cpu().numpy().astype(np.float64), causal, -scale,
                 rows=rows, label=f"persistent d={d} causal={causal} N={N}")
    say(st)


@pytest.mark.parametrize("B,causal", [(1, True), (2, False)])
def test_persistent_grouped_heads(B, causal):
    """Grouped K/V heads through the split entry point with one key range."""
    import torch
    import io_aware_exact_forward_amd as fa
    N, d, G = 4096, 128, 4
    H = heads_for_persistence(B, N)
    inp = W.random_inputs(B, H, N, d, "bf16", seed=431, key_len=None)
    say("case", f"grouped B={B} H={H} Hkv={H // G} N={N} d={d} causal={causal}")
    q, k, v, _ = to_device(inp)
    k, v = k[:, ::G].contiguous(), v[:, ::G].contiguous()
    scale = 1.0 / math.sqrt(d)
    o1, l1 = fa.forward_split(q, k, v, scale=scale, causal=causal, num_splits=1)
    kl = torch.full((B,), N, dtype=torch.int32, device=q.device)
    o2, l2 = fa.forward_split(q, k, v, scale=scale, causal=causal, num_splits=1, key_len=kl)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    # oracle: query head h reads key/value head h // G
    kx = np.repeat(inp.exact("k")[:, ::G], G, axis=1)
    vx = np.repeat(inp.exact("v")[:, ::G], G, axis=1)
    rows = sampled_rows(N, H, 6)
    o_ref, l_ref = oracle.attention(inp.exact("q"), kx, vx, scale, causal=causal, rows=rows)
    og = from_device(o1)
    lg = l1.cpu().numpy().astype(np.float64)
    og = np.stack([og[:, h, rows[h]] for h in range(H)], axis=1)
    lg = np.stack([lg[:, h, rows[h]] for h in range(H)], axis=1)
    err = np.abs(og - o_ref)
    tol = TOL["bf16"]
    assert err.max() <= tol["o_max"] and err.mean() <= tol["o_mean"], (err.max(), err.mean())
    assert np.abs(lg - l_ref).max() <= tol["lse"]
