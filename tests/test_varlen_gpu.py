"""GPU parity of the packed variable-length forward (fa_forward_varlen) with
grouped key/value heads against oracle.varlen_attention, every element.

Cases: lengths that include empty and one-token sequences and ragged tails at
d = 64 and 128; query chunks shorter than their keys (positions at the end of
each sequence); more queries than keys; a batch large enough that the 256-row
ping-pong configuration runs with short sequences in it; and the full-size
workload on sampled sequences.
"""
import numpy as np
import pytest

import oracle
from io_aware_exact_forward_amd import workloads as W
from parity_util import TOL

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def run(inp, causal, scale, max_q, max_k):
    import torch
    import io_aware_exact_forward_amd as fa
    cq = torch.from_numpy(inp.cu_q).to("cuda:0")
    ck = torch.from_numpy(inp.cu_k).to("cuda:0")
    o, lse = fa.forward_varlen(dev(inp.q), dev(inp.k), dev(inp.v), cq, ck, max_q, max_k,
                               scale=scale, causal=causal)
    torch.cuda.synchronize()
    o = W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)
    return o, lse.cpu().numpy().astype(np.float64)


def check(inp, causal, scale, o, lse, label, seqs=None):
    tol = TOL["bf16"]
    cq, ck = inp.cu_q, inp.cu_k
    if seqs is None:
        o_ref, l_ref = oracle.varlen_attention(inp.exact("q"), inp.exact("k"), inp.exact("v"),
                                               cq, ck, scale, causal)
        sel = np.ones(len(o), dtype=bool)
    else:
        o_ref = np.zeros_like(o)
        l_ref = np.full(lse.shape, -np.inf)
        sel = np.zeros(len(o), dtype=bool)
        qx, kx, vx = inp.exact("q"), inp.exact("k"), inp.exact("v")
        for b in seqs:
            a, z = oracle.varlen_attention(qx[cq[b]:cq[b + 1]], kx[ck[b]:ck[b + 1]],
                                           vx[ck[b]:ck[b + 1]],
                                           np.array([0, cq[b + 1] - cq[b]]),
                                           np.array([0, ck[b + 1] - ck[b]]), scale, causal)
            o_ref[cq[b]:cq[b + 1]] = a
            l_ref[cq[b]:cq[b + 1]] = z
            sel[cq[b]:cq[b + 1]] = True
    o, lse, o_ref, l_ref = o[sel], lse[sel], o_ref[sel], l_ref[sel]
    live = np.isfinite(l_ref)
    stats = {"label": label, "rows": int(live.sum()), "empty": int((~live).sum())}
    if live.any():
        err = np.abs(o - o_ref)[live]
        stats.update(o_max=float(err.max()), o_mean=float(err.mean()),
                     lse_max=float(np.abs(lse - l_ref)[live].max()))
        assert stats["o_max"] <= tol["o_max"], stats
        assert stats["o_mean"] <= tol["o_mean"], stats
        assert stats["lse_max"] <= tol["lse"], stats
    if (~live).any():
        assert np.all(o[~live] == 0) and np.all(lse[~live] == -np.inf), label
    say(stats)


CASES = [
    # (lens_q, lens_k, H, Hkv, d, seed)
    ([5, 0, 1, 300, 129, 64], None, 4, 2, 64, 9901),
    ([5, 0, 1, 300, 129, 64], None, 4, 4, 128, 9902),
    ([3, 100, 1, 0], [500, 100, 77, 9], 6, 2, 128, 9903),   # query chunks at the end of keys
    ([40, 7], [12, 0], 2, 1, 64, 9904),                      # more queries than keys; no keys
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"h{c[2]}kv{c[3]}d{c[4]}s{c[5]}")
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_against_oracle(case, causal):
    lens_q, lens_k, H, Hkv, d, seed = case
    lens_k = lens_q if lens_k is None else lens_k
    say("case", case, causal)
    inp = W.packed_inputs(lens_q, lens_k, H, Hkv, d, seed)
    o, lse = run(inp, causal, 1 / np.sqrt(d), max(lens_q), max(lens_k))
    check(inp, causal, 1 / np.sqrt(d), o, lse, f"{case} causal={causal}")


def test_varlen_ping_pong_configuration_with_short_sequences():
    """16 sequences x 16 heads with the longest at 300 rows: 512 tiles of 256
    rows, so the 8-wave configuration runs, with 1- and 17-token sequences in
    the batch."""
    rng = np.random.default_rng(9905)
    lens = [300, 1, 17] + rng.integers(1, 300, size=13).tolist()
    inp = W.packed_inputs(lens, lens, 16, 4, 128, 9906)
    for causal in (False, True):
        o, lse = run(inp, causal, 1 / np.sqrt(128), 300, 300)
        check(inp, causal, 1 / np.sqrt(128), o, lse, f"pp causal={causal}")


def test_varlen_full_size_sampled_sequences():
    """The packed workload at full size (16 causal sequences up to 8192 tokens,
    32 heads on 8 key/value heads, d = 128): every row of the shortest, the
    longest and two other sequences."""
    wl = W.VARLEN_WORKLOADS["varlen_b16_h32_hkv8_n8192_d128_bf16"]
    inp = W.varlen_inputs(wl)
    lens = np.diff(inp.cu_q)
    say("lengths", lens.tolist())
    o, lse = run(inp, True, wl.scale, int(lens.max()), int(lens.max()))
    assert np.all(np.isfinite(lse))
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 3, 11})
    check(inp, True, wl.scale, o, lse, "full size", seqs=seqs)
