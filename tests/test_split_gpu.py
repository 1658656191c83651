"""GPU parity of the split-KV forward (fa_forward_split) against the fp64 oracle.

Query rows sit at the end of each sequence's key cache (row i at key position
i + L_b - Nq); the oracle computes the same with ``end_aligned=True``.  Every
case compares all outputs element by element: rows that see at least one key
within the bf16 tolerances, rows that see none exactly 0 with LSE -inf.
Cases span several 128-key ranges with ragged tails, decode (one query row),
chunked prefill (Nq < Nk), more query rows than cached keys, empty caches,
the automatic and explicit range counts, and a peaky softmax whose ranges
have very different log-sum-exp values.
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


def run_split(inp, causal, scale, num_splits):
    import torch
    import io_aware_exact_forward_amd as fa
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    kl = None if inp.key_len is None else torch.from_numpy(inp.key_len).to("cuda:0")
    o, lse = fa.forward_split(q, k, v, scale=scale, causal=causal, key_len=kl,
                              num_splits=num_splits)
    torch.cuda.synchronize()
    o = W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)
    return o, lse.cpu().numpy().astype(np.float64)


def check(inp, causal, scale, o_gpu, lse_gpu, label, rows=None):
    """All rows (or rows [R] of every head) of the GPU result against the oracle."""
    tol = TOL["bf16"]
    H = inp.q.shape[1]
    kx = oracle.expand_kv_heads(inp.exact("k"), H)
    vx = oracle.expand_kv_heads(inp.exact("v"), H)
    o_ref, lse_ref = oracle.attention(inp.exact("q"), kx, vx, scale, causal=causal,
                                      key_len=inp.key_len, rows=rows, end_aligned=True)
    if rows is not None:
        o_gpu, lse_gpu = o_gpu[:, :, rows], lse_gpu[:, :, rows]
    live = np.isfinite(lse_ref)
    stats = {"label": label, "rows": int(live.sum()), "empty_rows": int((~live).sum())}
    if live.any():
        err = np.abs(o_gpu - o_ref)[live]
        lerr = np.abs(lse_gpu - lse_ref)[live]
        stats.update(o_max=float(err.max()), o_mean=float(err.mean()), lse_max=float(lerr.max()))
        assert np.all(np.isfinite(o_gpu[live])), f"{label}: non-finite output"
        assert stats["o_max"] <= tol["o_max"], f"{label}: O max {stats['o_max']:.3g}"
        assert stats["o_mean"] <= tol["o_mean"], f"{label}: O mean {stats['o_mean']:.3g}"
        assert stats["lse_max"] <= tol["lse"], f"{label}: LSE {stats['lse_max']:.3g}"
    if (~live).any():
        assert np.all(o_gpu[~live] == 0.0), f"{label}: rows with no key not exactly 0"
        assert np.all(lse_gpu[~live] == -np.inf), f"{label}: rows with no key: LSE not -inf"
    say(stats)
    return stats


CASES = [
    # (B, H, Nq, Nk, d, key_len, q_mult, seed)
    (1, 2, 1000, 1000, 64, None, 1.0, 9101),          # square, ragged tail
    (1, 2, 777, 777, 128, None, 1.0, 9102),
    (4, 3, 1, 3000, 128, [3000, 1, 0, 1777], 1.0, 9103),  # decode
    (4, 3, 1, 3000, 64, [3000, 129, 128, 2049], 1.0, 9104),
    (2, 2, 200, 1500, 128, [1500, 333], 1.0, 9105),   # chunked prefill
    (2, 2, 300, 256, 64, [100, 256], 1.0, 9106),      # more rows than cached keys
    (2, 2, 130, 2000, 128, None, 4.0, 9107),          # peaky rows
    (1, 2, 5, 9000, 64, None, 1.0, 9110),             # 64 asked: 36 ranges (more than 32 to merge)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}h{c[1]}q{c[2]}k{c[3]}d{c[4]}")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 64])
def test_split_against_oracle(case, causal, num_splits):
    B, H, Nq, Nk, d, key_len, q_mult, seed = case
    say("case", case, "causal", causal, "splits", num_splits)
    inp = W.cache_inputs(B, H, Nq, Nk, d, seed, q_mult=q_mult, key_len=key_len)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_split(inp, causal, scale, num_splits)
    check(inp, causal, scale, o, lse, f"{case} causal={causal} splits={num_splits}")


def test_split_no_keys():
    inp = W.cache_inputs(2, 2, 5, 0, 64, 9108)
    for causal in (False, True):
        o, lse = run_split(inp, causal, 0.125, 0)
        assert np.all(o == 0.0) and np.all(lse == -np.inf)


def test_split_matches_unsplit_forward_on_square_problem():
    """With Nq = Nk and no lengths the split call computes fa_forward's result:
    both within tolerance of the oracle, and within twice it of each other."""
    import torch
    import io_aware_exact_forward_amd as fa
    from parity_util import run_hip
    inp = W.random_inputs(1, 4, 2048, 128, "bf16", 9109)
    for causal in (False, True):
        say("square", causal)
        o1, l1 = run_hip(inp, causal, 1 / np.sqrt(128))
        o2, l2 = run_split(inp, causal, 1 / np.sqrt(128), 4)
        rows = np.array([0, 1, 127, 128, 1000, 2047])
        check(inp, causal, 1 / np.sqrt(128), o2, l2, "split", rows=rows)
        assert np.abs(o1 - o2).max() <= 2 * TOL["bf16"]["o_max"]
        assert np.abs(l1 - l2).max() <= 2 * TOL["bf16"]["lse"]
        torch.cuda.synchronize()


def test_split_reuses_a_caller_workspace():
    """A caller-owned workspace serves two calls of different shapes; the
    second, smaller call must not see the first call's partial results."""
    import torch
    import io_aware_exact_forward_amd as fa
    big = W.cache_inputs(2, 4, 3, 4096, 128, 9110, key_len=[4096, 2500])
    small = W.cache_inputs(1, 2, 1, 900, 128, 9111)
    need = max(fa.fa_split_workspace_bytes(2, 4, 3, 4096, 128, 16),
               fa.fa_split_workspace_bytes(1, 2, 1, 900, 128, 16))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    for inp in (big, small):
        B, H, Nq, _ = inp.q.shape
        q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
        kl = None if inp.key_len is None else torch.from_numpy(inp.key_len).to("cuda:0")
        o, lse = fa.forward_split(q, k, v, scale=1 / np.sqrt(128), causal=True, key_len=kl,
                                  num_splits=16, workspace=ws)
        torch.cuda.synchronize()
        og = W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)
        check(inp, True, 1 / np.sqrt(128), og, lse.cpu().numpy().astype(np.float64), "reuse")


def test_grouped_decode_full_size():
    """The grouped decode workload at full size (8 sequences, 32 query heads on
    8 key/value heads, one query row against caches of up to 16384 keys), in
    the automatic range count the benchmark uses; every row of every head
    against the oracle."""
    wl = W.DECODE_WORKLOADS["decode_b8_h32_hkv8_k16384_d128_bf16"]
    inp = W.decode_inputs(wl)
    say("decode", wl.name, "lengths", inp.key_len.tolist())
    o, lse = run_split(inp, True, wl.scale, 0)
    check(inp, True, wl.scale, o, lse, "grouped decode, all heads")


@pytest.mark.parametrize("G", [2, 4, 8])
def test_grouped_decode_negative_scale(G):
    """Grouped decode with a negative scale (the sign folded into each
    head's q) and several ranges."""
    B, H, Nk, d = 2, 2 * G, 900, 128
    inp = W.cache_inputs(B, H, 1, Nk, d, 9140 + G, key_len=[900, 301], Hkv=2)
    o, lse = run_split(inp, True, -0.1, 3)
    check(inp, True, -0.1, o, lse, f"grouped decode G={G}, negative scale")


def test_decode_full_size_sampled_heads():
    """The decode workload at full size (8 sequences, 32 heads, one query row
    against caches of up to 16384 keys with per-sequence lengths), in the
    automatic range count the benchmark uses; the oracle checks every row of
    four heads, and every row must be finite."""
    wl = W.DECODE_WORKLOADS["decode_b8_h32_k16384_d128_bf16"]
    inp = W.decode_inputs(wl)
    say("decode", wl.name, "lengths", inp.key_len.tolist())
    o, lse = run_split(inp, True, wl.scale, 0)
    assert np.all(np.isfinite(lse)) and np.all(np.isfinite(o))
    for h in (0, 7, 19, 31):
        sub = W.Inputs(inp.wl, inp.q[:, h:h + 1], inp.k[:, h:h + 1], inp.v[:, h:h + 1],
                       inp.key_len, None)
        check(sub, True, wl.scale, o[:, h:h + 1], lse[:, h:h + 1], f"decode head {h}")


GQA_CASES = [
    # (B, H, Hkv, Nq, Nk, d, key_len, seed)
    (2, 8, 2, 1, 2000, 128, [2000, 333], 9801),     # grouped decode (4 heads per group)
    (1, 6, 1, 130, 700, 64, None, 9802),            # multi-query, chunked prefill
    (2, 4, 2, 300, 300, 128, None, 9803),           # square
    # decode: the G query heads of a key/value head run as G rows of one
    # query tile (G = 2, 3, 4, 8 and 16 here)
    (3, 4, 2, 1, 1500, 64, [1500, 0, 1], 9804),
    (2, 16, 2, 1, 3001, 128, [3001, 2049], 9805),
    (2, 16, 2, 1, 999, 64, [17, 999], 9806),
    (1, 8, 1, 1, 1200, 128, [1200], 9807),
    (2, 6, 2, 1, 777, 128, [777, 128], 9808),
    (1, 16, 1, 1, 640, 64, [640], 9809),
]


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: f"h{c[1]}kv{c[2]}q{c[3]}k{c[4]}d{c[5]}")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_split_grouped_heads(case, causal, num_splits):
    B, H, Hkv, Nq, Nk, d, key_len, seed = case
    inp = W.cache_inputs(B, H, Nq, Nk, d, seed, key_len=key_len, Hkv=Hkv)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_split(inp, causal, scale, num_splits)
    check(inp, causal, scale, o, lse, f"gqa {case} causal={causal} splits={num_splits}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_decode_negative_scale_and_nan_padding(d, num_splits):
    """One query row per (sequence, head) with a negative scale (the sign is
    folded into q) and NaN in the K/V rows past a sequence's length, which
    must never be read: the result equals the oracle on the clean inputs."""
    import torch
    import io_aware_exact_forward_amd as fa
    B, H, Nk = 2, 3, 700
    inp = W.cache_inputs(B, H, 1, Nk, d, 9131 + d, key_len=[700, 333])
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    nan = torch.tensor(0x7FC0, dtype=torch.int16).view(torch.bfloat16)
    k[1, :, 333:] = nan
    v[1, :, 333:] = nan
    kl = torch.from_numpy(inp.key_len).to("cuda:0")
    scale = -0.1
    say("case", f"decode d={d} splits={num_splits} scale={scale}")
    o, lse = fa.forward_split(q, k, v, scale=scale, causal=True, key_len=kl,
                              num_splits=num_splits)
    torch.cuda.synchronize()
    og = W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)
    check(inp, True, scale, og, lse.cpu().numpy().astype(np.float64),
          f"decode d={d} splits={num_splits} negative scale, NaN padding")
