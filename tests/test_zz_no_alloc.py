"""fa_forward_split_noalloc, the entry point for callers that cannot
allocate device memory, against fa_forward_split with a caller workspace
(same kernels and range plan: the outputs must be identical bit for bit)
and against the fp64 oracle at the bf16 tolerances.  Two calls in a row on
one device, the second on a smaller problem, so the scratch the first call
filled is reused; then a call whose ranges need no scratch.
"""
import ctypes

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


def host(o):
    import torch
    return W.bf16_decode(o.view(torch.int16).cpu().numpy().view(np.uint16), np.float64)


def run_both(inp, H, Hkv, causal, num_splits):
    import torch
    import io_aware_exact_forward_amd as fa
    B, _, Nq, d = inp.q.shape
    Nk = inp.k.shape[2]
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    kl = None if inp.key_len is None else torch.from_numpy(inp.key_len).to("cuda:0")
    klp = kl.data_ptr() if kl is not None else 0
    scale = 1.0 / np.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for noalloc in (False, True):
        o = torch.full_like(q, 7.0)
        lse = torch.full((B, H, Nq), 7.0, device="cuda:0")
        if noalloc:
            st = fa.fa_forward_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                             lse.data_ptr(), B, H, Hkv, Nq, Nk, d, scale,
                                             int(causal), klp, fa.FA_DTYPE_BF16, num_splits,
                                             stream)
        else:
            need = fa.fa_split_workspace_bytes(B, H, Nq, Nk, d, num_splits)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda:0")
            st = fa.fa_forward_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), B, H, Hkv, Nq, Nk, d, scale, int(causal),
                                     klp, fa.FA_DTYPE_BF16, num_splits, ws.data_ptr(), need,
                                     stream)
        assert st == 0, fa.fa_status_string(st)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy().copy(), lse.cpu().numpy().copy()))
    return outs, scale


def check_oracle(inp, H, causal, scale, o_bits, lse):
    tol = TOL["bf16"]
    kx = oracle.expand_kv_heads(inp.exact("k"), H)
    vx = oracle.expand_kv_heads(inp.exact("v"), H)
    o_ref, l_ref = oracle.attention(inp.exact("q"), kx, vx, scale, causal=causal,
                                    key_len=inp.key_len, end_aligned=True)
    o = W.bf16_decode(o_bits.view(np.uint16), np.float64)
    live = np.isfinite(l_ref)
    err = np.abs(o - o_ref)[live]
    stats = dict(o_max=float(err.max()), o_mean=float(err.mean()),
                 lse_max=float(np.abs(lse[live] - l_ref[live]).max()))
    say(stats)
    assert stats["o_max"] <= tol["o_max"] and stats["o_mean"] <= tol["o_mean"], stats
    assert stats["lse_max"] <= tol["lse"], stats
    assert np.all(o[~live] == 0.0) and np.all(lse[~live] == -np.inf)


# (B, H, Hkv, Nq, Nk, d, key_len, causal, num_splits, seed); the second is
# smaller than the first and reuses the scratch the first call wrote
CALLS = [
    (4, 8, 2, 1, 5000, 128, [5000, 1, 0, 3777], True, 0, 7201),      # decode, automatic ranges
    (2, 4, 4, 200, 1500, 64, [1500, 333], True, 3, 7202),             # chunked prefill
]


def test_noalloc_matches_workspace_path_twice():
    import io_aware_exact_forward_amd as fa
    for (B, H, Hkv, Nq, Nk, d, kl, causal, ns, seed) in CALLS:
        need = fa.fa_split_workspace_bytes(B, H, Nq, Nk, d, ns)
        say(f"noalloc B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} splits={ns} "
            f"partials={need} bytes")
        assert 0 < need <= 32 << 20
        inp = W.cache_inputs(B, H, Nq, Nk, d, seed, key_len=kl, Hkv=Hkv)
        (o_ws, l_ws), (o_na, l_na) = run_both(inp, H, Hkv, causal, ns)[0]
        scale = 1.0 / np.sqrt(d)
        assert np.array_equal(o_ws, o_na), "outputs differ from the workspace path"
        assert np.array_equal(l_ws, l_na), "LSE differs from the workspace path"
        check_oracle(inp, H, causal, scale, o_na, l_na)


def test_noalloc_without_ranges_and_over_the_limit():
    import torch
    import io_aware_exact_forward_amd as fa
    # one range: no partial results, no scratch
    inp = W.cache_inputs(1, 2, 64, 700, 128, 7203)
    say("noalloc one range")
    (o_ws, l_ws), (o_na, l_na) = run_both(inp, 2, 2, True, 1)[0]
    assert np.array_equal(o_ws, o_na) and np.array_equal(l_ws, l_na)
    # partials beyond the scratch: refused before any launch, outputs untouched
    B, H, Nq, Nk, d, ns = 1, 8, 1024, 8192, 128, 64
    need = fa.fa_split_workspace_bytes(B, H, Nq, Nk, d, ns)
    assert need > 32 << 20
    q = torch.zeros(B, H, Nq, d, dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros(B, H, Nk, d, dtype=torch.bfloat16, device="cuda:0")
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, Nq), 7.0, device="cuda:0")
    say("noalloc over the limit")
    st = fa.fa_forward_split_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), B, H, H, Nq, Nk, d, 0.1, 1, 0,
                                     fa.FA_DTYPE_BF16, ns, torch.cuda.current_stream().cuda_stream)
    assert st == -8, fa.fa_status_string(st)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
