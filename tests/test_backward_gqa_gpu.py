"""GPU parity of the grouped-head and packed backward (fa_backward_gqa,
fa_backward_varlen) against the fp64 gradient oracle.

Each case runs the HIP forward of the same layout (fa_forward_split or
fa_forward_varlen) for O and LSE, then the HIP backward, and compares dQ, dK
and dV element by element with oracle.grouped_attention_backward /
oracle.varlen_attention_backward on the same exact bf16 inputs.  The
tolerance is the one derived for the square backward (test_backward_gpu.py):
per gradient tensor, max error <= 1.2e-2 * max |ref| and mean error <= 1.2e-2 *
mean |ref|; a key/value gradient sums H / Hkv such terms, each within that
bound relative to its own scale.  Where no pair is visible (keys at or beyond
a length, rows before the first key under the causal mask, sequences without
queries or keys) the gradients must be exactly zero.

Cases: grouped heads with fewer, equal and more query rows than keys (rows at
the end of the keys), lengths below the cache size, a decode row, d = 64 and
128, empty query and key sets; packed batches with empty, one-token and
ragged sequences and unequal query/key lengths; the full-size packed causal
workload (16 sequences up to 8192 tokens, 32 query heads on 8 key/value
heads) on sampled sequences and head groups.
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


def compare(got, ref, label):
    stats = {"label": label}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert g.shape == r.shape, (label, name, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite"
        if r.size == 0 or not np.any(r):
            assert np.all(g == 0), f"{label} {name}: expected zeros"
            continue
        err = np.abs(g - r)
        smax, smean = float(np.abs(r).max()), float(np.abs(r).mean())
        stats[name] = (float(err.max()) / smax, float(err.mean()) / smean)
        assert err.max() <= TOL_MAX * smax, f"{label} {name}: max err {err.max():.3g} vs {smax:.3g}"
        assert err.mean() <= TOL_MEAN * smean, f"{label} {name}: mean err {err.mean():.3g} vs {smean:.3g}"
    say(stats)


def bf16_normal(shape, rng):
    return W.bf16_encode(rng.standard_normal(shape, dtype=np.float32))


# ---------------------------------------------------------------------------
# grouped heads, dense layout (fa_backward_gqa)
# ---------------------------------------------------------------------------

def run_gqa(inp, do_bits, causal, scale, Hkv):
    import torch
    import io_aware_exact_forward_amd as fa
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(do_bits)
    kl = None if inp.key_len is None else torch.from_numpy(inp.key_len).to("cuda:0")
    o, lse = fa.forward_split(q, k, v, scale=scale, causal=causal, key_len=kl, num_splits=1)
    dq, dk, dv = fa.backward_gqa(q, k, v, o, lse, do, scale=scale, causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


GQA_CASES = [
    # (B, H, Hkv, Nq, Nk, d, key_len, seed)
    (2, 8, 2, 200, 200, 64, [200, 77], 9601),   # rows before the first key when L_b < Nq
    (1, 4, 1, 130, 300, 128, None, 9602),       # fewer rows than keys
    (1, 4, 4, 300, 130, 64, None, 9603),        # more rows than keys
    (2, 6, 3, 1, 257, 64, [257, 100], 9604),    # decode row
    (1, 2, 1, 64, 64, 128, None, 9605),         # one tile
    (1, 8, 1, 333, 333, 128, [5], 9606),        # multi-query, short length
]


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: f"h{c[1]}kv{c[2]}q{c[3]}k{c[4]}d{c[5]}")
@pytest.mark.parametrize("causal", [False, True])
def test_backward_gqa_against_oracle(case, causal):
    B, H, Hkv, Nq, Nk, d, key_len, seed = case
    say("case", case, "causal", causal)
    inp = W.cache_inputs(B, H, Nq, Nk, d, seed, key_len=key_len, Hkv=Hkv)
    do = bf16_normal((B, H, Nq, d), np.random.default_rng(seed + 50))
    scale = 1.0 / np.sqrt(d)
    got = run_gqa(inp, do, causal, scale, Hkv)
    ref = oracle.grouped_attention_backward(inp.exact("q"), inp.exact("k"), inp.exact("v"),
                                            W.bf16_decode(do, np.float64), scale, causal=causal,
                                            key_len=inp.key_len, end_aligned=True)[:3]
    compare(got, ref, f"{case} causal={causal}")
    # exact zeros: keys at or beyond L_b; rows that see no key (position
    # i + L_b - Nq < 0 under the causal mask, every row when L_b = 0)
    lens = [Nk] * B if key_len is None else np.clip(key_len, 0, Nk)
    for b, L in enumerate(lens):
        assert np.all(got[1][b, :, L:] == 0) and np.all(got[2][b, :, L:] == 0)
        blind = Nq if L == 0 else (max(0, Nq - L) if causal else 0)
        assert np.all(got[0][b, :, :blind] == 0)


def test_backward_gqa_empty_sides():
    """No query rows: dK = dV = 0.  No keys: dQ = 0."""
    import torch
    import io_aware_exact_forward_amd as fa
    rng = np.random.default_rng(9610)
    k = dev(bf16_normal((1, 2, 70, 64), rng))
    v = dev(bf16_normal((1, 2, 70, 64), rng))
    q0 = torch.empty((1, 4, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    lse0 = torch.empty((1, 4, 0), dtype=torch.float32, device="cuda:0")
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    fa.backward_gqa(q0, k, v, q0, lse0, q0, dk=dk, dv=dv, causal=True)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
    q = dev(bf16_normal((1, 4, 9, 64), rng))
    do = dev(bf16_normal((1, 4, 9, 64), rng))
    k0 = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    o, lse = fa.forward_split(q, k0, k0, causal=False)
    dq = torch.full_like(q, 7.0)
    fa.backward_gqa(q, k0, k0, o, lse, do, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


# ---------------------------------------------------------------------------
# packed batches (fa_backward_varlen)
# ---------------------------------------------------------------------------

def run_varlen(inp, do_bits, causal, scale, max_q, max_k):
    import torch
    import io_aware_exact_forward_amd as fa
    cq = torch.from_numpy(inp.cu_q).to("cuda:0")
    ck = torch.from_numpy(inp.cu_k).to("cuda:0")
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(do_bits)
    o, lse = fa.forward_varlen(q, k, v, cq, ck, max_q, max_k, scale=scale, causal=causal)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, lse, do, cq, ck, max_q, max_k, scale=scale,
                                    causal=causal)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


VARLEN_CASES = [
    # (lens_q, lens_k, H, Hkv, d, seed)
    ([0, 1, 63, 64, 65, 128, 129, 300], [5, 1, 63, 100, 65, 128, 0, 300], 4, 2, 64, 9701),
    ([200, 17, 513], [200, 17, 513], 6, 1, 128, 9702),
    ([40, 300, 1], [300, 40, 2], 4, 4, 128, 9703),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"h{c[2]}kv{c[3]}d{c[4]}s{c[5]}")
@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_against_oracle(case, causal):
    lens_q, lens_k, H, Hkv, d, seed = case
    say("case", case, "causal", causal)
    inp = W.packed_inputs(lens_q, lens_k, H, Hkv, d, seed)
    do = bf16_normal((int(inp.cu_q[-1]), H, d), np.random.default_rng(seed + 50))
    scale = 1.0 / np.sqrt(d)
    got = run_varlen(inp, do, causal, scale, max(lens_q), max(lens_k))
    ref = oracle.varlen_attention_backward(inp.exact("q"), inp.exact("k"), inp.exact("v"),
                                           W.bf16_decode(do, np.float64), inp.cu_q, inp.cu_k,
                                           scale, causal=causal)[:3]
    compare(got, ref, f"{case} causal={causal}")
    # exact zeros: keys of sequences without queries, rows that see no key
    for b, (lq, lk) in enumerate(zip(lens_q, lens_k)):
        if lq == 0:
            assert np.all(got[1][inp.cu_k[b]:inp.cu_k[b + 1]] == 0)
            assert np.all(got[2][inp.cu_k[b]:inp.cu_k[b + 1]] == 0)
        blind = lq if lk == 0 else (max(0, lq - lk) if causal else 0)
        assert np.all(got[0][inp.cu_q[b]:inp.cu_q[b] + blind] == 0)


def test_backward_varlen_full_size_sampled():
    """The full packed causal workload; dQ of two head groups and dK, dV of
    their key/value heads on the three shortest sequences and the one nearest
    2048 tokens, each against the oracle on that sequence alone."""
    wl = W.VARLEN_WORKLOADS["varlen_b16_h32_hkv8_n8192_d128_bf16"]
    inp = W.varlen_inputs(wl)
    lens = np.diff(inp.cu_q)
    Tq = int(inp.cu_q[-1])
    do = bf16_normal((Tq, wl.H, wl.d), np.random.default_rng(wl.seed + 50))
    say("full-size packed backward", wl.name, "tokens", Tq)
    got = run_varlen(inp, do, True, wl.scale, int(lens.max()), int(lens.max()))
    order = np.argsort(lens)
    seqs = sorted(set(order[:3].tolist()) | {int(np.argmin(np.abs(lens - 2048)))})
    G = wl.H // wl.Hkv
    kv_heads = [0, wl.Hkv - 1]
    heads = [h for g in kv_heads for h in range(g * G, g * G + G)]
    qx, kx, vx = inp.exact("q"), inp.exact("k"), inp.exact("v")
    dox = W.bf16_decode(do, np.float64)
    cq, ck = inp.cu_q, inp.cu_k
    for b in seqs:
        a, z = int(cq[b]), int(cq[b + 1])
        ka, kz = int(ck[b]), int(ck[b + 1])
        cu1q, cu1k = np.array([0, z - a]), np.array([0, kz - ka])
        ref = oracle.varlen_attention_backward(qx[a:z][:, heads], kx[ka:kz][:, kv_heads],
                                               vx[ka:kz][:, kv_heads], dox[a:z][:, heads],
                                               cu1q, cu1k, wl.scale, causal=True)[:3]
        sub = (got[0][a:z][:, heads], got[1][ka:kz][:, kv_heads], got[2][ka:kz][:, kv_heads])
        compare(sub, ref, f"{wl.name} sequence {b} (length {z - a})")
