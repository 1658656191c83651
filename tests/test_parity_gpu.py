"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases and the workloads up to 8 x 16 x 4096 compare every output
element; the 8-head N = 32768 workload compares 512 seeded query rows per
head, which the oracle computes one by one, plus properties that hold for
every row (finiteness).
"""
import math

import numpy as np
import pytest

from io_aware_exact_forward_amd import workloads as W
from parity_util import TOL, check_all_padding, compare, run_hip

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def sample_rows(N, H, per_head, seed, extra=()):
    rng = np.random.default_rng(seed)
    base = [r for r in extra if 0 <= r < N]
    out = []
    for _ in range(H):
        r = set(base) | set(rng.choice(N, min(per_head, N), replace=False).tolist())
        out.append(sorted(r))
    R = min(len(x) for x in out)
    return np.array([x[:R] for x in out], dtype=np.int64)


# ---------------------------------------------------------------------------
# The named workloads at full size, in the launch configuration the bench uses
# ---------------------------------------------------------------------------

def test_single_head_f32_full():
    wl = W.workload("single_head_n256_d64_f32")
    inp = W.make_inputs(wl)
    say("case", wl.name)
    o, lse = run_hip(inp, wl.causal, wl.scale)
    st = compare(inp, o, lse, wl.causal, wl.scale, label=wl.name)
    say(st)


def test_h32_n2048_causal_full():
    wl = W.workload("h32_n2048_d64_causal_bf16")
    inp = W.make_inputs(wl)
    say("case", wl.name)
    o, lse = run_hip(inp, wl.causal, wl.scale)
    st = compare(inp, o, lse, wl.causal, wl.scale, label=wl.name)
    say(st)


def test_h32_n8192_d128_causal_full():
    """Every row of every head (262,144 rows): O max and mean error and LSE
    error over all of them (the oracle takes ~15 s on 16 host threads)."""
    wl = W.workload("h32_n8192_d128_causal_bf16")
    inp = W.make_inputs(wl)
    say("case", wl.name)
    o, lse = run_hip(inp, wl.causal, wl.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    st = compare(inp, o, lse, wl.causal, wl.scale, label=wl.name)
    say(st)
    assert st["rows_checked"] == wl.B * wl.H * wl.N


def test_b8_keylen_full():
    """Every row of every (batch, head): valid rows against the oracle (max,
    mean and LSE error over all of them), padding rows exactly 0 / -inf."""
    wl = W.workload("b8_h16_n4096_d64_keylen_bf16")
    inp = W.make_inputs(wl)
    say("case", wl.name, "key_len", inp.key_len.tolist())
    o, lse = run_hip(inp, wl.causal, wl.scale)
    check_all_padding(inp, o, lse)
    st = compare(inp, o, lse, wl.causal, wl.scale, label=wl.name)
    say(st)
    lens = np.clip(inp.key_len.astype(np.int64), 0, wl.N)
    assert st["rows_checked"] == wl.H * int(lens.sum())


def test_h8_n32768_causal_sampled():
    wl = W.workload("h8_n32768_d128_causal_bf16")
    inp = W.make_inputs(wl)
    say("case", wl.name)
    o, lse = run_hip(inp, wl.causal, wl.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    st = compare(inp, o, lse, wl.causal, wl.scale, rows=inp.rows, label=wl.name)
    say(st)


# ---------------------------------------------------------------------------
# Launch forms chosen by grid size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_causal_grid_beyond_one_pass(d):
    """A causal batch whose 128-row grid does not fit the device at once
    (24 heads x 24 tiles = 576 workgroups > two per CU) but is too small for
    the 256-row form: the four-wave lockstep launch.  (Smaller causal grids,
    such as every case of the edge sweep below, take the two-key-group form,
    paired when the pairs fill the device.)
    Ragged N; every element compared."""
    N = 3000
    inp = W.random_inputs(3, 8, N, d, "bf16", seed=2100 + d)
    scale = 1.0 / math.sqrt(d)
    say("case lockstep causal", d)
    o, lse = run_hip(inp, True, scale)
    compare(inp, o, lse, True, scale, label=f"lockstep causal d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_causal_two_key_groups_odd_tiles(d):
    """The two-key-group form with an odd number of key tiles per query tile
    (group 1 idles on the last step), a ragged last query tile and several
    query tiles per head; every element compared."""
    N = 1000 if d == 64 else 900
    inp = W.random_inputs(2, 3, N, d, "bf16", seed=2200 + d)
    scale = 1.0 / math.sqrt(d)
    say("case two key groups", d)
    o, lse = run_hip(inp, True, scale)
    compare(inp, o, lse, True, scale, label=f"two key groups d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", [(2, 32, 1000), (5, 32, 300), (4, 64, 100)])
def test_causal_paired_tiles(d, B, H, N):
    """The paired form: a causal grid of 128-row tiles whose pairs (query tiles
    j and n - 1 - j of one head) fill the device's 256 compute units.  Even
    tile count with a middle pair whose second group sees only the light
    tile (N = 1000), odd count with the middle tile alone and a ragged last
    tile (N = 300), one tile per head (N = 100); every element compared."""
    inp = W.random_inputs(B, H, N, d, "bf16", seed=2300 + d + N)
    scale = 1.0 / math.sqrt(d)
    say("case paired", B, H, N, d)
    o, lse = run_hip(inp, True, scale)
    compare(inp, o, lse, True, scale, label=f"paired {B}x{H}x{N} d={d}")


# ---------------------------------------------------------------------------
# Edge sweep at small sizes: every element compared
# ---------------------------------------------------------------------------

EDGE_N = [1, 2, 3, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 300]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_sweep(dtype, d, causal):
    for N in EDGE_N:
        inp = W.random_inputs(2, 2, N, d, dtype, seed=1000 + N)
        scale = 1.0 / math.sqrt(d)
        say("case", dtype, d, causal, N)
        o, lse = run_hip(inp, causal, scale)
        compare(inp, o, lse, causal, scale, label=f"{dtype} d={d} causal={causal} N={N}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_key_length_mix(dtype, d, causal):
    N = 300
    # 0, 1, around both key-tile sizes (64, 128), N, beyond N (clamped), negative (clamped)
    key_len = [0, 1, 63, 64, 65, 127, 128, 129, 255, 300, 1000, -3]
    inp = W.random_inputs(len(key_len), 2, N, d, dtype, seed=77, key_len=key_len)
    scale = 1.0 / math.sqrt(d)
    say("case keylen", dtype, d, causal)
    o, lse = run_hip(inp, causal, scale)
    compare(inp, o, lse, causal, scale, label=f"keylen {dtype} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_key_lengths_longest_first_order(d):
    """A non-causal batch of at most 8 sequences with key lengths runs its
    sequences longest first, each followed by its padding tiles: lengths
    with ties, an empty, a negative and an over-long one, so that the
    ranking has to be a permutation for every tile to be written once."""
    import torch
    import io_aware_exact_forward_amd as fa
    from parity_util import from_device, to_device

    N = 300
    key_len = [300, 0, 129, 300, -3, 64, 1000, 129]
    inp = W.random_inputs(len(key_len), 2, N, d, "bf16", seed=88, key_len=key_len)
    scale = 1.0 / math.sqrt(d)
    say("case longest first", d)
    q, k, v, kl = to_device(inp)
    # outputs start as NaN, so a tile that no workgroup writes shows up
    out = torch.full_like(q, float("nan"))
    lse_t = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fa.forward(q, k, v, scale=scale, causal=False, key_len=kl, out=out, lse=lse_t)
    torch.cuda.synchronize()
    o, lse = from_device(out), lse_t.cpu().numpy().astype(np.float64)
    check_all_padding(inp, o, lse)
    compare(inp, o, lse, False, scale, label=f"longest first d={d}")


@pytest.mark.parametrize("q_mult", [3.0, 10.0])
@pytest.mark.parametrize("d", [64, 128])
def test_peaky_rows(q_mult, d):
    inp = W.random_inputs(1, 4, 513, d, "bf16", seed=5, q_mult=q_mult)
    scale = 1.0 / math.sqrt(d)
    for causal in (False, True):
        say("case peaky", q_mult, d, causal)
        o, lse = run_hip(inp, causal, scale)
        compare(inp, o, lse, causal, scale, label=f"peaky x{q_mult} d={d} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_dominant_key_in_last_block(dtype, d):
    """A key whose score exceeds all earlier ones by ~20-30 (natural-log
    units) arrives in the last tile, so the running state is rescaled by a
    factor near exp(-25).  The scale is the usual 1/sqrt(d): fp32 cannot hold
    a 1e-5 absolute output error when scores themselves reach the hundreds,
    because rounding a score s moves its weight by about |s| * 2^-24."""
    N = 400
    inp = W.random_inputs(1, 2, N, d, dtype, seed=9)
    qx = inp.exact("q")
    kdir = qx[0, :, :, :].mean(axis=1)  # [H, d]
    kdir /= np.linalg.norm(kdir, axis=1, keepdims=True)
    kbig = (kdir * 20.0 * math.sqrt(d)).astype(np.float32)
    for hh in range(2):
        if dtype == "bf16":
            inp.k[0, hh, N - 1] = W.bf16_encode(kbig[hh])
        else:
            inp.k[0, hh, N - 1] = kbig[hh]
    scale = 1.0 / math.sqrt(d)
    say("case dominant", dtype, d)
    o, lse = run_hip(inp, False, scale)
    compare(inp, o, lse, False, scale, label=f"dominant {dtype} d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scale_edge_cases(dtype):
    inp = W.random_inputs(1, 2, 200, 64, dtype, seed=11, key_len=None)
    for scale in (0.0, -0.125, 0.5):
        for causal in (False, True):
            say("case scale", dtype, scale, causal)
            o, lse = run_hip(inp, causal, scale)
            compare(inp, o, lse, causal, scale, label=f"scale={scale} {dtype} causal={causal}")


def test_nan_in_padding_is_ignored():
    """Keys and values beyond a sequence's length never reach the output."""
    N, d = 200, 64
    inp = W.random_inputs(2, 2, N, d, "bf16", seed=12, key_len=[70, 200])
    nan = W.bf16_encode(np.array([np.nan], np.float32))[0] | np.uint16(0x40)
    inp.k[0, :, 70:] = nan
    inp.v[0, :, 70:] = nan
    inp.q[0, :, 70:] = nan
    say("case nan padding")
    o, lse = run_hip(inp, True, 0.125)
    inp.k[0, :, 70:] = 0
    inp.v[0, :, 70:] = 0
    inp.q[0, :, 70:] = 0
    compare(inp, o, lse, True, 0.125, label="nan in padding")


# ---------------------------------------------------------------------------
# The glossary page's worked examples on the device (fp32)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("scores,values,expected", [
    ((1, 2, 3), (1, 2, 4), 17 / 6),
    ((1, 3, 2), (2, 6, 10), 20 / 3),
])
def test_worked_examples_on_device(scores, values, expected):
    """q = e_0 (d = 64), k_j = ln(w_j) e_0, v_j = value_j e_0, scale 1: the
    last query sees all three keys and its output is the printed value."""
    import torch
    import io_aware_exact_forward_amd as fa
    n, d = 3, 64
    q = torch.zeros(1, 1, n, d)
    k = torch.zeros(1, 1, n, d)
    v = torch.zeros(1, 1, n, d)
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = torch.tensor([math.log(w) for w in scores])
    v[0, 0, :, 0] = torch.tensor(values, dtype=torch.float32)
    say("case worked example", scores, values)
    for causal in (False, True):
        o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), scale=1.0, causal=causal)
        torch.cuda.synchronize()
        assert abs(o[0, 0, 2, 0].item() - expected) < 1e-5
        assert abs(lse[0, 0, 2].item() - math.log(6)) < 1e-5
        assert torch.all(o[0, 0, :, 1:] == 0)


def test_repeatable_bitwise():
    import torch
    wl = W.workload("h32_n2048_d64_causal_bf16")
    inp = W.make_inputs(wl, H=8)
    say("case determinism")
    o1, l1 = run_hip(inp, True, wl.scale)
    o2, l2 = run_hip(inp, True, wl.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------------------
# The materialised three-pass baseline (loosely gated: S and P are rounded
# to bf16 in device memory)
# ---------------------------------------------------------------------------

NAIVE_TOL = {"bf16": dict(o_max=6e-2, o_mean=6e-3, lse=3e-2), "f32": dict(o_max=1e-5, o_mean=1e-5, lse=1e-4)}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_naive_baseline_small(dtype, causal):
    inp = W.random_inputs(3, 2, 300, 64, dtype, seed=21, key_len=[300, 100, 0])
    say("case naive", dtype, causal)
    o, lse = run_hip(inp, causal, 0.125, naive=True)
    compare(inp, o, lse, causal, 0.125, tol=NAIVE_TOL[dtype], label=f"naive {dtype} causal={causal}")


def test_naive_baseline_h32_n2048():
    wl = W.workload("h32_n2048_d64_causal_bf16")
    inp = W.make_inputs(wl)
    say("case naive", wl.name)
    o, lse = run_hip(inp, True, wl.scale, naive=True)
    rows = sample_rows(wl.N, wl.H, 64, 3, extra=(0, 2047))
    st = compare(inp, o, lse, True, wl.scale, rows=rows, tol=NAIVE_TOL["bf16"], label="naive " + wl.name)
    say(st)
