"""GPU parity of the balanced decode step against the fp64 oracle.

A decode step (one query row per sequence and head, as many key/value heads
as query heads) with the automatic range count cuts the visible keys of all
rows, in 64-key units, into equal shares on the device.  A row inside one
share is written by the decode kernel; a row cut by share boundaries is
merged from its shares' partial results.  The cases cover more sequences
than one wave scans at once (B > 64), sequences with no key (length 0 or
negative), lengths past the cache (clamped), fewer units than shares (empty
shares), rows that are whole and rows that are cut, d = 64 and 128, and the
full-size decode workload, whose every row is checked against the oracle.
"""
import numpy as np
import pytest

from io_aware_exact_forward_amd import workloads as W
from test_split_gpu import check, run_split, say

pytestmark = pytest.mark.gpu


CASES = [
    # (B, H, Nk, d, key_len, seed)
    (130, 2, 700, 64, "random", 9901),        # 130 sequences: three scan blocks
    (130, 2, 700, 128, "random", 9902),
    (3, 4, 20000, 128, [20000, 64, 65], 9903),  # long and one- or two-unit rows
    (2, 2, 5000, 64, None, 9904),             # no lengths: every key visible
    (5, 3, 900, 128, [0, -3, 901, 1, 0], 9905),  # empty, negative, clamped, one key
    (1, 1, 40000, 128, [39999], 9906),        # one row over all shares
    (70, 1, 300, 64, "random", 9907),
]


def lengths(spec, B, Nk, seed):
    if spec != "random":
        return spec
    rng = np.random.default_rng(seed)
    kl = rng.integers(0, Nk + 1, size=B).astype(np.int32)
    kl[::17] = 0
    return kl.tolist()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}h{c[1]}k{c[2]}d{c[3]}")
def test_balanced_decode_against_oracle(case):
    B, H, Nk, d, spec, seed = case
    kl = lengths(spec, B, Nk, seed)
    say("case", case[:4], "lengths", kl if kl is None or len(kl) < 10 else f"{len(kl)} values")
    inp = W.cache_inputs(B, H, 1, Nk, d, seed, key_len=kl)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_split(inp, True, scale, 0)
    check(inp, True, scale, o, lse, f"balanced decode {case[:4]}")


def test_balanced_decode_all_sequences_empty():
    inp = W.cache_inputs(4, 2, 1, 500, 128, 9908, key_len=[0, 0, -1, 0])
    o, lse = run_split(inp, True, 0.1, 0)
    assert np.all(o == 0.0) and np.all(lse == -np.inf)


def test_balanced_decode_full_size_every_row():
    """The decode workload at full size (8 sequences, 32 heads, caches of up
    to 16384 keys with per-sequence lengths) through the balanced shares the
    benchmark times: every row against the oracle, and against the fixed
    ranges of two splits within the same tolerance."""
    wl = W.DECODE_WORKLOADS["decode_b8_h32_k16384_d128_bf16"]
    inp = W.decode_inputs(wl)
    say("decode", wl.name, "lengths", inp.key_len.tolist())
    o, lse = run_split(inp, True, wl.scale, 0)
    check(inp, True, wl.scale, o, lse, "balanced decode, full size")
    o2, lse2 = run_split(inp, True, wl.scale, 2)
    assert np.abs(o - o2).max() <= 2e-2 and np.abs(lse - lse2).max() <= 1e-4
