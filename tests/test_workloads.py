"""Host-side checks of the seeded input generators (no GPU, no attention math)."""
import numpy as np
import pytest
import torch

from io_aware_exact_forward_amd import workloads as W


def test_bf16_encode_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        np.array([0.0, -0.0, 1.0, -1.0, 1e-40, 3.3895314e38, 1.00390625, 1.01171875], np.float32),
    ])
    ours = W.bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_to_even():
    # 1 + 2^-8 lies exactly between two bf16 values: rounds to the even one (1.0)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)
    u = W.bf16_encode(x)
    assert W.bf16_decode(u)[0] == 1.0
    assert W.bf16_decode(u)[1] == 1.0 + 2.0 ** -6


def test_decode_is_exact_widening():
    u = np.arange(0, 65536, 7, dtype=np.uint16)
    f = W.bf16_decode(u, np.float32)
    assert np.array_equal(W.bf16_encode(f[np.isfinite(f)]), u[np.isfinite(f)])


def test_inputs_are_seeded_and_deterministic():
    wl = W.workload(1)
    a = W.make_inputs(wl, H=2, N=64)
    b = W.make_inputs(wl, H=2, N=64)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    c = W.make_inputs(wl, H=2, N=64, seed=wl.seed + 1)
    assert not np.array_equal(a.q, c.q)


def test_workload_shapes_and_extras():
    assert len(W.WORKLOADS) == 5
    wl = W.workload("b8_h16_n4096_d64_keylen_bf16")
    inp = W.make_inputs(wl, H=1, N=4096, d=8)
    assert inp.key_len.shape == (8,) and inp.key_len.dtype == np.int32
    assert inp.key_len.min() >= 1 and inp.key_len.max() <= 4096
    wl5 = W.workload(4)
    inp5 = W.make_inputs(wl5, H=2, N=2048, d=8)
    assert inp5.rows.shape == (2, 512)
    assert np.all(np.diff(inp5.rows, axis=1) > 0)
    assert W.workload(0).dtype == "f32" and W.make_inputs(W.workload(0)).q.dtype == np.float32


def test_q_multiplier_applied_before_encoding():
    wl = W.workload("b8_h16_n4096_d64_keylen_bf16")
    a = W.make_inputs(wl, B=1, H=1, N=16, d=8)
    b = W.make_inputs(wl, B=1, H=1, N=16, d=8, q_mult=1.0)
    assert np.allclose(W.bf16_decode(a.q), 3 * W.bf16_decode(b.q), rtol=2 ** -7)


@pytest.mark.parametrize("causal", [False, True])
def test_valid_pairs_counts(causal):
    N = 37
    key_len = [0, 1, 5, 37, 50]
    count = 0
    for L in key_len:
        L = min(L, N)
        for i in range(N):
            for j in range(N):
                if i < L and j < L and (not causal or j <= i):
                    count += 1
    assert W.valid_pairs(N, causal, key_len, B=len(key_len)) == count
    assert W.valid_pairs(N, causal) == (N * (N + 1) // 2 if causal else N * N)
