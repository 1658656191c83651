"""Seeded synthetic workloads for the attention forward pass.

This module only draws random numbers and encodes them; it performs none of
the attention arithmetic.  Both the HIP path (through the tests and the bench)
and the fp64 oracle consume what it produces, so it imports nothing but numpy.

The five workloads follow the shapes the pages use for long-context attention
("IO-aware exact attention", introduction: batch 1, 32 heads, N = 8192; the
same page's backward exercise uses batch 2, 16 heads, d = 64) plus a
correctness-sized case, a mid-size causal case, a padded case with
per-sequence key lengths, and a long-context causal case.

Recipe (fixed, so that any run can regenerate the exact bits):
  * ``rng = numpy.random.default_rng(seed)``;
  * Q, K, V drawn in that order with ``rng.standard_normal(shape, float32)``;
  * optional Q multiplier applied in fp32 before encoding (peaky softmax rows);
  * bf16 encoding is round-to-nearest-even on the fp32 bit pattern;
  * per-sequence key lengths, when present, are drawn after V with
    ``rng.integers(1, N, size=B, endpoint=True)``;
  * sampled query rows, when present, are drawn after that, per head, with
    ``rng.choice(N, rows, replace=False)`` and sorted.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "bf16_encode",
    "bf16_decode",
    "make_inputs",
    "valid_pairs",
    "cache_inputs",
    "decode_inputs",
    "DecodeWorkload",
    "DECODE_WORKLOADS",
    "Inputs",
    "grad_inputs",
    "BWD_WORKLOADS",
    "PackedInputs",
    "packed_inputs",
    "VarlenWorkload",
    "VARLEN_WORKLOADS",
    "varlen_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" or "bf16"
    causal: bool
    scale: float
    seed: int
    q_mult: float = 1.0
    ragged: bool = False  # per-sequence key lengths ~ U[1, N]
    sample_rows: int = 0  # >0: query rows per head the oracle checks

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "B": self.B, "H": self.H, "N": self.N, "d": self.d,
            "dtype": self.dtype, "causal": self.causal,
            "scale": self.scale, "q_mult": self.q_mult,
            "ragged_key_len": self.ragged,
        }


WORKLOADS = {
    # correctness-sized, fp32 end to end
    "single_head_n256_d64_f32": Workload(
        "single_head_n256_d64_f32", 1, 1, 256, 64, "f32", False, 1.0 / 8.0, 1001),
    # 32 heads, N=2048, d=64, causal
    "h32_n2048_d64_causal_bf16": Workload(
        "h32_n2048_d64_causal_bf16", 1, 32, 2048, 64, "bf16", True, 1.0 / 8.0, 1002),
    # 32 heads, N=8192, d=128, causal: the shape whose fp16 score matrix is ~4 GiB
    "h32_n8192_d128_causal_bf16": Workload(
        "h32_n8192_d128_causal_bf16", 1, 32, 8192, 128, "bf16", True,
        1.0 / math.sqrt(128.0), 1003),
    # batch 8, 16 heads, N=4096, d=64, Q x3, per-sequence key length
    "b8_h16_n4096_d64_keylen_bf16": Workload(
        "b8_h16_n4096_d64_keylen_bf16", 8, 16, 4096, 64, "bf16", False, 1.0 / 8.0, 1004,
        q_mult=3.0, ragged=True),
    # 8 heads, N=32768, d=128, causal long context; 512 sampled rows per head
    "h8_n32768_d128_causal_bf16": Workload(
        "h8_n32768_d128_causal_bf16", 1, 8, 32768, 128, "bf16", True,
        1.0 / math.sqrt(128.0), 1005, sample_rows=512),
}

# The order in which the workloads are listed above; index 0 is the small one.
WORKLOAD_ORDER = list(WORKLOADS)


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[WORKLOAD_ORDER[name_or_index]]
    return WORKLOADS[name_or_index]


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Inputs here are finite normal draws; NaN payloads are not handled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_decode(u: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bf16 bit pattern (uint16) -> exact float value (fp32 widened to ``dtype``)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    f = (u.astype(np.uint32) << 16).view(np.float32)
    return f.astype(dtype)


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs.

    ``q``, ``k`` and ``v`` hold the device encoding: uint16 bf16 bit patterns
    for bf16 workloads, float32 for f32 ones.  ``key_len`` is int32 [B] or
    None.  ``rows`` is int64 [H, R] (sorted per head) or None.
    """
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    key_len: np.ndarray | None
    rows: np.ndarray | None

    def exact(self, name: str) -> np.ndarray:
        """The exact fp64 value of a device tensor ('q', 'k' or 'v')."""
        a = getattr(self, name)
        if self.wl.dtype == "bf16":
            return bf16_decode(a, np.float64)
        return a.astype(np.float64)


def make_inputs(wl: Workload, *, B=None, H=None, N=None, d=None, seed=None,
                q_mult=None) -> Inputs:
    """Draw one workload's inputs; keyword overrides give smaller variants."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    N = wl.N if N is None else N
    d = wl.d if d is None else d
    seed = wl.seed if seed is None else seed
    q_mult = wl.q_mult if q_mult is None else q_mult
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    key_len = None
    if wl.ragged:
        key_len = rng.integers(1, N, size=B, endpoint=True, dtype=np.int64).astype(np.int32)
    rows = None
    if wl.sample_rows:
        r = min(wl.sample_rows, N)
        rows = np.stack([np.sort(rng.choice(N, r, replace=False)) for _ in range(H)])
        rows = rows.astype(np.int64)
    if wl.dtype == "bf16":
        q, k, v = bf16_encode(q), bf16_encode(k), bf16_encode(v)
    return Inputs(wl, q, k, v, key_len, rows)


def random_inputs(B, H, N, d, dtype, seed, *, q_mult=1.0, key_len=None):
    """Generic seeded draw (same recipe) for test shapes that are not a named workload."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    if dtype == "bf16":
        q, k, v = bf16_encode(q), bf16_encode(k), bf16_encode(v)
    kl = None if key_len is None else np.asarray(key_len, dtype=np.int32)
    wl = Workload(f"random_b{B}_h{H}_n{N}_d{d}_{dtype}", B, H, N, d, dtype, False,
                  1.0 / math.sqrt(d), seed, q_mult=q_mult)
    return Inputs(wl, q, k, v, kl, None)


def cache_inputs(B, H, Nq, Nk, d, seed, *, q_mult=1.0, key_len=None, Hkv=None):
    """Query rows against a longer key cache (same recipe, bf16): q [B, H, Nq, d]
    is drawn first, then k and v [B, Hkv, Nk, d] (Hkv = H unless given)."""
    Hkv = H if Hkv is None else Hkv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    kl = None if key_len is None else np.asarray(key_len, dtype=np.int32)
    wl = Workload(f"cache_b{B}_h{H}_q{Nq}_k{Nk}_d{d}_bf16", B, H, Nk, d, "bf16", False,
                  1.0 / math.sqrt(d), seed, q_mult=q_mult)
    return Inputs(wl, bf16_encode(q), bf16_encode(k), bf16_encode(v), kl, None)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One query row per (sequence, head) against a key cache of Nk rows
    whose per-sequence lengths are uniform on [1, Nk]; causal, bf16.  Hkv
    key/value heads (0: as many as query heads); query head h reads head
    h // (H // Hkv)."""
    name: str
    B: int
    H: int
    Nk: int
    d: int
    seed: int
    Hkv: int = 0

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "Hkv": self.kv_heads, "Nq": 1,
                "Nk": self.Nk, "d": self.d, "dtype": "bf16", "causal": True,
                "scale": self.scale, "key_len": "per sequence, uniform on [1, Nk]"}


DECODE_WORKLOADS = {
    # decode step of 8 sequences x 32 heads, d = 128, caches of up to 16384 keys
    "decode_b8_h32_k16384_d128_bf16": DecodeWorkload(
        "decode_b8_h32_k16384_d128_bf16", 8, 32, 16384, 128, 1006),
    # the same with 32 query heads on 8 key/value heads (four per group)
    "decode_b8_h32_hkv8_k16384_d128_bf16": DecodeWorkload(
        "decode_b8_h32_hkv8_k16384_d128_bf16", 8, 32, 16384, 128, 1007, Hkv=8),
}


def decode_inputs(wl: DecodeWorkload, *, B=None, H=None, Nk=None, seed=None) -> "Inputs":
    """q [B, H, 1, d], then k, v [B, Hkv, Nk, d], then key lengths (same
    recipe); keyword overrides give smaller variants."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    Nk = wl.Nk if Nk is None else Nk
    seed = wl.seed if seed is None else seed
    d = wl.d
    Hkv = H if not wl.Hkv else wl.Hkv * H // wl.H
    rng = np.random.default_rng(seed)
    q = bf16_encode(rng.standard_normal((B, H, 1, d), dtype=np.float32))
    k = bf16_encode(rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32))
    v = bf16_encode(rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32))
    kl = rng.integers(1, Nk, size=B, endpoint=True, dtype=np.int64).astype(np.int32)
    sq = Workload(wl.name, B, H, Nk, d, "bf16", True, wl.scale, seed, ragged=True)
    return Inputs(sq, q, k, v, kl, None)


@dataclasses.dataclass
class PackedInputs:
    """A packed batch: q [Tq, H, d], k and v [Tk, Hkv, d] as bf16 bits, and
    the int32 row offsets [B + 1] of the sequences."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray

    def exact(self, name: str) -> np.ndarray:
        return bf16_decode(getattr(self, name), np.float64)


def packed_inputs(lens_q, lens_k, H, Hkv, d, seed):
    """Packed variable-length batch (same recipe): q, then k, then v, each
    standard normal, rounded to bf16."""
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((int(cu_q[-1]), H, d), dtype=np.float32)
    k = rng.standard_normal((int(cu_k[-1]), Hkv, d), dtype=np.float32)
    v = rng.standard_normal((int(cu_k[-1]), Hkv, d), dtype=np.float32)
    return PackedInputs(bf16_encode(q), bf16_encode(k), bf16_encode(v), cu_q, cu_k)


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """A packed causal batch of B sequences whose lengths are drawn uniform on
    [1, max_len] (query and key lengths equal), H query heads sharing Hkv
    key/value heads."""
    name: str
    B: int
    H: int
    Hkv: int
    max_len: int
    d: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def lengths(self) -> np.ndarray:
        rng = np.random.default_rng(self.seed)
        return rng.integers(1, self.max_len, size=self.B, endpoint=True, dtype=np.int64)

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "Hkv": self.Hkv,
                "max_len": self.max_len, "d": self.d, "dtype": "bf16", "causal": True,
                "scale": self.scale, "lengths": "uniform on [1, max_len], packed"}


VARLEN_WORKLOADS = {
    # 16 packed causal sequences of up to 8192 tokens, 32 query heads on 8 key/value heads
    "varlen_b16_h32_hkv8_n8192_d128_bf16": VarlenWorkload(
        "varlen_b16_h32_hkv8_n8192_d128_bf16", 16, 32, 8, 8192, 128, 1008),
}


def varlen_inputs(wl: VarlenWorkload) -> PackedInputs:
    """Lengths from the workload's seed, then the tensors from seed + 1."""
    lens = wl.lengths()
    return packed_inputs(lens, lens, wl.H, wl.Hkv, wl.d, wl.seed + 1)


# The backward exercise of "IO-aware exact attention" (section "Measure
# stored-state and recomputed attention backward"): batch 2, 16 heads,
# d = 64, lengths 512 .. 4096; the named workload is its longest length.
BWD_WORKLOADS = {
    "bwd_b2_h16_n4096_d64_bf16": Workload(
        "bwd_b2_h16_n4096_d64_bf16", 2, 16, 4096, 64, "bf16", False, 1.0 / 8.0, 1007),
}


def grad_inputs(B, H, N, d, seed, *, q_mult=1.0, key_len=None):
    """Inputs of a backward pass (same recipe, bf16): Q, K, V, then the
    upstream gradient dO, each [B, H, N, d] standard normal.  Returns the
    Inputs of Q, K, V and the bf16 bits of dO."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    kl = None if key_len is None else np.asarray(key_len, dtype=np.int32)
    wl = Workload(f"grad_b{B}_h{H}_n{N}_d{d}_bf16", B, H, N, d, "bf16", False,
                  1.0 / math.sqrt(d), seed, q_mult=q_mult)
    return Inputs(wl, bf16_encode(q), bf16_encode(k), bf16_encode(v), kl, None), bf16_encode(do)


def valid_pairs(N: int, causal: bool, key_len=None, B: int = 1) -> int:
    """Number of (query, key) pairs that take part, per head, summed over batch.

    A key j is visible to query i when j < L (L = N, or the sequence's key
    length clamped to [0, N]), i < L, and, for causal attention, j <= i.
    """
    lens = [N] * B if key_len is None else [max(0, min(int(x), N)) for x in key_len]
    total = 0
    for L in lens:
        total += L * (L + 1) // 2 if causal else L * L
    return total
