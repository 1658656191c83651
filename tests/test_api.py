"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before any HIP call.

None of these calls launches work: every argument set below fails host
validation (or is empty), so they run on a machine without a GPU.
"""
import os
import re

import pytest

import io_aware_exact_forward_amd as fa
from io_aware_exact_forward_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")

OK, NULL, SHAPE, HEAD_DIM, DTYPE, ALIGN, SCALE, ALIAS, WORKSPACE, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
BF16, F32 = fa.FA_DTYPE_BF16, fa.FA_DTYPE_F32

# Fake, aligned, non-overlapping "device" addresses: never dereferenced,
# because every call below fails validation first.
A = 1 << 40
Q, K, V, O, L, KL, WS = (A + i * (1 << 34) for i in range(7))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(
        ["fa_forward", "fa_naive_workspace_bytes", "fa_naive_forward", "fa_split_workspace_bytes",
         "fa_forward_split", "fa_forward_varlen", "fa_forward_dropout", "fa_forward_bias",
         "fa_backward_workspace_bytes", "fa_backward", "fa_backward_gqa", "fa_backward_varlen",
         "fa_backward_dropout", "fa_backward_bias",
         "fa_naive_backward", "fa_forward_split_noalloc",
         "fa_status_string", "fa_abi_version"])


def test_library_loads_and_exports_every_declared_symbol():
    lib = fa.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(_lib.exported_symbols()) == set(declared_functions())
    assert fa.fa_abi_version() == (1 << 16) | 10


def test_status_strings():
    for st in (OK, NULL, SHAPE, HEAD_DIM, DTYPE, ALIGN, SCALE, ALIAS, WORKSPACE, HIP):
        s = fa.fa_status_string(st)
        assert isinstance(s, str) and s
    assert fa.fa_status_string(12345) == "unknown status"


def call(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=64, d=64, scale=0.125, causal=0, kl=0,
         dtype=BF16, stream=0):
    return fa.fa_forward(q, k, v, o, lse, B, H, N, d, scale, causal, kl, dtype, stream)


def test_bad_dtype_and_head_dim():
    assert call(dtype=2) == DTYPE
    assert call(dtype=-1) == DTYPE
    for d in (0, 32, 96, 256, -64):
        assert call(d=d) == HEAD_DIM
        assert call(d=d, dtype=F32) == HEAD_DIM


def test_bad_shapes():
    assert call(B=-1) == SHAPE
    assert call(H=-1) == SHAPE
    assert call(N=-5) == SHAPE
    # B*H*N*d beyond 2^62 elements
    assert call(B=2 ** 31 - 1, H=2 ** 31 - 1, N=2 ** 31 - 1) == SHAPE


def test_bad_scale():
    for s in (float("nan"), float("inf"), -float("inf"), 3e38):
        assert call(scale=s) == SCALE


def test_empty_problem_is_a_no_op():
    # nothing to do: returns OK without touching the (NULL) pointers
    for B, H, N in ((0, 2, 64), (1, 0, 64), (1, 2, 0)):
        assert call(q=0, k=0, v=0, o=0, lse=0, B=B, H=H, N=N) == OK
        assert fa.fa_naive_forward(0, 0, 0, 0, 0, B, H, N, 64, 1.0, 0, 0, BF16, 0, 0, 0) == OK


def test_null_pointers():
    for field in ("q", "k", "v", "o", "lse"):
        assert call(**{field: 0}) == NULL


def test_misaligned_pointers():
    for field in ("q", "k", "v", "o"):
        assert call(**{field: locals_default(field) + 8}) == ALIGN
    assert call(lse=L + 2) == ALIGN
    assert call(kl=KL + 1) == ALIGN


def locals_default(field):
    return {"q": Q, "k": K, "v": V, "o": O, "lse": L}[field]


def test_aliasing_outputs():
    assert call(o=Q) == ALIAS
    assert call(o=V + 64) == ALIAS          # partial overlap
    assert call(lse=K) == ALIAS
    assert call(lse=O + 1024) == ALIAS
    assert call(kl=O + 16) == ALIAS
    # inputs may alias each other (self-attention on one buffer)
    # -> validation passes; not called here because it would launch


def test_naive_workspace_size():
    # S and P, B*H*N*N each, in the input dtype
    assert fa.fa_naive_workspace_bytes(1, 32, 8192, BF16) == 2 * 32 * 8192 * 8192 * 2
    assert fa.fa_naive_workspace_bytes(1, 1, 3, F32) == 2 * 256
    assert fa.fa_naive_workspace_bytes(1, 1, 3, 7) == 0
    assert fa.fa_naive_workspace_bytes(-1, 1, 3, BF16) == 0


def test_naive_workspace_errors():
    need = fa.fa_naive_workspace_bytes(1, 2, 64, BF16)
    args = (Q, K, V, O, L, 1, 2, 64, 64, 0.125, 0, 0, BF16)
    assert fa.fa_naive_forward(*args, 0, need, 0) == WORKSPACE
    assert fa.fa_naive_forward(*args, WS, need - 1, 0) == WORKSPACE
    assert fa.fa_naive_forward(*args, WS + 16, need, 0) == WORKSPACE
    assert fa.fa_naive_forward(*args, Q, need, 0) == ALIAS


def test_python_wrapper_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FAError):
        fa.forward(x, x, x)


# ---- split-KV entry point -------------------------------------------------------

def split_call(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Hkv=2, Nq=64, Nk=1024, d=64, scale=0.125,
               causal=0, kl=0, dtype=BF16, num_splits=4, ws=WS, wsb=1 << 30, stream=0):
    return fa.fa_forward_split(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, kl, dtype,
                               num_splits, ws, wsb, stream)


def test_split_workspace_size():
    # fp32 partial outputs [ranges, B*H*Nq, d] then their LSE [ranges, B*H*Nq],
    # each rounded up to 256 bytes; ranges are whole 128-key blocks
    assert fa.fa_split_workspace_bytes(1, 2, 64, 1024, 64, 4) == 4 * 128 * 64 * 4 + 4 * 128 * 4
    # one range: no workspace
    assert fa.fa_split_workspace_bytes(1, 2, 64, 1024, 64, 1) == 0
    # automatic: 2 query tiles -> as many ranges as 128-key blocks (8)
    assert fa.fa_split_workspace_bytes(1, 2, 64, 1024, 64, 0) == 8 * 128 * 64 * 4 + 8 * 128 * 4
    # more ranges asked than blocks: one block per range
    assert fa.fa_split_workspace_bytes(1, 2, 64, 1024, 64, 100) == 8 * 128 * 64 * 4 + 8 * 128 * 4
    # 8 blocks in 3 ranges of 3, 3, 2 blocks; d = 128; one decode row per head
    assert fa.fa_split_workspace_bytes(2, 3, 1, 1000, 128, 3) == 3 * 6 * 128 * 4 + 256
    # a decode step (one query row, as many key/value heads as query heads)
    # with the automatic count: P = min(512, B*H*ceil(Nk/64)) balanced shares,
    # partials in 4 (P + B*H) slots (one per wave of a share and row), then
    # the unit prefix cum [B + 1] (int64)
    r256 = lambda x: (x + 255) // 256 * 256
    for B, H, Nk, d in ((2, 3, 1000, 128), (8, 32, 16384, 128), (130, 2, 700, 64)):
        P = min(512, B * H * -(-Nk // 64))
        slots = 4 * (P + B * H)
        bal = r256(slots * d * 4) + r256(slots * 4) + r256((B + 1) * 8)
        # (the size covers every Hkv dividing H, so grouped heads may need more)
        assert fa.fa_split_workspace_bytes(B, H, 1, Nk, d, 0) >= bal, (B, H, Nk, d)
        if (B, H) == (2, 3):  # Hkv = 1 needs 8 ranges x 6 rows here: less
            assert fa.fa_split_workspace_bytes(B, H, 1, Nk, d, 0) == bal
    # many query tiles: the automatic choice stays at one range
    assert fa.fa_split_workspace_bytes(1, 32, 8192, 8192, 128, 0) == 0
    # no keys, empty problems and invalid arguments: 0
    assert fa.fa_split_workspace_bytes(1, 2, 64, 0, 64, 4) == 0
    assert fa.fa_split_workspace_bytes(0, 2, 64, 1024, 64, 4) == 0
    assert fa.fa_split_workspace_bytes(-1, 2, 64, 1024, 64, 4) == 0
    assert fa.fa_split_workspace_bytes(1, 2, 64, 1024, 96, 4) == 0
    assert fa.fa_split_workspace_bytes(1, 2, 64, 1024, 64, -1) == 0
    assert fa.fa_split_workspace_bytes(1, 2, 64, 1024, 64, 65537) == 0


def test_split_bad_arguments():
    assert split_call(dtype=F32) == DTYPE
    assert split_call(dtype=3) == DTYPE
    assert split_call(d=96) == HEAD_DIM
    for bad in (dict(B=-1), dict(H=-1), dict(Nq=-1), dict(Nk=-1), dict(num_splits=-1),
                dict(num_splits=65537), dict(Hkv=0), dict(Hkv=3), dict(H=6, Hkv=4)):
        assert split_call(**bad) == SHAPE, bad
    # one (batch, head) slice above 2^31 - 1 bytes
    assert split_call(Nq=1 << 24, d=128) == SHAPE
    assert split_call(Nk=1 << 24, d=128) == SHAPE
    for s in (float("nan"), float("inf"), 3e38):
        assert split_call(scale=s) == SCALE


def test_split_empty_is_a_no_op():
    for B, H, Nq in ((0, 2, 64), (1, 0, 64), (1, 2, 0)):
        assert split_call(q=0, k=0, v=0, o=0, lse=0, B=B, H=H, Nq=Nq, ws=0, wsb=0) == OK


def test_split_pointer_checks():
    for field in ("q", "k", "v", "o", "lse"):
        assert split_call(**{field: 0}) == NULL
    for field, val in (("q", Q + 8), ("k", K + 8), ("v", V + 8), ("o", O + 8), ("lse", L + 2),
                       ("kl", KL + 1)):
        assert split_call(**{field: val}) == ALIGN, field
    assert split_call(o=Q) == ALIAS
    assert split_call(lse=V + 4) == ALIAS
    assert split_call(o=L) == ALIAS


def test_split_workspace_errors():
    need = fa.fa_split_workspace_bytes(1, 2, 64, 1024, 64, 4)
    assert need > 0
    assert split_call(ws=0, wsb=need) == WORKSPACE
    assert split_call(wsb=need - 1) == WORKSPACE
    assert split_call(ws=WS + 16, wsb=need) == WORKSPACE   # 256-byte alignment
    assert split_call(ws=Q, wsb=need) == ALIAS
    assert split_call(ws=O - 256, wsb=need) == ALIAS          # tail overlaps the output
    assert split_call(ws=KL, wsb=need, kl=KL + need - 4) == ALIAS


def test_python_split_wrapper_rejects_bad_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FAError):
        fa.forward_split(x, x, x)
    y = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FAError):
        fa.forward_split(x, y, y)   # heads differ


# ---- backward entry point -------------------------------------------------------

DQ, DK, DV, DO, OO = (A + (7 + i) * (1 << 34) for i in range(5))


def bwd_call(q=Q, k=K, v=V, o=OO, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, B=1, H=2, N=64, d=64,
             scale=0.125, causal=0, kl=0, dtype=BF16, ws=WS, wsb=1 << 20, stream=0):
    return fa.fa_backward(q, k, v, o, lse, do, dq, dk, dv, B, H, N, d, scale, causal, kl, dtype,
                          ws, wsb, stream)


def test_backward_workspace_size():
    # fp32 D per row, rounded up to 256 bytes
    assert fa.fa_backward_workspace_bytes(2, 16, 4096, 64, BF16) == 2 * 16 * 4096 * 4
    assert fa.fa_backward_workspace_bytes(1, 1, 3, 64, BF16) == 256
    assert fa.fa_backward_workspace_bytes(1, 1, 3, 64, F32) == 0
    assert fa.fa_backward_workspace_bytes(1, 1, 3, 128, BF16) == 256
    assert fa.fa_backward_workspace_bytes(1, 1, 3, 96, BF16) == 0
    assert fa.fa_backward_workspace_bytes(0, 1, 3, 64, BF16) == 0


def test_backward_bad_arguments():
    assert bwd_call(dtype=F32) == DTYPE
    assert bwd_call(d=96) == HEAD_DIM
    assert bwd_call(d=32) == HEAD_DIM
    assert bwd_call(N=-1) == SHAPE
    assert bwd_call(scale=float("nan")) == SCALE
    for field in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert bwd_call(**{field: 0}) == NULL, field
    for field, val in (("q", Q + 8), ("dk", DK + 8), ("do", DO + 2), ("lse", L + 2)):
        assert bwd_call(**{field: val}) == ALIGN, field
    assert bwd_call(ws=0) == WORKSPACE
    assert bwd_call(wsb=64) == WORKSPACE
    assert bwd_call(ws=WS + 16) == WORKSPACE
    assert bwd_call(dq=Q) == ALIAS
    assert bwd_call(dk=DQ + 64) == ALIAS
    assert bwd_call(dv=OO) == ALIAS
    assert bwd_call(ws=DO) == ALIAS
    assert bwd_call(ws=DV) == ALIAS


def test_backward_empty_is_a_no_op():
    for B, H, N in ((0, 2, 64), (1, 0, 64), (1, 2, 0)):
        assert bwd_call(q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, ws=0, wsb=0,
                        B=B, H=H, N=N) == OK


def test_backward_dropout_bad_arguments():
    def bd(**kw):
        a = dict(q=Q, k=K, v=V, o=OO, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, B=1, H=2, N=64, d=64,
                 scale=0.125, causal=0, kl=0, dtype=BF16, p=0.1, seed=5, offset=0, ws=WS,
                 wsb=1 << 20)
        a.update(kw)
        return fa.fa_backward_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                      a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"],
                                      a["scale"], a["causal"], a["kl"], a["dtype"], a["p"],
                                      a["seed"], a["offset"], a["ws"], a["wsb"], 0)
    assert bd(dtype=F32) == DTYPE
    for bad in (-0.1, 1.0, 1.5, float("nan")):
        assert bd(p=bad) == SCALE, bad
    assert bd(d=96) == HEAD_DIM
    assert bd(dq=0) == NULL
    assert bd(dk=DK + 8) == ALIGN
    assert bd(ws=0) == WORKSPACE
    assert bd(dv=Q) == ALIAS
    assert bd(B=0, q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, ws=0, wsb=0) == OK


def test_backward_bias_bad_arguments():
    BI = A + 14 * (1 << 34)

    def bb(**kw):
        a = dict(q=Q, k=K, v=V, o=OO, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, bias=BI, B=2, H=2, N=64,
                 d=64, scale=0.125, causal=0, kl=0, dtype=BF16, sb=2 * 64 * 64, sh=64 * 64, ld=64,
                 ws=WS, wsb=1 << 20)
        a.update(kw)
        return fa.fa_backward_bias(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                   a["dk"], a["dv"], a["bias"], a["B"], a["H"], a["N"], a["d"],
                                   a["scale"], a["causal"], a["kl"], a["dtype"], a["sb"], a["sh"],
                                   a["ld"], a["ws"], a["wsb"], 0)
    assert bb(dtype=F32) == DTYPE
    assert bb(d=96) == HEAD_DIM
    for bad in (dict(ld=60), dict(ld=66), dict(sb=-4), dict(sh=6)):
        assert bb(**bad) == SHAPE, bad
    assert bb(bias=0) == NULL
    assert bb(bias=BI + 8) == ALIGN
    assert bb(dq=BI + 1024) == ALIAS           # an output over the mask
    assert bb(ws=BI) == ALIAS
    assert bb(ws=0) == WORKSPACE
    assert bb(B=0, q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, bias=0, ws=0, wsb=0) == OK


def gqa_call(q=Q, k=K, v=V, o=OO, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, B=2, H=8, Hkv=2, Nq=64,
             Nk=100, d=64, scale=0.125, causal=1, kl=0, dtype=BF16, ws=WS, wsb=1 << 20, stream=0):
    return fa.fa_backward_gqa(q, k, v, o, lse, do, dq, dk, dv, B, H, Hkv, Nq, Nk, d, scale, causal,
                              kl, dtype, ws, wsb, stream)


def test_backward_gqa_bad_arguments():
    assert gqa_call(dtype=F32) == DTYPE
    assert gqa_call(d=96) == HEAD_DIM
    for bad in (dict(B=-1), dict(Nq=-1), dict(Nk=-1), dict(H=-2), dict(Hkv=0), dict(Hkv=3),
                dict(Nq=1 << 24, d=128)):
        assert gqa_call(**bad) == SHAPE, bad
    assert gqa_call(scale=float("nan")) == SCALE
    for field in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert gqa_call(**{field: 0}) == NULL, field
    for field, val in (("q", Q + 8), ("dv", DV + 8), ("lse", L + 2), ("kl", KL + 2)):
        assert gqa_call(**{field: val}) == ALIGN, field
    assert gqa_call(ws=0) == WORKSPACE
    assert gqa_call(wsb=2 * 8 * 64 * 4 - 4) == WORKSPACE
    assert gqa_call(ws=WS + 64) == WORKSPACE
    assert gqa_call(dq=OO) == ALIAS
    assert gqa_call(dk=DV - 1024) == ALIAS          # dk runs into dv
    assert gqa_call(ws=L) == ALIAS
    assert gqa_call(dv=KL - 64, kl=KL) == ALIAS      # dv runs into the lengths


def test_backward_gqa_batch_zero_is_a_no_op():
    assert gqa_call(q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, ws=0, wsb=0, B=0) == OK


def bvl_call(q=Q, k=K, v=V, o=OO, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, cuq=A + 12 * (1 << 34),
             cuk=A + 13 * (1 << 34), B=3, H=4, Hkv=2, tq=100, tk=120, mq=50, mk=60, d=64,
             scale=0.125, causal=1, dtype=BF16, ws=WS, wsb=1 << 20, stream=0):
    return fa.fa_backward_varlen(q, k, v, o, lse, do, dq, dk, dv, cuq, cuk, B, H, Hkv, tq, tk, mq,
                                 mk, d, scale, causal, dtype, ws, wsb, stream)


def test_backward_varlen_bad_arguments():
    assert bvl_call(dtype=F32) == DTYPE
    assert bvl_call(d=32) == HEAD_DIM
    for bad in (dict(B=-1), dict(tq=-1), dict(tk=-1), dict(mq=-1), dict(Hkv=0), dict(Hkv=3),
                dict(mk=1 << 24, d=128)):
        assert bvl_call(**bad) == SHAPE, bad
    assert bvl_call(scale=float("inf")) == SCALE
    for field in ("q", "k", "o", "lse", "do", "dq", "dk", "cuq", "cuk"):
        assert bvl_call(**{field: 0}) == NULL, field
    for field, val in (("q", Q + 8), ("dq", DQ + 4), ("lse", L + 2), ("cuk", A + 13 * (1 << 34) + 2)):
        assert bvl_call(**{field: val}) == ALIGN, field
    assert bvl_call(ws=0) == WORKSPACE
    assert bvl_call(wsb=100 * 4 * 4 - 4) == WORKSPACE
    assert bvl_call(dq=Q) == ALIAS
    assert bvl_call(ws=A + 12 * (1 << 34)) == ALIAS   # workspace over the offsets
    assert bvl_call(dv=DK + 64) == ALIAS


def test_backward_varlen_batch_zero_is_a_no_op():
    assert bvl_call(q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, cuq=0, cuk=0, ws=0, wsb=0,
                    B=0) == OK


def test_naive_backward_bad_arguments():
    def nb(**kw):
        a = dict(q=Q, k=K, v=V, o=OO, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, B=1, H=2, N=64, d=64,
                 scale=0.125, causal=0, kl=0, dtype=BF16, ws=WS,
                 wsb=fa.fa_naive_workspace_bytes(1, 2, 64, BF16), stream=0)
        a.update(kw)
        return fa.fa_naive_backward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                    a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                                    a["causal"], a["kl"], a["dtype"], a["ws"], a["wsb"], a["stream"])
    assert nb(dtype=F32) == DTYPE
    assert nb(d=96) == HEAD_DIM
    assert nb(dq=0) == NULL
    assert nb(dk=DK + 4) == ALIGN
    assert nb(ws=0) == WORKSPACE
    assert nb(wsb=100) == WORKSPACE
    assert nb(dv=K) == ALIAS
    assert nb(B=0, q=0, k=0, v=0, o=0, lse=0, do=0, dq=0, dk=0, dv=0, ws=0, wsb=0) == OK



# ---- packed variable-length entry point -------------------------------------

CUQ, CUK = A + 12 * (1 << 34), A + 13 * (1 << 34)


def varlen_call(q=Q, k=K, v=V, o=O, lse=L, cuq=CUQ, cuk=CUK, B=3, H=4, Hkv=2, tq=100, tk=120,
                mq=50, mk=60, d=64, scale=0.125, causal=1, dtype=BF16, stream=0):
    return fa.fa_forward_varlen(q, k, v, o, lse, cuq, cuk, B, H, Hkv, tq, tk, mq, mk, d, scale,
                                causal, dtype, stream)


def test_varlen_bad_arguments():
    assert varlen_call(dtype=F32) == DTYPE
    assert varlen_call(d=32) == HEAD_DIM
    for bad in (dict(B=-1), dict(tq=-1), dict(mk=-1), dict(Hkv=0), dict(Hkv=3),
                dict(mq=1 << 24, d=128)):
        assert varlen_call(**bad) == SHAPE, bad
    assert varlen_call(scale=float("inf")) == SCALE
    for field in ("q", "o", "lse", "cuq", "cuk", "k", "v"):
        assert varlen_call(**{field: 0}) == NULL, field
    for field, val in (("q", Q + 8), ("o", O + 4), ("lse", L + 2), ("cuq", CUQ + 2)):
        assert varlen_call(**{field: val}) == ALIGN, field
    assert varlen_call(o=Q) == ALIAS
    assert varlen_call(lse=CUK) == ALIAS
    assert varlen_call(o=L - 1024) == ALIAS


def test_varlen_empty_is_a_no_op():
    for kw in (dict(B=0), dict(H=0), dict(tq=0), dict(mq=0)):
        assert varlen_call(q=0, k=0, v=0, o=0, lse=0, cuq=0, cuk=0, **kw) == OK



def test_dropout_bad_arguments():
    def dc(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=64, d=64, scale=0.125, causal=0, kl=0,
                 dtype=BF16, p=0.1, seed=1, offset=0)
        a.update(kw)
        return fa.fa_forward_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                     a["N"], a["d"], a["scale"], a["causal"], a["kl"], a["dtype"],
                                     a["p"], a["seed"], a["offset"], 0)
    assert dc(dtype=F32) == DTYPE
    for bad in (-0.1, 1.0, 1.5, float("nan")):
        assert dc(p=bad) == SCALE, bad
    assert dc(d=96) == HEAD_DIM
    assert dc(o=0) == NULL
    assert dc(o=Q) == ALIAS
    assert dc(B=0, q=0, k=0, v=0, o=0, lse=0) == OK
    assert dc(seed=2 ** 64 - 1, o=0) == NULL   # the full 64-bit seed range passes marshalling



BI = A + 20 * (1 << 34)


def test_bias_bad_arguments():
    def bc(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, bias=BI, B=2, H=2, N=64, d=64, scale=0.125, causal=0,
                 kl=0, dtype=BF16, sb=2 * 64 * 64, sh=64 * 64, ld=64)
        a.update(kw)
        return fa.fa_forward_bias(a["q"], a["k"], a["v"], a["o"], a["lse"], a["bias"], a["B"],
                                  a["H"], a["N"], a["d"], a["scale"], a["causal"], a["kl"],
                                  a["dtype"], a["sb"], a["sh"], a["ld"], 0)
    assert bc(dtype=F32) == DTYPE
    for bad in (dict(ld=60), dict(ld=66), dict(sb=-4), dict(sh=2), dict(sb=6)):
        assert bc(**bad) == SHAPE, bad
    assert bc(bias=0) == NULL
    assert bc(bias=BI + 4) == ALIGN
    assert bc(o=BI) == ALIAS
    assert bc(lse=BI + 2 * 64 * 64 * 4) == ALIAS
    assert bc(B=0, q=0, k=0, v=0, o=0, lse=0, bias=0) == OK


def test_output_validation_helper():
    """Caller-supplied outputs are checked for shape, dtype, device and
    contiguity before any launch (the C ABI cannot see buffer sizes)."""
    import torch
    from io_aware_exact_forward_amd import _output, _workspace
    dev = torch.device("cuda:0")
    good_shape = (1, 2, 4, 64)
    with pytest.raises(fa.FAError):     # wrong shape
        _output(torch.zeros(1, 2, 3, 64, dtype=torch.bfloat16), good_shape, torch.bfloat16, dev, "out")
    with pytest.raises(fa.FAError):     # wrong dtype
        _output(torch.zeros(good_shape, dtype=torch.float32), good_shape, torch.bfloat16, dev, "out")
    with pytest.raises(fa.FAError):     # host memory
        _output(torch.zeros(good_shape, dtype=torch.bfloat16), good_shape, torch.bfloat16, dev, "out")
    with pytest.raises(fa.FAError):     # host workspace
        _workspace(torch.zeros(16, dtype=torch.uint8), 16, dev)


def test_split_noalloc_validates_before_any_hip_call():
    """The allocation-free split entry point refuses bad arguments, and
    problems whose partial results exceed its scratch, before touching the
    device (these calls run without a GPU)."""
    call = lambda **kw: fa.fa_forward_split_noalloc(*_noalloc_args(**kw))
    assert call(q=0) == NULL
    assert call(d=96) == HEAD_DIM
    assert call(dtype=F32) == DTYPE
    assert call(o=Q) == ALIAS
    assert call(q=Q + 2) == ALIGN
    # 8 heads x 1024 rows x 64 ranges of fp32 partials: 269 MB > 32 MiB
    assert call(H=8, Nq=1024, Nk=8192, d=128, num_splits=64) == WORKSPACE
    assert call(B=0) == OK


def _noalloc_args(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Hkv=2, Nq=64, Nk=1024, d=64, scale=0.125,
                  causal=0, kl=0, dtype=BF16, num_splits=4, stream=0):
    return (q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, kl, dtype, num_splits, stream)


def test_probe_library_exports_and_rejects_bad_arguments():
    """The matrix-core rate probe bench.py reports beside the roofline is a
    separate library (not part of the attention ABI); bad arguments return -1
    before any HIP call."""
    import ctypes

    from io_aware_exact_forward_amd import build as _b

    path = _b.probe_lib_path()
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(path)
    lib.fa_probe_mfma_bf16.restype = ctypes.c_int
    lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_mfma_flops.restype = ctypes.c_double
    lib.fa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    assert lib.fa_probe_mfma_bf16(0, 10, ctypes.c_void_p(A), None) == -1
    assert lib.fa_probe_mfma_bf16(4, 0, ctypes.c_void_p(A), None) == -1
    assert lib.fa_probe_mfma_bf16(4, 10, None, None) == -1
    # 8 waves x 16 MFMAs per iteration x 32768 flops each
    assert lib.fa_probe_mfma_flops(2, 3) == 2 * 3 * 8 * 16 * 2 * 32 * 32 * 16
