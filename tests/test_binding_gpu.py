"""The Python binding rejects caller-supplied outputs and workspaces of the
wrong shape, dtype, device placement or layout with FAError before anything
is enqueued: the C ABI takes plain pointers and cannot check buffer sizes,
so a too-small output would otherwise be written out of bounds.  Each case
checks that an output prefilled with a sentinel is left untouched."""
import pytest

import io_aware_exact_forward_amd as fa

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def tensors(B=1, H=2, N=64, d=64):
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(3)
    mk = lambda: torch.randn(B, H, N, d, device=dev, dtype=torch.bfloat16, generator=g)
    return mk(), mk(), mk()


def bad_outputs(shape, dtype):
    import torch
    dev = torch.device("cuda:0")
    wrong_shape = list(shape)
    wrong_shape[-1] -= 1
    other = torch.float32 if dtype == torch.bfloat16 else torch.bfloat16
    strided = torch.empty(list(shape[:-1]) + [2 * shape[-1]], dtype=dtype, device=dev)[..., ::2]
    return {"shape": torch.empty(wrong_shape, dtype=dtype, device=dev),
            "dtype": torch.empty(shape, dtype=other, device=dev),
            "host": torch.empty(shape, dtype=dtype),
            "strided": strided}


@pytest.mark.parametrize("which", ["shape", "dtype", "host", "strided"])
def test_forward_rejects_bad_out_and_lse(which):
    import torch
    q, k, v = tensors()
    say(f"forward bad out/lse: {which}")
    sentinel = torch.full((1, 2, 64), 7.0, device="cuda:0")
    with pytest.raises(fa.FAError):
        fa.forward(q, k, v, out=bad_outputs(q.shape, q.dtype)[which], lse=sentinel)
    with pytest.raises(fa.FAError):
        fa.forward(q, k, v, lse=bad_outputs((1, 2, 64), torch.float32)[which])
    with pytest.raises(fa.FAError):
        fa.forward_dropout(q, k, v, p_drop=0.1, seed=1, out=bad_outputs(q.shape, q.dtype)[which],
                           lse=sentinel)
    with pytest.raises(fa.FAError):
        fa.forward_split(q, k, v, out=bad_outputs(q.shape, q.dtype)[which], lse=sentinel)
    bias = torch.zeros(1, 1, 64, 64, device="cuda:0")
    with pytest.raises(fa.FAError):
        fa.forward_bias(q, k, v, bias, out=bad_outputs(q.shape, q.dtype)[which], lse=sentinel)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


@pytest.mark.parametrize("which", ["shape", "dtype", "host", "strided"])
def test_backward_rejects_bad_gradients(which):
    import torch
    q, k, v = tensors()
    o, lse = fa.forward(q, k, v)
    dout = torch.ones_like(q)
    torch.cuda.synchronize()
    say(f"backward bad dq/dk/dv: {which}")
    sentinel = torch.full_like(q, 7.0)
    for name in ("dq", "dk", "dv"):
        grads = {"dq": sentinel, "dk": torch.empty_like(k), "dv": torch.empty_like(v)}
        if name == "dq":
            grads = {"dq": bad_outputs(q.shape, q.dtype)[which], "dk": sentinel,
                     "dv": torch.empty_like(v)}
        else:
            grads[name] = bad_outputs(q.shape, q.dtype)[which]
        with pytest.raises(fa.FAError):
            fa.backward(q, k, v, o, lse, dout, **grads)
        with pytest.raises(fa.FAError):
            fa.backward_gqa(q, k, v, o, lse, dout, **grads)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


def test_varlen_rejects_bad_out():
    import torch
    dev = torch.device("cuda:0")
    T, H, d = 100, 2, 64
    g = torch.Generator(device=dev).manual_seed(4)
    q, k, v = (torch.randn(T, H, d, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(3))
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device=dev)
    sentinel = torch.full((T, H), 7.0, device=dev)
    for which, bad in bad_outputs(q.shape, q.dtype).items():
        say(f"varlen bad out: {which}")
        with pytest.raises(fa.FAError):
            fa.forward_varlen(q, k, v, cu, cu, 60, 60, out=bad, lse=sentinel)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())


def test_bad_workspace_is_rejected():
    import torch
    q, k, v = tensors()
    sentinel = torch.full((1, 2, 64), 7.0, device="cuda:0")
    with pytest.raises(fa.FAError):
        fa.forward_split(q, k, v, num_splits=2, workspace=torch.empty(1 << 20, dtype=torch.uint8),
                         lse=sentinel)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())
