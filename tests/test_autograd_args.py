"""The autograd wrapper's argument checks, on the CPU: each bad argument is refused with a clear
error before anything reaches the library or a GPU (host tensors are refused by the binding's
own checks, which run before any HIP call)."""
import pytest
import torch

from bit_trainable_attention_amd.autograd import sagebwd_attention


def _qkv(shape=(1, 2, 128, 64), dtype=torch.float16):
    return tuple(torch.zeros(shape, dtype=dtype, requires_grad=True) for _ in range(3))


@pytest.mark.parametrize("kw,err", [
    (dict(fmt="int4"), "fmt"),
    (dict(split="fp4"), "split"),
    (dict(layout="nhd"), "layout"),
])
def test_bad_option_strings(kw, err):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match=err):
        sagebwd_attention(q, k, v, **kw)


def test_float32_inputs_refused():
    q, k, v = _qkv(dtype=torch.float32)
    with pytest.raises(TypeError, match="float16 or bfloat16"):
        sagebwd_attention(q, k, v)


def test_three_dimensional_inputs_refused():
    q, k, v = _qkv(shape=(2, 128, 64))
    with pytest.raises(ValueError, match="4-d"):
        sagebwd_attention(q, k, v)


def test_gains_go_together():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="together"):
        sagebwd_attention(q, k, v, q_gain=torch.ones(2, 64))


def test_host_tensors_refused_by_the_binding():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="device tensors"):
        sagebwd_attention(q, k, v)
