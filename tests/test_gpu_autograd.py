"""The autograd wrapper (bit_trainable_attention_amd.autograd) returns exactly what the C-ABI
calls return on the same inputs (it only marshals arguments), in both layouts, and through
them meets the quantised oracle's bar: O, dQ, dK, dV within rel-L2 2e-3, LSE within 1e-4."""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import quant as oq
from tests.harness import gpu_run, host_inputs, rel_l2, spec_for, to_device

pytestmark = pytest.mark.gpu
W = wl.WORKLOADS

CASES = [
    ("tiny", W["tiny"]),
    ("bf16_d64_causal", W["bf16_d64"].with_shape(B=1, H=2, N=512)),
    ("d128_causal", W["n8192_d128"].with_shape(B=1, H=2, N=384)),
    ("ragged", W["tiny"].with_shape(B=1, H=2, N=200)),
]


def _say(msg):
    print(msg, flush=True)


def _wrapper_run(w, x, layout, fmt="int8"):
    import torch
    from bit_trainable_attention_amd.autograd import sagebwd_attention
    q, k, v, dO = (to_device(x[n], w.dtype) for n in ("Q", "K", "V", "dO"))
    if layout == "bnhd":
        q, k, v, dO = (t.transpose(1, 2).contiguous() for t in (q, k, v, dO))
    q, k, v = (t.requires_grad_() for t in (q, k, v))
    O, lse = sagebwd_attention(q, k, v, causal=w.causal, qk_norm=w.qk_norm, k_smooth=w.k_smooth, blk=w.blk,
                               eps=w.eps, sm_scale=w.sm_scale, layout=layout, return_lse=True, fmt=fmt)
    O.backward(dO)
    torch.cuda.synchronize()
    out = {"O": O, "dQ": q.grad, "dK": k.grad, "dV": v.grad}
    if layout == "bnhd":
        out = {n: t.transpose(1, 2) for n, t in out.items()}
    res = {n: t.detach().float().cpu().numpy().astype(np.float64) for n, t in out.items()}
    assert tuple(lse.shape) == (w.B, w.H, w.N), tuple(lse.shape)
    res["LSE"] = lse.cpu().numpy()
    return res


@pytest.mark.parametrize("name,w", CASES)
def test_wrapper_equals_c_abi(name, w):
    _say(f"[autograd] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} causal={w.causal}")
    x = host_inputs(w)
    direct = gpu_run(w, x)
    for layout in ("bhnd", "bnhd"):
        _say(f"[autograd] {name}: wrapper, layout {layout}")
        got = _wrapper_run(w, x, layout)
        for n in ("O", "LSE", "dQ", "dK", "dV"):
            assert np.array_equal(got[n], direct[n]), (layout, n, float(np.max(np.abs(got[n] - direct[n]))))


def test_wrapper_fp8_equals_c_abi():
    """fmt="fp8" reaches the library through the wrapper: the same bits as the C ABI's FP8 run."""
    name, w = CASES[0]
    _say(f"[autograd] {name}: FP8 wrapper")
    x = host_inputs(w)
    direct = gpu_run(w, x, fmt="fp8")
    got = _wrapper_run(w, x, "bhnd", fmt="fp8")
    for n in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(got[n], direct[n]), (n, float(np.max(np.abs(got[n] - direct[n]))))


def test_wrapper_meets_oracle_bar():
    name, w = CASES[1]
    x = host_inputs(w)
    _say(f"[autograd] {name}: wrapper against the quantised oracle")
    got = _wrapper_run(w, x, "bhnd")
    o = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec_for(w))
    errs = {n: rel_l2(got[n], o[n]) for n in ("O", "dQ", "dK", "dV")}
    lse = float(np.max(np.abs(got["LSE"].astype(np.float64) - o["LSE"])))
    _say(f"[autograd] {name}: rel-L2 {errs}, max|dLSE| {lse:.2e}")
    assert lse < 1e-4 * max(1.0, float(np.max(np.abs(o["LSE"]))))
    for n, e in errs.items():
        assert e <= 2e-3, (n, e)


def test_no_second_derivative():
    """The backward runs in the library, so it has no derivative of its own: asking for one
    (create_graph, then differentiating the gradients) raises instead of returning zeros."""
    import torch
    from bit_trainable_attention_amd.autograd import sagebwd_attention
    w = wl.WORKLOADS["tiny"].with_shape(N=128)
    x = host_inputs(w)
    q, k, v = (to_device(x[n], w.dtype).requires_grad_() for n in ("Q", "K", "V"))
    _say("[autograd] second derivative request")
    o = sagebwd_attention(q, k, v, causal=w.causal, qk_norm=w.qk_norm, k_smooth=w.k_smooth, blk=w.blk, eps=w.eps)
    (gq,) = torch.autograd.grad(o.float().sum(), q, create_graph=True)
    with pytest.raises(RuntimeError):
        gq.float().sum().backward()
