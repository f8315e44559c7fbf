"""The three calls run on the stream they are given (the header: every call enqueues on its
stream argument and returns without waiting).

The inputs are written on a side stream behind a queue of unrelated work (a chain of matrix
products), and the prologue, forward and backward are then called on that stream: the
prologue through the current-stream default, the backward with the stream passed explicitly.
A call that ran on any other stream would read its inputs before the copies that fill them
(PyTorch's side streams do not wait for the null stream), so every output must equal a plain
run on the default stream bit for bit."""
import pytest

from bit_trainable_attention_amd import workloads as wl
from tests.harness import host_inputs, params_for, to_device

pytestmark = pytest.mark.gpu


def _calls(api, p, Q, K, V, dO, stream=None):
    pro = api.sagebwd_quant_prologue(p, Q, K, V)
    O, lse = api.sagebwd_forward(p, pro, V=V)
    g = api.sagebwd_backward(p, Q, K, V, pro, O, lse, dO, stream=stream)
    return dict(O=O, lse=lse, dQ=g["dQ"], dK=g["dK"], dV=g["dV"], Qc=pro["Qc"], Kc=pro["Kc"], Vtc=pro["Vtc"])


def test_calls_follow_the_callers_stream():
    import torch
    from bit_trainable_attention_amd import api
    w = wl.WORKLOADS["n8192_d128"].with_shape(B=1, H=4, N=1024)
    x = host_inputs(w)
    p = params_for(w)
    src = {k: to_device(x[k], w.dtype) for k in ("Q", "K", "V", "dO")}
    torch.cuda.synchronize()
    print("[stream] reference run on the default stream", flush=True)
    ref = _calls(api, p, src["Q"], src["K"], src["V"], src["dO"])
    torch.cuda.synchronize()

    side = torch.cuda.Stream()          # default priority
    print("[stream] queued work, input copies and the three calls on a side stream", flush=True)
    with torch.cuda.stream(side):
        m = torch.randn(4096, 4096, device="cuda:0") / 64.0
        for _ in range(16):            # a few milliseconds of unrelated work ahead of the copies
            m = torch.tanh(m @ m)
        ins = {k: torch.empty_like(t) for k, t in src.items()}
        for k in ins:
            ins[k].copy_(src[k])
        got = _calls(api, p, ins["Q"], ins["K"], ins["V"], ins["dO"], stream=side)
    side.synchronize()
    for k, t in ref.items():
        assert torch.equal(got[k], t), k
    assert bool(torch.isfinite(m).all())


def test_two_problems_at_once_on_two_streams():
    """Two different problems (shapes, masks, layouts, dQ modes) enqueued alternately on two
    streams run concurrently; the library keeps no state between calls, so each must equal its
    own run on the default stream bit for bit (dQ of the float32-atomic mode: within rel-L2 1e-4,
    since the order in which the atomics land varies and only that float32 rounding moves)."""
    import torch
    from bit_trainable_attention_amd import api
    cases = [(wl.WORKLOADS["n8192_d128"].with_shape(B=1, H=4, N=1024), dict(dq_mode=1)),
             (wl.WORKLOADS["bf16_d64"].with_shape(B=2, H=2, N=700, causal=False), dict(dq_mode=2, layout="bnhd"))]
    prepared = []
    for w, kw in cases:
        x = host_inputs(w)
        tr = (lambda t: t.transpose(1, 2).contiguous()) if kw.get("layout") == "bnhd" else (lambda t: t)
        t = {k: tr(to_device(x[k], w.dtype)) for k in ("Q", "K", "V", "dO")}
        prepared.append((params_for(w, **kw), t))
    torch.cuda.synchronize()
    print("[stream] two problems: references on the default stream", flush=True)
    refs = [_calls(api, p, t["Q"], t["K"], t["V"], t["dO"]) for p, t in prepared]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    print("[stream] two problems: four rounds on two streams at once", flush=True)
    for _ in range(4):
        got = [None, None]
        for i, ((p, t), s) in enumerate(zip(prepared, streams)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                got[i] = _calls(api, p, t["Q"], t["K"], t["V"], t["dO"], stream=s)
        for s in streams:
            s.synchronize()
        for i in range(2):
            for k, t in refs[i].items():
                if i == 1 and k == "dQ":      # float32 atomics: summation order varies
                    assert float((got[i][k].float() - t.float()).norm() / t.float().norm()) < 1e-4, (i, k)
                else:
                    assert torch.equal(got[i][k], t), (i, k)
