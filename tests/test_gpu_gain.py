"""Learnable QK-norm gains (sagebwd_params.qk_gain): Q^ = g_Q o RMSNorm(Q), K^ = g_K o RMSNorm(K)
per head and channel, and the gains' gradients. The prologue's codes, scales and statistics
equal the oracle's bit for bit (one more float32 product per element); O, dQ, dK, dV and both
gain gradients meet rel-L2 2e-3 against the quantised oracle with the same gains, in both dQ
modes, both layouts and with Q-smoothing; unit gains reproduce the run without gains bit for
bit."""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import exact
from oracle import quant as oq
from tests.harness import check_prologue, cosine, gpu_run, host_inputs, rel_l2, spec_for

pytestmark = pytest.mark.gpu
W = wl.WORKLOADS

CASES = [
    ("bf16_d64_causal", W["bf16_d64"].with_shape(B=2, H=2, N=512), 0, "bhnd"),
    ("d128_causal_blk128", W["n8192_d128"].with_shape(B=2, H=2, N=384), 0, "bhnd"),
    ("d128_noncausal_blk64", W["n8192_d128"].with_shape(B=1, H=3, N=256, blk=64, causal=False), 0, "bhnd"),
    ("d128_atomic_dq", W["n8192_d128"].with_shape(B=2, H=2, N=256), 2, "bhnd"),
    ("d64_bnhd", W["llama325m"].with_shape(B=2, H=3, N=256), 0, "bnhd"),
    ("d128_qsmooth", W["n8192_d128"].with_shape(B=1, H=2, N=256, q_smooth=True, q_bias_var=4.0), 0, "bhnd"),
]


def _gains(w, seed):
    rng = np.random.default_rng(seed)
    return tuple((1.0 + 0.3 * rng.standard_normal((w.H, w.d))).astype(np.float32) for _ in range(2))


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,w,dq_mode,layout", CASES)
def test_gain_parity(name, w, dq_mode, layout):
    _say(f"[gain] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} causal={w.causal} "
         f"dq_mode={dq_mode} layout={layout}")
    x = host_inputs(w)
    gq, gk = _gains(w, 300 + w.N + w.d)
    g = gpu_run(w, x, dq_mode=dq_mode, layout=layout, gains=(gq, gk))
    o = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec_for(w), q_gain=gq, k_gain=gk)
    check_prologue(g, o)
    errs = {k: rel_l2(g[k], o[k]) for k in ("O", "dQ", "dK", "dV", "dq_gain", "dk_gain")}
    _say(f"[gain] {name}: rel-L2 {errs}")
    for k, e in errs.items():
        assert e <= 2e-3, (k, e)
    if w.N <= 512:
        ref = exact.attention(x["Qf"], x["Kf"], x["Vf"], x["dOf"], causal=w.causal, qk_norm=w.qk_norm,
                              eps=w.eps, q_gain=gq, k_gain=gk)
        cos = {k: cosine(g[k], ref[k]) for k in ("O", "dQ", "dK", "dV", "dq_gain", "dk_gain")}
        _say(f"[gain] {name}: cosine vs exact {cos}")
        assert cos["O"] >= 0.995 and min(cos[k] for k in ("dQ", "dK", "dV")) >= 0.98


def test_unit_gains_equal_no_gains():
    w = CASES[1][1]
    x = host_inputs(w)
    ones = np.ones((w.H, w.d), np.float32)
    a = gpu_run(w, x)
    b = gpu_run(w, x, gains=(ones, ones))
    for k in ("Qc", "Kc", "Qs", "Ks", "k_mean", "O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[k], b[k]), k


def test_autograd_gains_equal_c_abi():
    """The autograd wrapper's gain gradients (and dQ, dK, dV, O) equal the direct C-ABI run."""
    import torch
    from bit_trainable_attention_amd.autograd import sagebwd_attention
    from tests.harness import to_device
    w = CASES[0][1]
    x = host_inputs(w)
    gq, gk = _gains(w, 77)
    direct = gpu_run(w, x, gains=(gq, gk))
    q, k, v, dO = (to_device(x[n], w.dtype) for n in ("Q", "K", "V", "dO"))
    q, k, v = (t.requires_grad_() for t in (q, k, v))
    tgq, tgk = (torch.from_numpy(g).to("cuda:0").requires_grad_() for g in (gq, gk))
    O = sagebwd_attention(q, k, v, causal=w.causal, qk_norm=w.qk_norm, k_smooth=w.k_smooth, blk=w.blk, eps=w.eps,
                          q_gain=tgq, k_gain=tgk)
    O.backward(dO)
    torch.cuda.synchronize()
    got = {"O": O, "dQ": q.grad, "dK": k.grad, "dV": v.grad, "dq_gain": tgq.grad, "dk_gain": tgk.grad}
    for n, t in got.items():
        assert np.array_equal(t.detach().float().cpu().numpy().astype(np.float64), direct[n]), n
