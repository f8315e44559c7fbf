"""GPU parity of the Q-Attn precision split (sagebwd_params.split = QATTN; Full-Stack FP4 page,
section 2.4): QK^T and the dS products on the low-bit MFMA, PV, P^T dO and dO V^T on the 16-bit
MFMA, against the oracle run with Spec.split = "qattn" on the same seeded inputs.

Bars: the prologue's Q and K codes, scales and statistics bit-exact; O, dQ, dK, dV within
rel-L2 2e-3 of the quantised oracle (INT8 codes; 1e-2 with FP8 codes, the FP8 recipe's bar)
and the per-row bar; LSE within 1e-4 relative; cosine to exact float64 attention >= 0.995
(O) and >= 0.98 (gradients). Cases cover both dtypes, d in {64, 128}, blk in {64, 128},
masks, ragged N, [B,N,H,d], gains, both dQ modes and both code formats. The split's O and dV
must also be markedly closer to exact attention than the SageBwd split's on the same inputs,
and the autograd wrapper must give the C ABI's results bit for bit.
"""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import exact
from oracle import quant as oq
from tests.harness import ROW_TOL, check_prologue, cosine, gpu_run, host_inputs, rel_l2, row_rel_max, spec_for

pytestmark = pytest.mark.gpu
W = wl.WORKLOADS
OUTS = ("O", "dQ", "dK", "dV")

CASES = [
    # name, workload, dq_mode, layout, gains, fmt
    ("tiny_noncausal", W["tiny"], 0, "bhnd", False, "int8"),
    ("d128_blk128_causal", W["n8192_d128"].with_shape(B=1, H=2, N=512), 0, "bhnd", False, "int8"),
    ("bf16_d64_blk64", W["bf16_d64"].with_shape(B=1, H=2, N=512), 0, "bhnd", False, "int8"),
    ("bf16_d128_blk128", W["n8192_d128"].with_shape(B=1, H=2, N=384, dtype="bf16"), 0, "bhnd", False, "int8"),
    ("fp16_d64_blk128_ragged", W["tiny"].with_shape(B=1, H=2, N=300, blk=128, causal=True, qk_norm=True), 0,
     "bhnd", False, "int8"),
    ("d128_blk64_ragged_atomic", W["n8192_d128"].with_shape(B=1, H=2, N=200, blk=64), 2, "bhnd", False, "int8"),
    ("d64_bnhd_gains", W["llama325m"].with_shape(B=2, H=2, N=256), 0, "bnhd", True, "int8"),
    ("d128_noncausal_bnhd", W["n32768"].with_shape(B=1, H=2, N=320, causal=False), 0, "bnhd", False, "int8"),
    ("fp8_d128_blk128", W["n8192_d128"].with_shape(B=1, H=2, N=512), 0, "bhnd", False, "fp8"),
    ("fp8_bf16_d64_ragged_atomic", W["bf16_d64"].with_shape(B=1, H=2, N=333), 2, "bhnd", False, "fp8"),
]


def _gains(w, seed):
    rng = np.random.default_rng(seed)
    return tuple((1.0 + 0.3 * rng.standard_normal((w.H, w.d))).astype(np.float32) for _ in range(2))


@pytest.mark.parametrize("name,w,dq_mode,layout,gained,fmt", CASES)
def test_qattn_parity(name, w, dq_mode, layout, gained, fmt):
    print(f"[qattn] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} causal={w.causal} qk_norm={w.qk_norm} "
          f"dq_mode={dq_mode} layout={layout} gains={gained} fmt={fmt} seed={w.seed}", flush=True)
    x = host_inputs(w)
    gains = _gains(w, 900 + w.N) if gained else None
    g = gpu_run(w, x, dq_mode=dq_mode, layout=layout, gains=gains, fmt=fmt, split="qattn")
    o = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec_for(w, fmt=fmt, split="qattn"),
               q_gain=None if gains is None else gains[0], k_gain=None if gains is None else gains[1])
    check_prologue(g, o, check_v=False)
    keys = OUTS + (("dq_gain", "dk_gain") if gains else ())
    errs = {k: rel_l2(g[k], o[k]) for k in keys}
    rows = {k: row_rel_max(g[k], o[k]) for k in OUTS}
    lse = float(np.max(np.abs(g["LSE"].astype(np.float64) - o["LSE"])))
    ex = exact.attention(x["Qf"], x["Kf"], x["Vf"], x["dOf"], causal=w.causal, qk_norm=w.qk_norm, eps=w.eps,
                         q_gain=None if gains is None else gains[0], k_gain=None if gains is None else gains[1])
    cos = {k: cosine(g[k], ex[k]) for k in OUTS}
    print(f"[qattn] {name}: rel-L2 vs O-Q(qattn) {errs}, worst row {rows}, max|dLSE| {lse:.2e}, "
          f"cosine vs O-X {cos}", flush=True)
    tol = 1e-2 if fmt == "fp8" else 2e-3
    assert lse < 1e-4 * max(1.0, float(np.max(np.abs(o["LSE"]))))
    for k, e in errs.items():
        assert e <= tol, (k, e)
    for k, e in rows.items():
        assert e <= (5 if fmt == "fp8" else 1) * ROW_TOL, (k, e)
    assert cos["O"] >= 0.995 and min(cos[k] for k in OUTS[1:]) >= 0.98, cos


@pytest.mark.parametrize("name", ["n8192_d128", "bf16_d64"])
def test_qattn_closer_to_exact_than_sagebwd(name):
    """The same inputs through both splits on the GPU. O's error has two sources, the shared
    QK^T quantisation and PV's, which only the SageBwd split has; dV's error is dominated by
    the P^T dO quantisation, which the Q-Attn split removes. So O must be closer to exact
    attention with the Q-Attn split, and dV clearly closer (by at least 20%; measured 1.7x
    with the x20 outlier keys of the B2 H16 N8192 d128 distribution, 4x without them); dQ and
    dK share the INT8 dS path and stay within 10% of each other."""
    w = W[name].with_shape(B=1, H=2, N=1024)
    x = host_inputs(w)
    qa = gpu_run(w, x, split="qattn")
    sb = gpu_run(w, x)
    ex = exact.attention(x["Qf"], x["Kf"], x["Vf"], x["dOf"], causal=w.causal, qk_norm=w.qk_norm, eps=w.eps)
    e_qa = {k: rel_l2(qa[k], ex[k]) for k in OUTS}
    e_sb = {k: rel_l2(sb[k], ex[k]) for k in OUTS}
    print(f"[qattn] {name} vs exact: Q-Attn {e_qa}, SageBwd {e_sb}", flush=True)
    assert e_qa["O"] < e_sb["O"], (e_qa["O"], e_sb["O"])
    assert e_qa["dV"] < 0.8 * e_sb["dV"], (e_qa["dV"], e_sb["dV"])
    for k in ("dQ", "dK"):
        assert abs(e_qa[k] - e_sb[k]) <= 0.1 * e_sb[k], (k, e_qa[k], e_sb[k])


def test_qattn_autograd_matches_c_abi():
    import torch
    from bit_trainable_attention_amd.autograd import sagebwd_attention
    from tests.harness import to_device
    w = W["n8192_d128"].with_shape(B=1, H=2, N=384)
    x = host_inputs(w)
    ref = gpu_run(w, x, split="qattn")
    q, k, v = (to_device(x[n], w.dtype).requires_grad_() for n in ("Q", "K", "V"))
    o = sagebwd_attention(q, k, v, causal=w.causal, qk_norm=w.qk_norm, k_smooth=w.k_smooth, blk=w.blk, eps=w.eps,
                          split="qattn")
    o.backward(to_device(x["dO"], w.dtype))
    torch.cuda.synchronize()
    for name, t in (("O", o), ("dQ", q.grad), ("dK", k.grad), ("dV", v.grad)):
        assert np.array_equal(t.detach().float().cpu().numpy(), ref[name]), name
