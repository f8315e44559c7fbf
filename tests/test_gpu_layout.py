"""The [B,N,H,d] layout of the 16-bit tensors (sagebwd_params.layout = SAGEBWD_LAYOUT_BNHD):
the kernels read Q, K, V, dO and write O, dQ, dK, dV in place, and every output equals the
[B,H,N,d] run on the same values bit for bit (only the addressing differs), in both dQ modes
and with Q-smoothing; one case is also held to the quantised oracle's bar directly."""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import quant as oq
from tests.harness import check_prologue, gpu_run, host_inputs, rel_l2, spec_for

pytestmark = pytest.mark.gpu
W = wl.WORKLOADS

CASES = [
    ("tiny", W["tiny"], 0),
    ("bf16_d64_causal", W["bf16_d64"].with_shape(B=2, H=3, N=512), 0),
    ("d128_causal_blk128", W["n8192_d128"].with_shape(B=1, H=3, N=384), 0),
    ("d128_causal_atomic", W["n8192_d128"].with_shape(B=2, H=2, N=256), 2),
    ("d128_blk64_qsmooth", W["n8192_d128"].with_shape(B=1, H=2, N=256, blk=64, q_smooth=True, q_bias_var=4.0), 0),
]


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,w,dq_mode", CASES)
def test_bnhd_equals_bhnd(name, w, dq_mode):
    _say(f"[layout] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} causal={w.causal} dq_mode={dq_mode}")
    x = host_inputs(w)
    ref = gpu_run(w, x, dq_mode=dq_mode)
    got = gpu_run(w, x, dq_mode=dq_mode, layout="bnhd")
    for k in ("Qc", "Kc", "Vtc", "Qs", "Ks", "Vs", "q_rstd", "k_rstd", "k_mean", "O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(got[k], ref[k]), (name, k)


def test_bnhd_meets_oracle_bar():
    name, w, _ = CASES[2]
    x = host_inputs(w)
    _say(f"[layout] {name}: [B,N,H,d] run against the quantised oracle")
    got = gpu_run(w, x, layout="bnhd")
    o = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec_for(w))
    check_prologue(got, o)
    errs = {k: rel_l2(got[k], o[k]) for k in ("O", "dQ", "dK", "dV")}
    _say(f"[layout] {name}: rel-L2 {errs}")
    for k, e in errs.items():
        assert e <= 2e-3, (k, e)
