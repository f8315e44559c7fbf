"""Q-smoothing through the HIP path against the quantised oracle (oracle.quant with
Spec.q_smooth): prologue codes, scales and the query mean bit-exact, the key bias within
float32 rounding, O/dQ/dK/dV within rel-L2 2e-3 and LSE within 1e-4, as for the default path.
Every case adds a per-(head, channel) offset to Q (drawn last), so mu_Q and the bias terms
are large."""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import quant as oq
from tests.harness import check_prologue, cosine, gpu_run, host_inputs, rel_l2, spec_for

pytestmark = pytest.mark.gpu
TOL = 2e-3
W = wl.WORKLOADS

CASES = [
    ("bf16_d64_causal", W["bf16_d64"].with_shape(B=1, H=2, N=512, q_smooth=True, q_bias_var=4.0), 0),
    ("d128_causal", W["n8192_d128"].with_shape(B=1, H=2, N=512, q_smooth=True, q_bias_var=4.0), 0),
    ("d128_blk64_noncausal", W["n8192_d128"].with_shape(B=1, H=2, N=256, blk=64, causal=False, q_smooth=True,
                                                         q_bias_var=2.0), 0),
    ("d64_blk128_no_k_smooth", W["llama325m"].with_shape(B=1, H=2, N=384, blk=128, k_smooth=False, q_smooth=True,
                                                          q_bias_var=4.0), 0),
    ("d128_atomic_dq", W["n8192_d128"].with_shape(B=1, H=2, N=384, q_smooth=True, q_bias_var=4.0), 2),
]


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,w,dq_mode", CASES)
def test_q_smoothing_parity(name, w, dq_mode):
    _say(f"[qsmooth] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} causal={w.causal} "
         f"k_smooth={w.k_smooth} dq_mode={dq_mode}")
    x = host_inputs(w)
    g = gpu_run(w, x, dq_mode=dq_mode)
    o = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec_for(w))
    check_prologue(g, o)
    errs = {k: rel_l2(g[k], o[k]) for k in ("O", "dQ", "dK", "dV")}
    lse = float(np.max(np.abs(g["LSE"].astype(np.float64) - o["LSE"])))
    _say(f"[qsmooth] {name}: rel-L2 {errs}, max|dLSE| {lse:.2e}, |kbias| max {np.max(np.abs(o['kbias'])):.3f}")
    assert lse < 1e-4 * max(1.0, float(np.max(np.abs(o["LSE"]))))
    for k, e in errs.items():
        assert e <= TOL, (k, e)


def test_q_smoothing_terms_matter():
    """Q-smoothing is a reparametrisation: the GPU's Q-smoothed outputs approximate the same
    attention as the oracle's run without Q-smoothing on the same inputs (whose Q offsets
    make the key bias large, |b| ~ 25, so a missing or wrong bias term would not)."""
    name, w, _ = CASES[1]
    x = host_inputs(w)
    g = gpu_run(w, x)
    plain = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec_for(w.with_shape(q_smooth=False)))
    for k in ("O", "dQ", "dK", "dV"):
        c = cosine(g[k], plain[k])
        _say(f"[qsmooth] {name}: cosine(GPU Q-smoothed, oracle without Q-smoothing) {k} {c:.5f}")
        assert c > 0.99, (k, c)
