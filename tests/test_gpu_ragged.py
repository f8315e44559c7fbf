"""Sequence lengths that are not a multiple of the quantisation block: the last block of a
head holds N mod blk tokens. The prologue's codes, scales and statistics equal the oracle's
bit for bit over all Np = ceil(N / blk) * blk rows (the padding rows: codes 0), the dO codes
in the backward's packets too, and O, dQ, dK, dV over the N real tokens meet rel-L2 2e-3;
across dtypes, head dims, blocks, masks, both dQ modes, both layouts, Q-smoothing and gains.
The 16-bit tensors hold exactly N tokens per head (no padding is read or written there)."""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import exact
from oracle import quant as oq
from tests.harness import check_prologue, cosine, gpu_run, host_inputs, rel_l2, spec_for

pytestmark = pytest.mark.gpu
W = wl.WORKLOADS

CASES = [
    ("bf16_d64_causal_n300", W["bf16_d64"].with_shape(B=2, H=2, N=300), 0, "bhnd", False),
    ("d128_causal_blk128_n200", W["n8192_d128"].with_shape(B=1, H=2, N=200), 0, "bhnd", False),
    ("d128_noncausal_blk64_n100", W["n8192_d128"].with_shape(B=1, H=3, N=100, blk=64, causal=False), 0, "bhnd", False),
    ("d128_causal_atomic_n333", W["n8192_d128"].with_shape(B=2, H=2, N=333), 2, "bhnd", False),
    ("d64_bnhd_gains_qsmooth_n257", W["llama325m"].with_shape(B=2, H=2, N=257, q_smooth=True, q_bias_var=4.0),
     0, "bnhd", True),
    ("d64_noncausal_blk128_n65", W["llama325m"].with_shape(B=1, H=2, N=65, blk=128, causal=False), 0, "bhnd", False),
    # eps = 0: the padding tokens must not be normalised (1/sqrt(0) would turn them into NaN)
    ("d128_eps0_gains_n200", W["n8192_d128"].with_shape(B=1, H=2, N=200, eps=0.0), 0, "bhnd", True),
    ("d64_eps0_atomic_n100", W["llama325m"].with_shape(B=1, H=2, N=100, eps=0.0), 2, "bhnd", False),
]


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,w,dq_mode,layout,gained", CASES)
def test_ragged_parity(name, w, dq_mode, layout, gained):
    _say(f"[ragged] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} causal={w.causal} "
         f"dq_mode={dq_mode} layout={layout} gains={gained} q_smooth={w.q_smooth}")
    x = host_inputs(w)
    gains = None
    if gained:
        rng = np.random.default_rng(500 + w.N)
        gains = tuple((1.0 + 0.3 * rng.standard_normal((w.H, w.d))).astype(np.float32) for _ in range(2))
    g = gpu_run(w, x, dq_mode=dq_mode, layout=layout, gains=gains)
    o = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec_for(w), q_gain=None if gains is None else gains[0],
               k_gain=None if gains is None else gains[1])
    check_prologue(g, o)
    assert np.array_equal(g["dOtc"], np.swapaxes(o["dOc"], -1, -2)), "dO codes"
    assert np.array_equal(g["dOs"], o["dOs"]), "dO scales"
    keys = ("O", "dQ", "dK", "dV") + (("dq_gain", "dk_gain") if gains else ())
    for k in ("O", "dQ", "dK", "dV"):
        assert g[k].shape == (w.B, w.H, w.N, w.d), (k, g[k].shape)
    errs = {k: rel_l2(g[k], o[k]) for k in keys}
    lse = float(np.max(np.abs(g["LSE"].astype(np.float64) - o["LSE"])))
    _say(f"[ragged] {name}: rel-L2 {errs}, max|dLSE| {lse:.2e}")
    assert lse < 1e-4 * max(1.0, float(np.max(np.abs(o["LSE"]))))
    for k, e in errs.items():
        assert e <= 2e-3, (k, e)
    ref = exact.attention(x["Qf"], x["Kf"], x["Vf"], x["dOf"], causal=w.causal, qk_norm=w.qk_norm, eps=w.eps,
                          q_gain=None if gains is None else gains[0], k_gain=None if gains is None else gains[1])
    cos = {k: cosine(g[k], ref[k]) for k in ("O", "dQ", "dK", "dV")}
    _say(f"[ragged] {name}: cosine vs exact {cos}")
    assert cos["O"] >= 0.995 and min(cos[k] for k in ("dQ", "dK", "dV")) >= 0.98
