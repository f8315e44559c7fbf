"""GPU parity of the FP8 (e4m3) recipe: the HIP path with sagebwd_params.fmt = FP8 against the
oracle run with Spec.fmt = "fp8" on the same seeded inputs.

Bars: the prologue's e4m3 codes, block scales and statistics, and the dO codes and scales,
are bit-exact (both sides round fl(x * 448/absmax) to nearest even); O, dQ, dK, dV reach
rel-L2 <= 1e-2 against the quantised oracle. The tolerance is looser than the INT8 bar
because the FP8 matrix cores accumulate in float32 without exactness (deviations near 2^-16
of the sum of |terms| were measured on the hardware, against exact int32 sums for INT8), and
the moved scores flip P~, P and dS codes at near-ties by one e4m3 step (up to 1/8 of a
value; INT8: 1/127 of the tile maximum). tests/test_oracle_fp8_model.py puts that error into
the oracle's products on these very cases: 8e-4 to 9.1e-3; the bar is its worst case rounded
up.
"""
import sys

import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import exact
from oracle import quant as oq
from tests.harness import check_prologue, cosine, gpu_run, host_inputs, rel_l2, spec_for

pytestmark = pytest.mark.gpu

TOL_FP8 = 1e-2
W = wl.WORKLOADS

CASES = {
    "tiny": W["tiny"],
    "n8192_d128_small": W["n8192_d128"].with_shape(B=1, H=2, N=512),
    "bf16_d64_small": W["bf16_d64"].with_shape(B=1, H=2, N=512),
    "d128_blk64_ragged": W["n8192_d128"].with_shape(B=1, H=2, N=200, blk=64, k_outlier_channels=0),
    "d64_blk128_noncausal_bf16": W["bf16_d64"].with_shape(B=1, H=2, N=384, blk=128, causal=False),
    "no_norm_no_smooth": W["tiny"].with_shape(N=320, causal=True, qk_norm=False, k_smooth=False),
    # the remaining (dtype, d, blk) instantiations the library dispatches
    "fp16_d64_blk128": W["tiny"].with_shape(B=1, H=2, N=384, blk=128, causal=True, qk_norm=True),
    "bf16_d128_blk64": W["n8192_d128"].with_shape(B=1, H=2, N=320, blk=64, dtype="bf16"),
    "bf16_d128_blk128": W["n8192_d128"].with_shape(B=1, H=2, N=512, dtype="bf16"),
    # a ragged last block whose second 64-key group is all padding: that dS tile is all zero
    # (its inverse scale must not become inf, or the FP8 codes turn NaN and so does dQ)
    "d128_blk128_padding_dS_tile": W["n8192_d128"].with_shape(B=1, H=2, N=300),
}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _errs(g, o):
    return {k: rel_l2(g[k], o[k]) for k in ("O", "dQ", "dK", "dV")}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_end_to_end(name):
    w = CASES[name]
    spec = spec_for(w, fmt="fp8")
    _say(f"[fp8] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} causal={w.causal} seed={w.seed}")
    x = host_inputs(w)
    g = gpu_run(w, x, fmt="fp8")
    o = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec)
    check_prologue(g, o)
    assert np.array_equal(g["dOtc"], np.swapaxes(o["dOc"], -1, -2))
    assert np.array_equal(g["dOs"], o["dOs"])
    errs = _errs(g, o)
    lse_err = float(np.max(np.abs(g["LSE"].astype(np.float64) - o["LSE"])))
    ex = exact.attention(x["Qf"], x["Kf"], x["Vf"], x["dOf"], causal=w.causal, qk_norm=w.qk_norm, eps=w.eps)
    cos = {k: cosine(g[k], ex[k]) for k in ("O", "dQ", "dK", "dV")}
    _say(f"[fp8] {name}: rel-L2 vs O-Q(fp8) {errs}, max|dLSE| {lse_err:.2e}, cosine vs O-X {cos}")
    assert lse_err < 1e-3 * max(1.0, float(np.max(np.abs(o["LSE"]))))
    for k, e in errs.items():
        assert e <= TOL_FP8, (k, e)


def test_fp8_dq_modes_agree():
    w = CASES["n8192_d128_small"]
    x = host_inputs(w)
    o = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec_for(w, fmt="fp8"))
    gs = gpu_run(w, x, dq_mode=1, fmt="fp8")
    ga = gpu_run(w, x, dq_mode=2, fmt="fp8")
    _say(f"[fp8] dq modes: spill {_errs(gs, o)} atomic {_errs(ga, o)}")
    for g in (gs, ga):
        for k in ("dQ", "dK", "dV"):
            assert rel_l2(g[k], o[k]) <= TOL_FP8, k
    assert np.array_equal(gs["dK"], ga["dK"]) and np.array_equal(gs["dV"], ga["dV"])
    assert rel_l2(gs["dQ"], ga["dQ"]) < 1e-3


def test_fp8_codes_differ_from_int8():
    """The flag reaches the kernels: the same inputs give e4m3 codes (scale absmax/448) with
    fmt FP8 and integer codes (absmax/127) with INT8."""
    w = CASES["tiny"]
    x = host_inputs(w)
    g8 = gpu_run(w, x, stages=("prologue",), fmt="fp8")
    gi = gpu_run(w, x, stages=("prologue",))
    np.testing.assert_allclose(g8["Qs"] * 448.0, gi["Qs"] * 127.0, rtol=1e-6)
    assert not np.array_equal(g8["Qc"].view(np.int8), gi["Qc"])
