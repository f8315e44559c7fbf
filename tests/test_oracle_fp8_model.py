"""Where the FP8 parity bar (rel-L2 1e-2 of O, dQ, dK, dV against the FP8 oracle) comes from:
a CPU model of the FP8 matrix cores' float32 accumulation.

The INT8 products are exact int32 sums, so the INT8 path differs from its oracle only by the
float32 arithmetic around them (bar 2e-3). The FP8 MFMAs sum their products in float32 but
not exactly: a probe on gfx950 measured deviations near 2^-16 of the sum of |terms| against
the exact sum. The model replaces each low-bit product element of the oracle (QK^T in both
passes, PV, dV, dK, dQ; oracle.quant.lowbit_product) by exact + u * 2^-16 * sum|terms|, u
uniform in [-1, 1], independent per element and per pass (the forward and backward recompute
QK^T with different MFMA forms), and runs the FP8 oracle on the shapes and seeded inputs of
the FP8 GPU tests. The error moves scores, so P~, P and dS codes flip at near-ties; those flips
(one e4m3 step, up to 1/8 of a value) dominate the discrepancy. The hardware reciprocal the
kernels use for tile scales (about one ulp) moves a code only within ~2^-19 of a tie:
negligible.

Result (printed): 8e-4 to 9.1e-3, the largest on the bf16 d64 case (dQ 9.1e-3, dK 8.2e-3),
whose dO of standard deviation 0.1 makes dS small and its tile codes coarse. The bar is the
model's worst case rounded up to 1e-2; asserted: every case and output stays within it. The
model is pessimistic (it spreads the probe's bound uniformly): the GPU measures 0.6e-3 to
4.2e-3 on the same cases.
"""
import numpy as np
import pytest

from oracle import quant as oq
from tests.harness import host_inputs, rel_l2, spec_for

BAR_FP8 = 1e-2
OUTS = ("O", "dQ", "dK", "dV")


def _cases():
    from tests.test_gpu_fp8 import CASES
    return sorted(CASES.items())


def noisy_product(rng, rel=2.0 ** -16):
    def mm(a, b):
        exact = a @ b
        mag = np.abs(a) @ np.abs(b)
        return exact + rng.uniform(-1.0, 1.0, exact.shape) * rel * mag
    return mm


def run_modelled(x, spec, seed, **kw):
    """oracle.quant.run with every low-bit product replaced by the noise model (seeded)."""
    real = oq.lowbit_product
    oq.lowbit_product = noisy_product(np.random.default_rng(seed))
    try:
        return oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec, **kw)
    finally:
        oq.lowbit_product = real


def model_discrepancy(w, seed=0):
    x = host_inputs(w)
    spec = spec_for(w, fmt="fp8")
    ref = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec)
    got = run_modelled(x, spec, seed)
    return {k: rel_l2(got[k], ref[k]) for k in OUTS}


@pytest.mark.parametrize("name,w", _cases(), ids=[n for n, _ in _cases()])
def test_fp8_bar_covers_modelled_accumulation(name, w):
    e = model_discrepancy(w)
    print(f"[fp8 model] {name}: rel-L2 modelled FP8 accumulation vs exact products {e}", flush=True)
    for k, v in e.items():
        assert v <= BAR_FP8, (k, v)


def test_model_is_inert_for_int8_sums():
    """The same noise model with rel = 0 reproduces the oracle bit for bit (the seam changes
    nothing by itself)."""
    from bit_trainable_attention_amd import workloads as wl
    w = wl.WORKLOADS["tiny"].with_shape(N=128)
    x = host_inputs(w)
    spec = spec_for(w, fmt="fp8")
    ref = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec)
    real = oq.lowbit_product
    oq.lowbit_product = noisy_product(np.random.default_rng(1), rel=0.0)
    try:
        got = oq.run(x["Qf"], x["Kf"], x["Vf"], x["dOf"], spec)
    finally:
        oq.lowbit_product = real
    for k in OUTS:
        assert np.array_equal(got[k], ref[k]), k
