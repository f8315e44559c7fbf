"""A synthetic study of gradient bias against averaging (the SageBwd article's account of why
large tokens-per-step budgets leave low-bit training behind: averaging over more tokens
removes the gradient noise but not the bias that the quantisation adds).

Fixed Q, K, V play the parameters; each "batch" i has an upstream gradient
dO_i = S + sigma * Z_i (a fixed signal S plus independent noise). For fixed Q, K, V the exact
gradients are linear in dO, so the exact gradient of an average of k batches is the exact
gradient at the average dO (one float64 evaluation per k). The quantised path is not linear
(dO is quantised per block, P and dS per tile). Its averaged gradient
g_k = mean_{i<k} g_q(dO_i) is compared with g_exact(mean_{i<k} dO_i):

    err_k = ||g_k - g_exact(mean dO)|| / ||g_exact(S)||.

Independent zero-mean rounding errors shrink like 1/sqrt(k); a bias does not. Fitting
err_k^2 = b^2 + v / k at k = 1 and k = 64 splits the two. The test prints the curve and the
fit for the INT8 and FP8 recipes. It asserts only what averaging must give when the noise
term dominates one batch (err_64 below err_1), that the single-batch error is not smaller than
the fitted floor, and that every figure is finite.
"""
import sys

import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import exact
from tests.harness import gpu_run, host_inputs

pytestmark = pytest.mark.gpu

KS = (1, 4, 16, 64)
SIGMA = 3.0


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_tps_bias_curve(fmt):
    w = wl.WORKLOADS["n8192_d128"].with_shape(B=1, H=2, N=1024)
    x = host_inputs(w)
    S = x["dOf"].astype(np.float64)
    rng = np.random.default_rng(7100)
    kmax = max(KS)
    grads, dos = [], []
    _say(f"[tps] {fmt}: {kmax} batches, B{w.B} H{w.H} N{w.N} d{w.d} {w.dtype}, sigma {SIGMA}")
    for i in range(kmax):
        d32 = (S + SIGMA * rng.standard_normal(S.shape)).astype(np.float32)
        bits = wl.f32_to_bits(d32, w.dtype)
        xi = dict(x, dO=bits, dOf=wl.bits_to_f32(bits, w.dtype))
        g = gpu_run(w, xi, fmt=fmt)
        grads.append(np.concatenate([g[k].ravel() for k in ("dQ", "dK", "dV")]))
        dos.append(xi["dOf"].astype(np.float64))

    def g_exact(dO):
        e = exact.attention(x["Qf"], x["Kf"], x["Vf"], dO, causal=w.causal, qk_norm=w.qk_norm, eps=w.eps)
        return np.concatenate([e[k].ravel() for k in ("dQ", "dK", "dV")])

    ref_norm = np.linalg.norm(g_exact(S))
    errs = {}
    for k in KS:
        gk = np.mean(grads[:k], axis=0)
        errs[k] = float(np.linalg.norm(gk - g_exact(np.mean(dos[:k], axis=0))) / ref_norm)
    # err_k^2 = b^2 + v/k from k = 1 and k = kmax
    v = (errs[1] ** 2 - errs[kmax] ** 2) / (1.0 - 1.0 / kmax)
    b2 = errs[kmax] ** 2 - v / kmax
    b = float(np.sqrt(max(b2, 0.0)))
    _say(f"[tps] {fmt}: err_k {errs}; fitted bias floor {b:.3e}, noise term sqrt(v) {np.sqrt(max(v, 0.0)):.3e} "
         f"(1/sqrt(k) prediction at k={kmax}: {errs[1] / np.sqrt(kmax):.3e})")
    assert all(np.isfinite(e) for e in errs.values())
    assert errs[kmax] < errs[1]
    assert errs[1] >= b
