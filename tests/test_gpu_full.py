"""GPU parity at the full workload shapes, in the launch configuration bench.py times.

The HIP path runs on every head; the oracle checks
  - the prologue (codes, scales, rstd, mean) on every head, bit for bit;
  - O, LSE, dQ, dK, dV on sampled heads that it recomputes whole (or, at N = 32768, on sampled
    query tiles and the last key blocks, with the oracle forward run on exactly the rows that
    those need), against the rel-L2 <= 2e-3 bar.
"""
import sys

import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import quant as oq
from tests.harness import gpu_run, host_inputs, rel_l2, spec_for

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _head(a, w, bh):
    """Flattened head bh of a [B,H,...] array, as [1,1,...]."""
    return a.reshape((w.B * w.H,) + a.shape[2:])[bh][None, None]


def _check_prologue_all_heads(g, x, w):
    spec = spec_for(w)
    o = oq.prologue(x["Qf"], x["Kf"], x["Vf"], spec)
    for k in ("Qc", "Kc", "Qs", "Ks", "Vs", "q_rstd", "k_rstd", "k_mean"):
        assert np.array_equal(g[k], o[k]), (k, int(np.sum(g[k] != o[k])))
    assert np.array_equal(g["Vtc"], np.swapaxes(o["Vc"], -1, -2))
    dOc, dOs = oq.quant_blocks_f32(x["dOf"], w.blk)
    assert np.array_equal(g["dOtc"], np.swapaxes(dOc, -1, -2))
    assert np.array_equal(g["dOs"], dOs)


@pytest.mark.parametrize("name,heads", [("bf16_d64", [0, 37]), ("n8192_d128", [31]), ("llama325m", [77])])
def test_full_shape_whole_heads(name, heads):
    w = wl.WORKLOADS[name]
    _say(f"[full] {name}: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk} {w.dtype} seed={w.seed}: GPU on all heads")
    x = host_inputs(w)
    g = gpu_run(w, x)
    _check_prologue_all_heads(g, x, w)
    w1 = w.with_shape(B=1, H=1)
    spec = spec_for(w1)
    for bh in heads:
        _say(f"[full] {name}: oracle on head {bh}")
        xh = {k: _head(x[k], w, bh) for k in ("Qf", "Kf", "Vf", "dOf")}
        o = oq.run(xh["Qf"], xh["Kf"], xh["Vf"], xh["dOf"], spec)
        errs = {k: rel_l2(_head(g[k], w, bh), o[k]) for k in ("O", "dQ", "dK", "dV")}
        lse = float(np.max(np.abs(_head(g["LSE"], w, bh).astype(np.float64) - o["LSE"])))
        _say(f"[full] {name} head {bh}: rel-L2 {errs}, max|dLSE| {lse:.2e}")
        assert lse < 1e-4 * max(1.0, float(np.max(np.abs(o["LSE"]))))
        for k, e in errs.items():
            assert e <= TOL, (k, e)


def test_full_shape_long_sequence_sampled():
    """N = 32768: sampled query tiles and the last key blocks of one head."""
    w = wl.WORKLOADS["n32768"]
    _say(f"[full] n32768: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk}: GPU on all heads")
    x = host_inputs(w)
    g = gpu_run(w, x)
    _check_prologue_all_heads(g, x, w)
    bh = 5
    w1 = w.with_shape(B=1, H=1)
    spec = spec_for(w1)
    xh = {k: _head(x[k], w, bh) for k in ("Qf", "Kf", "Vf", "dOf")}
    pro = oq.prologue(xh["Qf"], xh["Kf"], xh["Vf"], spec)
    N, tq, btq, sk = w.N, spec.fwd_tq, spec.bwd_tq, spec.sk
    k_blocks = [N // sk - 2, N // sk - 1]                   # dK, dV: last two key blocks
    q_bwd = [3, 170, N // btq - 1]                          # dQ: sampled query tiles (btq rows)
    rows = set(range(k_blocks[0] * sk, N))                  # rows the sampled pairs need O/LSE for
    for it in q_bwd:
        rows |= set(range(it * btq, (it + 1) * btq))
    q_fwd = sorted({r // tq for r in rows})
    _say(f"[full] n32768 head {bh}: oracle forward on {len(q_fwd)} query tiles")
    O, L = oq.forward(pro["Qc"], pro["Kc"], pro["Vc"], pro["Qs"], pro["Ks"], pro["Vs"], spec, q_tiles=q_fwd)
    _say("[full] n32768: oracle backward on the sampled tiles")
    gb = oq.backward(pro, xh["Qf"], xh["Kf"], xh["Vf"], O, L, xh["dOf"], spec, q_tiles=q_bwd, k_tiles=k_blocks)
    r = np.array(sorted(rows))
    errO = rel_l2(_head(g["O"], w, bh)[..., r, :], O[..., r, :])
    qr = np.concatenate([np.arange(it * btq, (it + 1) * btq) for it in q_bwd])
    kr = np.arange(k_blocks[0] * sk, N)
    errs = {"O": errO,
            "dQ": rel_l2(_head(g["dQ"], w, bh)[..., qr, :], gb["dQ"][..., qr, :]),
            "dK": rel_l2(_head(g["dK"], w, bh)[..., kr, :], gb["dK"][..., kr, :]),
            "dV": rel_l2(_head(g["dV"], w, bh)[..., kr, :], gb["dV"][..., kr, :])}
    lse = float(np.max(np.abs(_head(g["LSE"], w, bh)[..., r].astype(np.float64) - L[..., r])))
    _say(f"[full] n32768 head {bh}: rel-L2 {errs}, max|dLSE| {lse:.2e}")
    assert lse < 1e-4 * max(1.0, float(np.nanmax(np.abs(L[..., r]))))
    for k, e in errs.items():
        assert e <= TOL, (k, e)
