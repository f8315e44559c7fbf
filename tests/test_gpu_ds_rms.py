"""RMS(dS) against N on the GPU path (SageBwd article, dS-magnitude paragraph: RMS(dS) falls
with the sequence length, like 1/sqrt(N) by an upper-bound analysis, which makes dS the
low-SNR operand of INT8).

Inputs: the long-sequence workload's distribution (fp16 N(0,1), d = 128, causal, QK-norm,
K-smoothing, 128-token blocks), one head, N = 2048 ... 32768. The backward runs with the dS
spill, whose workspace holds every visible tile's INT8 dS codes and, per 64 keys, the dQ
multiplier sm_scale * s_dS * s_K (layout in include/sagebwd.h). Dividing by sm_scale * s_K
gives each tile's dS scale, so the GPU's own quantised dS, code * s_dS, is read back without
any extra kernel output. Reported per N: the elementwise RMS of the GPU's quantised dS over the
visible (query, key) pairs, the share of visible pairs whose dS code is 0, and (N <= 8192)
the RMS of exact float64 dS. Asserted: the GPU's RMS(dS) falls with N at least like N^-0.4
(the bound's N^-0.5, with the tolerance the oracle's own pin uses), and stays within a
factor 2 of the exact RMS where both are computed.
"""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from oracle import exact
from tests.harness import host_inputs, params_for, to_device

pytestmark = pytest.mark.gpu

NS = (2048, 4096, 8192, 16384, 32768)
EXACT_MAX_N = 8192


def _gpu_ds_stats(w):
    import torch
    from bit_trainable_attention_amd import api
    x = host_inputs(w)
    p = params_for(w, dq_mode=1)
    Q, K, V, dO = (to_device(x[k], w.dtype) for k in ("Q", "K", "V", "dO"))
    pro = api.sagebwd_quant_prologue(p, Q, K, V)
    O, lse = api.sagebwd_forward(p, pro)
    g = api.sagebwd_backward(p, Q, K, V, pro, O, lse, dO)
    torch.cuda.synchronize()
    lay = api.backward_workspace_layout(p)
    assert lay["spill"] == 1
    ws = g["workspace"]
    blk, N, T = w.blk, w.N, lay["tiles_per_head"]
    nb, nt, r = N // blk, N // 64, blk // 64
    kd = blk // 64
    codes = ws[lay["dsp"]:lay["dsp"] + T * 64 * blk].view(torch.int8).view(T, blk, 64)   # one head
    mult = ws[lay["dsm"]:lay["dsm"] + T * kd * 4].view(torch.float32).view(T, kd)
    # key block of every tile (causal: key block kb holds the query tiles kb*r .. nt-1)
    kb_of = np.concatenate([np.full(nt - kb * r, kb) for kb in range(nb)])
    assert kb_of.size == T
    sk = pro["Ks"].view(-1)[:nb]
    s_ds = mult / (float(w.sm_scale) * sk[torch.from_numpy(kb_of).to(ws.device)])[:, None]    # [T, kd]
    sq, zeros = 0.0, 0
    for t0 in range(0, T, 4096):
        c = codes[t0:t0 + 4096].float().view(-1, kd, 64, 64)                                   # [t, group, key, q]
        sq += float(((c * c).sum(dim=(2, 3)) * s_ds[t0:t0 + 4096] ** 2).sum())
        zeros += int((c == 0).sum())
    visible = N * (N + 1) // 2
    masked = T * 64 * blk - visible      # diagonal tiles' masked pairs hold code 0
    return float(np.sqrt(sq / visible)), (zeros - masked) / visible, x


def _fit(ns, vals):
    return float(np.polyfit(np.log(ns), np.log(vals), 1)[0])


def test_ds_rms_falls_with_n():
    base = wl.WORKLOADS["n32768"]
    gpu, zero, ex = {}, {}, {}
    for N in NS:
        w = base.with_shape(B=1, H=1, N=N)
        print(f"[ds_rms] N={N}: GPU prologue/forward/backward (dS spill), seed={w.seed}", flush=True)
        gpu[N], zero[N], x = _gpu_ds_stats(w)
        if N <= EXACT_MAX_N:
            e = exact.attention(x["Qf"], x["Kf"], x["Vf"], x["dOf"], causal=True, qk_norm=True, eps=w.eps,
                                want_ds_stats=True)
            ex[N] = float(np.sqrt(np.sum(e["ds_l2"] ** 2) / (N * (N + 1) / 2)))
        print(f"[ds_rms] N={N}: RMS(dS) GPU (dequantised codes) {gpu[N]:.4e}, exact "
              f"{ex.get(N, float('nan')):.4e}, visible dS codes equal to 0: {100 * zero[N]:.2f}%", flush=True)
    fg = _fit(NS, [gpu[n] for n in NS])
    fe = _fit(sorted(ex), [ex[n] for n in sorted(ex)])
    print(f"[ds_rms] fitted exponent of RMS(dS) in N: GPU {fg:.3f} (N {NS[0]}..{NS[-1]}), exact {fe:.3f} "
          f"(N {min(ex)}..{max(ex)})", flush=True)
    assert fg <= -0.4, fg
    for n, v in ex.items():
        assert 0.5 <= gpu[n] / v <= 2.0, (n, gpu[n], v)
