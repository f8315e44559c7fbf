"""The allocation-free prologue entry point (sagebwd_quant_prologue_noalloc) against the
existing one (sagebwd_quant_prologue), through the C ABI: every output equal bit for bit, on
two calls in a row, the second with a smaller input (its scratch, the static per-device
array, then holds the first call's block sums, which the second call must not read). The
cases exercise both scratch regions (K-smoothing and Q-smoothing block sums), a ragged last
block and gains."""
import numpy as np
import pytest

from bit_trainable_attention_amd import workloads as wl
from tests.harness import host_inputs, params_for, to_device

pytestmark = pytest.mark.gpu
W = wl.WORKLOADS


def _run_both(w, gains=False):
    import torch
    from bit_trainable_attention_amd import api
    x = host_inputs(w)
    p = params_for(w, qk_gain=gains)
    Q, K, V = (to_device(x[k], w.dtype) for k in ("Q", "K", "V"))
    gq = gk = None
    if gains:
        rng = np.random.default_rng(700 + w.N)
        gq, gk = (torch.from_numpy((1 + 0.3 * rng.standard_normal((w.H, w.d))).astype(np.float32)).to("cuda:0")
                  for _ in range(2))
    ref = api.sagebwd_quant_prologue(p, Q, K, V, q_gain=gq, k_gain=gk)
    # outputs preallocated and filled with a pattern, so stale values would show
    out = {k: torch.full_like(v, 77) if v.dtype == torch.int8 else torch.full_like(v, -3.5) for k, v in ref.items()}
    got = api.sagebwd_quant_prologue_noalloc(p, Q, K, V, out=out, q_gain=gq, k_gain=gk)
    torch.cuda.synchronize()
    assert got is out
    for k in ref:
        a, b = ref[k].cpu().numpy(), got[k].cpu().numpy()
        assert a.dtype == b.dtype and np.array_equal(a, b), (k, int(np.sum(a != b)))
    return ref


def test_noalloc_matches_prologue_twice_shrinking():
    big = W["llama325m"].with_shape(B=2, H=4, N=1024, q_smooth=True, q_bias_var=4.0)
    small = W["n8192_d128"].with_shape(B=1, H=2, N=200, q_smooth=True, q_bias_var=4.0)
    print(f"[noalloc] call 1: B{big.B} H{big.H} N{big.N} d{big.d} blk{big.blk} q_smooth", flush=True)
    _run_both(big)
    print(f"[noalloc] call 2: B{small.B} H{small.H} N{small.N} d{small.d} blk{small.blk} q_smooth gains", flush=True)
    _run_both(small, gains=True)


def test_noalloc_metric_shape_k_smoothing():
    """At the metric's full shape (B2 H16 N8192 d128, K-smoothing: 1 MiB of block sums),
    then a smaller non-smoothed call (no scratch at all)."""
    w = W["n8192_d128"]
    print(f"[noalloc] call 1: B{w.B} H{w.H} N{w.N} d{w.d} blk{w.blk}", flush=True)
    _run_both(w)
    w2 = W["tiny"].with_shape(k_smooth=False, N=128)
    print(f"[noalloc] call 2: B{w2.B} H{w2.H} N{w2.N} d{w2.d} k_smooth off", flush=True)
    _run_both(w2)
