"""Pins of the oracle's Q-Attn precision split (Spec.split = "qattn"; Full-Stack FP4 page,
section 2.4: QK^T and dS low-bit, PV, P^T dO and dO V^T in 16 bits).

- Reduction: with the dS tiles left unquantised and no 16-bit rounding (dtype "f64"), the
  split must equal exact float64 attention on the dequantised Q and K codes with the raw V and
  dO: S comes from the INT8 codes, nothing else is quantised. The SageBwd split (P~, V, P, dO
  quantised) must not.
- Planted mistakes: V or dO quantised, or P~ quantised, breaks the reduction.
- With a 16-bit dtype P~ and P are rounded (the result moves by about the rounding, bf16 more
  than fp16), and the split's O and dV are closer to exact attention than the SageBwd split's.
"""
import numpy as np
import pytest

from oracle import exact
from oracle import quant as oq

F32 = np.float32


def _case(seed, N=192, d=32, B=1, H=2):
    rng = np.random.default_rng(seed)
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    K = (K + 2 * rng.standard_normal((1, H, 1, d))).astype(F32)
    return Q, K, V, dO


def _deq_reference(Q, K, V, dO, spec):
    """Exact attention on the dequantised prologue codes of Q and (smoothed) K, raw V and dO."""
    pro = oq.prologue(Q, K, V, spec)
    blk = spec.blk
    qd = pro["Qc"].astype(np.float64) * np.repeat(pro["Qs"], blk, axis=-1)[..., None]
    kd = pro["Kc"].astype(np.float64) * np.repeat(pro["Ks"], blk, axis=-1)[..., None]
    return exact.attention(qd, kd, V, dO, causal=spec.causal, qk_norm=False, sm_scale=spec.scale)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _spec(causal, split="qattn", dtype="f64", N=192, d=32):
    return oq.Spec(N=N, d=d, blk=64, causal=causal, qk_norm=False, k_smooth=True, dtype=dtype, split=split,
                   fwd_tk=64 if split == "qattn" else None)


@pytest.mark.parametrize("causal", [False, True])
def test_qattn_reduces_to_exact_on_dequantised_qk(causal):
    Q, K, V, dO = _case(21 + causal)
    spec = _spec(causal)
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant)
    ref = _deq_reference(Q, K, V, dO, spec)
    # O in float64 throughout; the backward's P = exp(s - LSE) takes the float32 LSE the
    # forward stores (relative 1e-7)
    assert _rel(got["O"], ref["O"]) < 1e-10, _rel(got["O"], ref["O"])
    for k in ("dQ", "dK", "dV"):
        assert _rel(got[k], ref[k]) < 1e-6, (k, _rel(got[k], ref[k]))
    np.testing.assert_allclose(got["LSE"], ref["LSE"], rtol=1e-6, atol=1e-6)
    # the SageBwd split quantises P~, V, P and dO: far from this reference
    sb = oq.run(Q, K, V, dO, _spec(causal, split="sagebwd"), tile_quant=oq.identity_tile_quant)
    assert _rel(sb["O"], ref["O"]) > 1e-3 and _rel(sb["dV"], ref["dV"]) > 1e-3


@pytest.mark.parametrize("mistake", ["v_and_dO_quantised", "ptilde_quantised"])
def test_qattn_planted_mistake_is_caught(monkeypatch, mistake):
    Q, K, V, dO = _case(31)
    spec = _spec(True)
    ref = _deq_reference(Q, K, V, dO, spec)
    if mistake == "v_and_dO_quantised":
        monkeypatch.setattr(oq, "identity_block_quant", oq.quant_blocks_f32)
    else:
        monkeypatch.setattr(oq, "half_round_tile", lambda dtype: oq.int8_tile_quant)
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant)
    assert max(_rel(got[k], ref[k]) for k in ("O", "dV")) > 1e-4, mistake


def test_qattn_rounds_p_to_the_dtype():
    """With fp16 / bf16 the P~ and P operands are rounded: O and dV move from the unrounded
    result by roughly the type's relative precision (bf16 2^-9, fp16 2^-12), bf16 more."""
    Q, K, V, dO = _case(41)
    base = oq.run(Q, K, V, dO, _spec(True), tile_quant=oq.identity_tile_quant)
    e = {}
    for dt in ("fp16", "bf16"):
        r = oq.run(Q, K, V, dO, _spec(True, dtype=dt), tile_quant=oq.identity_tile_quant)
        e[dt] = max(_rel(r["O"], base["O"]), _rel(r["dV"], base["dV"]))
    assert 1e-5 < e["fp16"] < e["bf16"] < 1e-2, e


@pytest.mark.parametrize("causal", [False, True])
def test_qattn_closer_to_exact_than_sagebwd(causal):
    """INT8 codes everywhere they apply: the Q-Attn split (PV and P^T dO in 16 bits) gives O and
    dV markedly closer to exact attention than the SageBwd split (both in INT8)."""
    Q, K, V, dO = _case(51 + causal, N=256)
    kw = dict(N=256, d=32, blk=64, causal=causal, qk_norm=True, k_smooth=True, dtype="fp16")
    qa = oq.run(Q, K, V, dO, oq.Spec(split="qattn", fwd_tk=64, **kw))
    sb = oq.run(Q, K, V, dO, oq.Spec(**kw))
    ex = exact.attention(Q, K, V, dO, causal=causal, qk_norm=True)
    for k in ("O", "dV"):
        assert _rel(qa[k], ex[k]) < 0.5 * _rel(sb[k], ex[k]), (k, _rel(qa[k], ex[k]), _rel(sb[k], ex[k]))
    for k in ("dQ", "dK"):   # still through INT8 dS codes: comparable errors
        assert _rel(qa[k], ex[k]) < 1.2 * _rel(sb[k], ex[k]), k
