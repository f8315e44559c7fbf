"""Pins of where the oracle's in-kernel quantisers sit (the tile placement), against a fixture
derived in exact rational arithmetic without the oracle (tests/golden/make_tile_fixture.py ->
tile_placement_fixture.json):

  - forward: P~ is quantised on fwd_tq x fwd_tk tiles, the running max moves once per key tile,
    and l sums P~ before quantisation (so LSE does not depend on the P~ quantiser at all);
  - backward: P on bwd_tq x bwd_pk tiles (dV), dS on bwd_tq x bwd_sk tiles (dK, dQ).

The oracle run with any other tile shape (a per-row P~ scale, a taller tile, a per-key running
max, P or dS tiles of other shapes) must miss the fixture. A spy quantiser checks that the
tiles handed to the quantiser have the Spec's shapes and count on a larger causal case.
"""
import json
import os

import numpy as np
import pytest

from oracle import exact
from oracle import quant as oq

F32 = np.float32
FIX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tile_placement_fixture.json")))


def _spec(**over):
    s = dict(FIX["spec"])
    s.update(over)
    return oq.Spec(**s)


def _inputs():
    return {k: np.asarray(v, dtype=F32)[None, None] for k, v in FIX["inputs"].items()}


def _forward(spec):
    x = _inputs()
    pro = oq.prologue(x["Q"], x["K"], x["V"], spec)
    # every block's absmax is 127: scale 1 and the codes are the values
    assert np.array_equal(pro["Qc"], x["Q"].astype(np.int8)) and np.all(pro["Qs"] == 1)
    return oq.forward(pro["Qc"], pro["Kc"], pro["Vc"], pro["Qs"], pro["Ks"], pro["Vs"], spec)


def _backward(spec):
    x = _inputs()
    pro = oq.prologue(x["Q"], x["K"], x["V"], spec)
    O = np.asarray(FIX["expected"]["O"], np.float64)[None, None]
    lse = np.asarray(FIX["expected"]["LSE"], F32)[None, None]
    return oq.backward(pro, x["Q"], x["K"], x["V"], O, lse, x["dO"], spec)


def _close(a, b, rtol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return bool(np.all(np.abs(a - b) <= rtol * np.maximum(np.abs(b), 1e-3 * np.max(np.abs(b)))))


def test_fixture_forward():
    O, lse = _forward(_spec())
    assert _close(O[0, 0], FIX["expected"]["O"], 1e-6), O[0, 0]
    assert _close(lse[0, 0], FIX["expected"]["LSE"], 1e-6), lse[0, 0]


@pytest.mark.parametrize("over", [dict(fwd_tq=1), dict(fwd_tq=4), dict(fwd_tk=1), dict(fwd_tk=4),
                                  dict(fwd_tq=1, fwd_tk=4)])
def test_fixture_forward_other_tiles_miss(over):
    """A per-row P~ scale (fwd_tq 1), a 4-row tile, a running max per key (fwd_tk 1) or per 4
    keys: O moves by 1e-3 and more of its values."""
    O, _ = _forward(_spec(**over))
    assert not _close(O[0, 0], FIX["expected"]["O"], 1e-4), over


def test_fixture_backward():
    g = _backward(_spec())
    for k in ("dQ", "dK", "dV"):
        assert _close(g[k][0, 0], FIX["expected"][k], 1e-5), (k, g[k][0, 0], FIX["expected"][k])


@pytest.mark.parametrize("over", [dict(bwd_tq=1), dict(bwd_tq=4), dict(bwd_pk=2), dict(bwd_sk=1, bwd_pk=1),
                                  dict(bwd_sk=4), dict(bwd_tq=4, bwd_sk=4, bwd_pk=4)])
def test_fixture_backward_other_tiles_miss(over):
    """P or dS quantised on other tiles: some of dQ, dK, dV move by 1e-3 and more."""
    g = _backward(_spec(**over))
    assert not all(_close(g[k][0, 0], FIX["expected"][k], 1e-4) for k in ("dQ", "dK", "dV")), over


def test_lse_does_not_depend_on_the_ptilde_quantiser():
    """l sums P~ before quantisation, so even a two-level P~ quantiser leaves LSE at the exact
    logsumexp (float32), while O moves; l summed from the dequantised codes would move LSE."""
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 128, 16
    Q, K, V = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(3))
    spec = oq.Spec(N=N, d=d, blk=64, causal=True, qk_norm=False, k_smooth=False, dtype="f64")
    pro = oq.prologue(Q, K, V, spec, block_quant=oq.identity_block_quant)

    def two_level(x):
        x = np.asarray(x, np.float64)
        a = x.reshape(x.shape[0], -1).max(axis=1)
        return np.where(x >= 0.5 * a[:, None, None], 1.0, 0.0), a

    args = (pro["Qc"], pro["Kc"], pro["Vc"], pro["Qs"], pro["Ks"], pro["Vs"], spec)
    O_c, lse_c = oq.forward(*args, tile_quant=two_level)
    ex = exact.attention(Q, K, V, causal=True, qk_norm=False)
    np.testing.assert_allclose(lse_c, ex["LSE"], rtol=2e-7, atol=2e-7)
    assert np.linalg.norm(O_c - ex["O"]) > 0.1 * np.linalg.norm(ex["O"])


def test_spy_tile_shapes_and_counts():
    """The quantiser sees P~ tiles of fwd_tq x fwd_tk (one per visible query-tile / key-tile
    pair), then per visible backward pair one dS tile of bwd_tq x bwd_sk and bwd_sk/bwd_pk P
    tiles of bwd_tq x bwd_pk (causal, all dimensions distinct)."""
    rng = np.random.default_rng(6)
    B, H, N, d = 1, 2, 256, 16
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    spec = oq.Spec(N=N, d=d, blk=128, causal=True, qk_norm=True, k_smooth=True, fwd_tq=32, fwd_tk=64,
                   bwd_tq=64, bwd_pk=16, bwd_sk=32)
    seen = []

    def spy(x):
        seen.append(np.shape(x))
        return oq.int8_tile_quant(x)

    pro = oq.prologue(Q, K, V, spec)
    O, lse = oq.forward(pro["Qc"], pro["Kc"], pro["Vc"], pro["Qs"], pro["Ks"], pro["Vs"], spec, tile_quant=spy)
    fwd_pairs = sum(1 for it in range(N // 32) for jt in range(N // 64) if jt * 64 <= it * 32 + 31)
    assert seen == [(B * H, 32, 64)] * fwd_pairs
    seen.clear()
    oq.backward(pro, Q, K, V, O, lse, dO, spec, tile_quant=spy)
    bwd_pairs = sum(1 for it in range(N // 64) for jt in range(N // 32) if jt * 32 <= it * 64 + 63)
    assert seen == ([(B * H, 64, 32)] + [(B * H, 64, 16)] * 2) * bwd_pairs


def test_round_to_dtype_matches_torch():
    """The output rounding to bf16 and fp16 (nearest even) equals torch's float32 -> bf16 and
    float64 -> fp16 conversions, on random values across magnitudes, exact ties, subnormals
    and values that overflow to infinity."""
    import torch
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))
    ties_bf16 = (np.arange(1, 200, dtype=np.float64) * 2.0 ** -7 + 2.0 ** -8) * 2.0 ** rng.integers(-5, 5, 199)
    ties_fp16 = (1024 + np.arange(0, 200) + 0.5) * 2.0 ** -10
    big = np.array([3.39e38, -3.39e38, 65519.0, 65520.0, -65536.0, 1e-40, 6e-8, 3e-8])
    v = np.concatenate([x, ties_bf16, -ties_bf16, ties_fp16, big])
    bf = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oq.round_to_dtype(v, "bf16"), bf)
    # fp16: against torch's float32 -> fp16 on float32 values (torch's float64 -> fp16 goes
    # through float32, a second rounding; the oracle rounds float64 once)
    v32 = v.astype(np.float32)
    with np.errstate(over="ignore"):
        got = oq.round_to_dtype(v32.astype(np.float64), "fp16")
    fp = torch.from_numpy(v32).to(torch.float16).double().numpy()
    np.testing.assert_array_equal(got, fp)
    # one rounding of float64: 12219.9995 lies below the midpoint 12220 of the fp16 neighbours
    # 12216 and 12224, so it rounds down (rounding first to float32 gives 12220, a tie -> 12224)
    assert oq.round_to_dtype(np.array([12219.99951325]), "fp16")[0] == 12216.0
    # the bf16 branch rounds twice (float64 -> float32 -> bf16), as the kernels' float32
    # values are rounded once to bf16; it differs from one direct rounding only within 2^-24
    # relative of a bf16 tie. Here t lies just above the midpoint 1 + 2^-8 of the bf16
    # neighbours 1 and 1 + 2^-7 (a direct rounding gives 1 + 2^-7), but float32 puts it on the
    # midpoint and nearest-even then gives 1 (torch's float64 -> bf16 does the same)
    t = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert np.float32(t[0]) == 1.0 + 2.0 ** -8
    assert oq.round_to_dtype(t, "bf16")[0] == 1.0
    assert torch.from_numpy(t).to(torch.bfloat16).double().item() == 1.0
