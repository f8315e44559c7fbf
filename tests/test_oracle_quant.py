"""Pins for the quantised oracle (oracle.quant) against things other than itself.

- hand-worked examples of the float32 prologue (exact values, rounding ties, the
  ascending summation order that bit-exactness depends on), stored as small text
  fixtures under tests/golden/ with the reasoning that gives each number,
- error bounds of the float32 steps against exact float64,
- the quantisation rule's closed-form properties,
- identity-quantiser reduction: with every quantisation replaced by the identity the
  tiled online-softmax forward and the tiled backward must equal oracle.exact,
- lossless-quantiser reduction: inputs built as code * 2^e per block quantise without
  loss, so with the real per-block rule (and identity tiles) the result must again
  equal oracle.exact; this pins which block scale multiplies which product,
- planted mistakes: a dropped or misplaced term in a copy of the oracle must break
  one of these pins.
"""
import json
import os

import numpy as np
import pytest

from oracle import exact
from oracle import quant as oq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- prologue

def test_rms_norm_hand_examples():
    g = _golden("prologue_hand_examples.json")
    for case in g["rms_norm"]:
        x = np.array(case["x"], dtype=F32)[None, :]
        xh, r = oq.rms_norm_f32(x, case["eps"])
        assert r[0] == F32(case["rstd"]), case
        np.testing.assert_array_equal(xh[0], np.array(case["xhat"], dtype=F32))


def test_rms_norm_chunk_tree_order():
    """d = 128, x = [4096, 1 x 127]: chunk 0 (channels 0..7) starts at 4096^2 = 2^24 and
    absorbs each of its seven 1s (2^24 + 1 rounds to even, 2^24); chunks 1..15 sum to 8.
    The pairwise tree then stays exact: 2^24 + 8, + 16, + 32, + 64 -> ss = 2^24 + 120,
    ms = 2^17 + 15/16 exactly. An ascending sum would give 2^24 and the exact sum
    2^24 + 127; both give a different float32 rstd."""
    x = np.ones((1, 128), dtype=F32)
    x[0, 0] = 4096.0
    _, r = oq.rms_norm_f32(x, 0.0)
    ms = F32(2.0 ** 17 + 15.0 / 16.0)
    assert r[0] == F32(1.0) / np.sqrt(ms)
    assert r[0] != F32(1.0) / np.sqrt(F32(2.0 ** 17))               # ascending order
    assert r[0] != F32(1.0 / np.sqrt((2.0 ** 24 + 127) / 128))       # exact sum


def test_rms_norm_small_d_tree():
    """d = 16 (one channel per chunk), x = [4096, 1 x 15]: the tree's first pair absorbs
    the 1 (2^24), the others pair to 2, then 2^24 + 2, + 4, + 8 -> ss = 2^24 + 14."""
    x = np.ones((1, 16), dtype=F32)
    x[0, 0] = 4096.0
    _, r = oq.rms_norm_f32(x, 0.0)
    assert r[0] == F32(1.0) / np.sqrt(F32((2.0 ** 24 + 14) / 16))


def test_rms_norm_error_bound():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 128)).astype(np.float16).astype(F32)
    x[:3] *= 100
    xh, r = oq.rms_norm_f32(x, 1e-6)
    r64 = 1.0 / np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=-1) + 1e-6)
    assert np.max(np.abs(r / r64 - 1)) < 4e-7      # a few float32 roundings
    assert np.max(np.abs(xh / (x * r64[:, None] + 1e-30) - 1)[x != 0]) < 6e-7


def test_k_smooth_hand_examples():
    g = _golden("prologue_hand_examples.json")
    for case in g["k_smooth"]:
        k = np.array(case["khat"], dtype=F32)[:, None]  # [N, 1]
        kt, mu = oq.k_smooth_f32(k, case["blk"])
        assert mu[0] == F32(case["mu"]), case
        np.testing.assert_array_equal(kt[:, 0], np.array(case["ktilde"], dtype=F32))


def test_k_smooth_group_tree_order():
    """One block of 32 tokens of one channel: token 0 = 2^24, tokens 1..31 = 1. Groups
    t mod 16: group 0 = 2^24 + 1 -> 2^24 (tie to even), groups 1..15 = 2. The tree then
    stays exact: 2^24 + 2, + 4, + 8, + 16 -> 2^24 + 30, so mu = (2^24 + 30) / 32 =
    2^19 + 15/16 exactly (an ascending sum would give 2^24 / 32 = 2^19)."""
    k = np.ones((32, 1), dtype=F32)
    k[0, 0] = 2.0 ** 24
    kt, mu = oq.k_smooth_f32(k, 32)
    assert mu[0] == F32(2.0 ** 19 + 15.0 / 16.0)
    assert kt[1, 0] == F32(1.0) - mu[0]


def test_k_smooth_mean_zero():
    rng = np.random.default_rng(1)
    kh = (rng.standard_normal((2, 512, 64)) + 5).astype(F32)
    kt, mu = oq.k_smooth_f32(kh, 64)
    np.testing.assert_allclose(mu, kh.astype(np.float64).mean(axis=1), rtol=2e-6)
    assert np.max(np.abs(kt.astype(np.float64).mean(axis=1))) < 1e-5


def test_quant_rule_hand_examples():
    g = _golden("prologue_hand_examples.json")
    for case in g["quant"]:
        x = np.array(case["x"], dtype=F32)[None]  # one block
        q, s = oq.quant_blocks_f32(x, x.shape[1])
        np.testing.assert_array_equal(q[0], np.array(case["codes"], dtype=np.int8))
        assert s[0] == F32(case["scale"]), case


def test_quant_rule_properties():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((3, 4, 256, 64)) * rng.uniform(1e-3, 1e3, (3, 4, 1, 1))).astype(F32)
    x[0, 0, :64] = 0.0                                  # an all-zero block
    x[0, 1, 64:128] = -np.abs(x[0, 1, 64:128])          # a block whose absmax is negative
    q, s = oq.quant_blocks_f32(x, 64)
    qb = q.reshape(3, 4, 4, 64, 64).astype(np.int32)
    xb = x.reshape(3, 4, 4, 64, 64).astype(np.float64)
    amax = np.max(np.abs(qb), axis=(-1, -2))
    assert s[0, 0, 0] == 0 and amax[0, 0, 0] == 0
    nz = s > 0
    assert np.all(amax[nz] == 127)                       # absmax element maps to +-127
    assert q.min() >= -127                               # never -128
    err = np.abs(xb - qb * s[..., None, None].astype(np.float64))
    assert np.all(err <= 0.5 * s[..., None, None] * (1 + 2e-5) + 1e-38)
    np.testing.assert_allclose(s[nz], (np.max(np.abs(xb), axis=(-1, -2)) / 127)[nz], rtol=6e-8)


def test_integer_products_exact():
    rng = np.random.default_rng(3)
    a = rng.integers(-127, 128, (64, 128))
    b = rng.integers(-127, 128, (64, 128))
    a[0] = 127; b[0] = 127
    assert np.array_equal(a @ b.T, (a.astype(np.float64) @ b.T.astype(np.float64)).astype(np.int64))
    assert np.max(np.abs(a @ b.T)) == 128 * 127 * 127 < 2 ** 24


# ----------------------------------------------------------------------------- reductions

def _exact_all(Q, K, V, dO, spec, **kw):
    return exact.attention(Q, K, V, dO, causal=spec.causal, qk_norm=spec.qk_norm, eps=spec.eps,
                           sm_scale=spec.scale, **kw)


def _rel(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tiles", [dict(blk=64, fwd_tq=32, bwd_tq=64, bwd_pk=32),
                                   dict(blk=128, fwd_tq=32, fwd_tk=64, bwd_tq=32, bwd_pk=16, bwd_sk=64)])
def test_identity_quant_equals_exact(causal, tiles):
    """All quantisers = identity, QK-norm and smoothing off: the tiled online-softmax
    forward and the tiled backward are exactly attention (to float64 rounding)."""
    rng = np.random.default_rng(4)
    B, H, N, d = 1, 2, 256, 16
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    spec = oq.Spec(N=N, d=d, causal=causal, qk_norm=False, k_smooth=False, dtype="f64", **tiles)
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant,
                 block_quant=oq.identity_block_quant)
    ref = _exact_all(Q, K, V, dO, spec)
    assert _rel(got["O"], ref["O"]) < 1e-12
    # LSE is stored as float32, and the backward reads it back, so P (and the gradients)
    # carry a relative error up to |LSE| * 2^-24.
    assert _rel(got["LSE"], ref["LSE"]) < 1e-7
    for name in ("dQ", "dK", "dV"):
        assert _rel(got[name], ref[name]) < 2e-6, name


@pytest.mark.parametrize("causal", [False, True])
def test_identity_quant_with_norm_and_smoothing(causal):
    """Identity quantisers with QK-norm and K-smoothing on: equal to exact attention up to
    the float32 prologue; smoothing changes nothing and needs no gradient correction."""
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 128, 32
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    K = (K + 4 * rng.standard_normal((1, H, 1, d))).astype(F32)
    spec = oq.Spec(N=N, d=d, blk=64, causal=causal, qk_norm=True, k_smooth=True, dtype="f64")
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant,
                 block_quant=oq.identity_block_quant)
    ref = _exact_all(Q, K, V, dO, spec)
    for name in ("O", "dQ", "dK", "dV"):
        assert _rel(got[name], ref[name]) < 3e-6, name


def _lossless(rng, shape, blk, emin=-6, emax=3):
    """Values code * 2^e with one exponent per block and one element at +-127 per block."""
    B, H, N, d = shape
    codes = rng.integers(-127, 128, shape).astype(np.float64)
    codes.reshape(B, H, N // blk, blk * d)[..., 0] = 127.0 * rng.choice([-1, 1], (B, H, N // blk))
    e = rng.integers(emin, emax + 1, (B, H, N // blk))
    x = codes * np.repeat(np.exp2(e.astype(np.float64)), blk, axis=-1)[..., None]
    return x.astype(F32), e


@pytest.mark.parametrize("causal", [False, True])
def test_lossless_block_quant_equals_exact(causal):
    """Per-block exponents differ, so a scale applied to the wrong block breaks this."""
    rng = np.random.default_rng(6)
    shape = (1, 2, 256, 16)
    blk = 64
    Q, eq = _lossless(rng, shape, blk, -7, -5)
    K, ek = _lossless(rng, shape, blk, -7, -5)
    V, ev = _lossless(rng, shape, blk)
    dO, ed = _lossless(rng, shape, blk)
    spec = oq.Spec(N=256, d=16, blk=blk, causal=causal, qk_norm=False, k_smooth=False, dtype="f64")
    pro = oq.prologue(Q, K, V, spec)
    np.testing.assert_array_equal(pro["Qs"], np.exp2(eq).astype(F32))
    np.testing.assert_array_equal(pro["Vs"], np.exp2(ev).astype(F32))
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant)
    np.testing.assert_array_equal(got["dOs"], np.exp2(ed).astype(F32))
    ref = _exact_all(Q, K, V, dO, spec)
    assert _rel(got["O"], ref["O"]) < 1e-12
    # LSE is stored as float32, and the backward reads it back, so P (and the gradients)
    # carry a relative error up to |LSE| * 2^-24.
    assert _rel(got["LSE"], ref["LSE"]) < 1e-7
    for name in ("dQ", "dK", "dV"):
        assert _rel(got[name], ref[name]) < 2e-6, name


@pytest.mark.parametrize("causal", [False, True])
def test_int8_close_to_exact(causal):
    """The real INT8 path stays close to exact attention (a gross indexing error would not)."""
    rng = np.random.default_rng(7)
    B, H, N, d = 1, 2, 256, 64
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(np.float16).astype(F32) for _ in range(4))
    spec = oq.Spec(N=N, d=d, blk=64, causal=causal, qk_norm=True, k_smooth=True, dtype="f64")
    got = oq.run(Q, K, V, dO, spec)
    ref = _exact_all(Q, K, V, dO, spec)

    def cos(a, b):
        a = a.ravel(); b = b.ravel()
        return a @ b / np.linalg.norm(a) / np.linalg.norm(b)
    assert cos(got["O"], ref["O"]) > 0.999
    for name in ("dQ", "dK", "dV"):
        assert cos(got[name], ref[name]) > 0.99, name


def test_sampled_tiles_match_full():
    """Restricting the oracle to some query/key tiles gives the same values there."""
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 1, 256, 32
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(np.float16).astype(F32) for _ in range(4))
    spec = oq.Spec(N=N, d=d, blk=64, causal=True, qk_norm=True, k_smooth=True, dtype="fp16")
    full = oq.run(Q, K, V, dO, spec)
    pro = oq.prologue(Q, K, V, spec)
    O, L = oq.forward(pro["Qc"], pro["Kc"], pro["Vc"], pro["Qs"], pro["Ks"], pro["Vs"], spec, q_tiles=[1, 6])
    for it in (1, 6):
        sl = slice(it * 32, it * 32 + 32)
        np.testing.assert_array_equal(O[..., sl, :], full["O"][..., sl, :])
        np.testing.assert_array_equal(L[..., sl], full["LSE"][..., sl])
    g = oq.backward(pro, Q, K, V, full["O"], full["LSE"], dO, spec, q_tiles=[2], k_tiles=[1])
    np.testing.assert_allclose(g["dQ"][..., 128:192, :], full["dQ"][..., 128:192, :], rtol=0, atol=0)
    np.testing.assert_allclose(g["dK"][..., 64:128, :], full["dK"][..., 64:128, :], rtol=0, atol=0)
    np.testing.assert_allclose(g["dV"][..., 64:128, :], full["dV"][..., 64:128, :], rtol=0, atol=0)


# ----------------------------------------------------------------------------- planted mistakes

def _identity_case(causal=True):
    rng = np.random.default_rng(9)
    Q, K, V, dO = (rng.standard_normal((1, 1, 128, 16)).astype(F32) for _ in range(4))
    spec = oq.Spec(N=128, d=16, blk=64, causal=causal, qk_norm=True, k_smooth=False, dtype="f64")
    return Q, K, V, dO, spec


def _identity_pin_passes(Q, K, V, dO, spec):
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant,
                 block_quant=oq.identity_block_quant)
    ref = _exact_all(Q, K, V, dO, spec)
    return all(_rel(got[n], ref[n]) < 3e-6 for n in ("O", "dQ", "dK", "dV"))


def test_pins_pass_unplanted():
    assert _identity_pin_passes(*_identity_case())


@pytest.mark.parametrize("mistake", ["rmsnorm_bwd_drop_mean", "rmsnorm_bwd_sign",
                                     "ds_drop_D", "dk_transposed", "tile_scale_dropped"])
def test_planted_mistake_is_caught(monkeypatch, mistake):
    if mistake == "rmsnorm_bwd_drop_mean":
        monkeypatch.setattr(oq, "rms_norm_backward",
                            lambda dy, y, r: np.asarray(r)[..., None] * np.asarray(dy))
    elif mistake == "rmsnorm_bwd_sign":
        monkeypatch.setattr(oq, "rms_norm_backward",
                            lambda dy, y, r: np.asarray(r)[..., None] * (dy + y * np.mean(dy * y, -1, keepdims=True)))
    elif mistake == "tile_scale_dropped":
        Q, K, V, dO, spec = _identity_case()
        got = oq.run(Q, K, V, dO, spec, tile_quant=lambda x: (np.asarray(x, np.float64) / 2, np.ones(np.shape(x)[0])),
                     block_quant=oq.identity_block_quant)
        ref = _exact_all(Q, K, V, dO, spec)
        assert not all(_rel(got[n], ref[n]) < 3e-6 for n in ("O", "dQ", "dK", "dV"))
        return
    elif mistake == "ds_drop_D":
        real_bp = oq.backward_pre
        monkeypatch.setattr(oq, "backward_pre",
                            lambda O, dO, spec, block_quant=oq.quant_blocks_f32: (
                                0 * real_bp(O, dO, spec, block_quant)[0],) + tuple(real_bp(O, dO, spec, block_quant)[1:]))
    elif mistake == "dk_transposed":
        real_tq = oq.identity_tile_quant

        def tq_T(x):
            x = np.asarray(x, np.float64)
            if x.shape[-1] == x.shape[-2] and x.shape[-1] == 64:  # dS tiles: swap axes
                return x.transpose(0, 2, 1), np.ones(x.shape[0])
            return real_tq(x)
        Q, K, V, dO, spec = _identity_case()
        spec = oq.Spec(N=128, d=16, blk=64, causal=False, qk_norm=True, k_smooth=False, dtype="f64")
        got = oq.run(Q, K, V, dO, spec, tile_quant=tq_T, block_quant=oq.identity_block_quant)
        ref = _exact_all(Q, K, V, dO, spec)
        assert not all(_rel(got[n], ref[n]) < 3e-6 for n in ("dQ", "dK"))
        return
    assert not _identity_pin_passes(*_identity_case())


# ----------------------------------------------------------------------------- Q-smoothing

def _qs_case(seed, N=128, d=32, causal=True):
    rng = np.random.default_rng(seed)
    B, H = 1, 2
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    # a strong per-channel query offset, so mu_Q (and every term it enters) is large
    Q = (Q + 3 * rng.standard_normal((1, H, 1, d))).astype(F32)
    K = (K + 2 * rng.standard_normal((1, H, 1, d))).astype(F32)
    return Q, K, V, dO


@pytest.mark.parametrize("causal", [False, True])
def test_identity_quant_with_q_smoothing(causal):
    """With identity quantisers, Q~ K^T + 1 (K mu_Q)^T is Q^ K^T and dS^T Q~ + (dS^T 1) mu_Q^T
    is dS^T Q^: the Q-smoothed path equals exact attention (to the float32 prologue's
    rounding). A dropped or mis-signed bias term, or mu_Q over the wrong axis, breaks it."""
    Q, K, V, dO = _qs_case(11, causal=causal)
    spec = oq.Spec(N=128, d=32, blk=64, causal=causal, qk_norm=True, k_smooth=True, q_smooth=True, dtype="f64")
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant, block_quant=oq.identity_block_quant)
    ref = _exact_all(Q, K, V, dO, spec)
    for name in ("O", "dQ", "dK", "dV"):
        assert _rel(got[name], ref[name]) < 3e-6, name
    # the bias is not negligible here: without it the scores would be far off
    assert np.max(np.abs(got["kbias"])) > 0.5


def test_q_smooth_removes_query_mean():
    Q, K, V, dO = _qs_case(12)
    spec = oq.Spec(N=128, d=32, blk=64, causal=True, qk_norm=True, k_smooth=True, q_smooth=True, dtype="f64")
    pro = oq.prologue(Q, K, V, spec, block_quant=oq.identity_block_quant)
    qt = pro["Qc"].astype(np.float64)          # identity "codes" = Q~
    assert np.max(np.abs(qt.mean(axis=-2))) < 1e-6 * np.max(np.abs(qt))
    np.testing.assert_allclose(pro["q_mean"], pro["Qhat"].astype(np.float64).mean(axis=-2), rtol=1e-5, atol=1e-6)
    # off: the mean is zero and the keys carry no bias
    off = oq.prologue(Q, K, V, oq.Spec(N=128, d=32, blk=64, causal=True, qk_norm=True, k_smooth=True, dtype="f64"))
    assert not np.any(off["q_mean"]) and not np.any(off["kbias"])


@pytest.mark.parametrize("causal", [False, True])
def test_int8_q_smoothing_close_to_exact(causal):
    Q, K, V, dO = _qs_case(13, N=256, d=64, causal=causal)
    Q, K, V, dO = (x.astype(np.float16).astype(F32) for x in (Q, K, V, dO))
    spec = oq.Spec(N=256, d=64, blk=64, causal=causal, qk_norm=True, k_smooth=True, q_smooth=True, dtype="f64")
    got = oq.run(Q, K, V, dO, spec)
    ref = _exact_all(Q, K, V, dO, spec)

    def cos(a, b):
        a = a.ravel(); b = b.ravel()
        return a @ b / np.linalg.norm(a) / np.linalg.norm(b)
    assert cos(got["O"], ref["O"]) > 0.999
    for name in ("dQ", "dK", "dV"):
        assert cos(got[name], ref[name]) > 0.99, name


@pytest.mark.parametrize("mistake", ["qs_drop_kbias", "qs_drop_dk_bias", "qs_dk_bias_sign"])
def test_q_smoothing_planted_mistake_is_caught(monkeypatch, mistake):
    if mistake == "qs_drop_kbias":
        monkeypatch.setattr(oq, "key_bias", lambda Kc, Ks, mu_q, blk: np.zeros(np.shape(Kc)[:-1]))
    elif mistake == "qs_drop_dk_bias":
        monkeypatch.setattr(oq, "q_smooth_dk_bias", lambda qdS, sdS, mu_q, sm: 0.0)
    else:
        real = oq.q_smooth_dk_bias
        monkeypatch.setattr(oq, "q_smooth_dk_bias", lambda qdS, sdS, mu_q, sm: -real(qdS, sdS, mu_q, sm))
    Q, K, V, dO = _qs_case(11)
    spec = oq.Spec(N=128, d=32, blk=64, causal=True, qk_norm=True, k_smooth=True, q_smooth=True, dtype="f64")
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant, block_quant=oq.identity_block_quant)
    ref = _exact_all(Q, K, V, dO, spec)
    assert not all(_rel(got[n], ref[n]) < 3e-6 for n in ("O", "dQ", "dK", "dV"))


# ----------------------------------------------------------------- learnable QK-norm gains

def _gain_case(seed, causal=True, N=128, d=32):
    rng = np.random.default_rng(seed)
    B, H = 2, 2
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    gq = (1.0 + 0.4 * rng.standard_normal((H, d))).astype(F32)
    gk = (1.0 + 0.4 * rng.standard_normal((H, d))).astype(F32)
    spec = oq.Spec(N=N, d=d, blk=64, causal=causal, qk_norm=True, k_smooth=True, dtype="f64")
    return Q, K, V, dO, gq, gk, spec


@pytest.mark.parametrize("causal", [False, True])
def test_identity_quant_with_gains(causal):
    """Identity quantisers with learnable QK-norm gains: equal to exact attention with the same
    gains (O, dQ, dK, dV and both gain gradients), up to the float32 prologue."""
    Q, K, V, dO, gq, gk, spec = _gain_case(81 + causal, causal)
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant, block_quant=oq.identity_block_quant,
                 q_gain=gq, k_gain=gk)
    ref = exact.attention(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64),
                          dO.astype(np.float64), causal=causal, qk_norm=True, eps=spec.eps,
                          q_gain=gq.astype(np.float64), k_gain=gk.astype(np.float64))
    for name in ("O", "dQ", "dK", "dV", "dq_gain", "dk_gain"):
        assert _rel(got[name], ref[name]) < 3e-6, name


def test_gain_prologue_power_of_two_exact():
    """A power-of-two gain scales the normalised values exactly, so every code is unchanged
    and every block scale of Q and K is multiplied by exactly that power (K-smoothing
    commutes with it: the mean scales by the same power)."""
    Q, K, V, dO, _, _, spec = _gain_case(91)
    H, d = Q.shape[1], Q.shape[3]
    rng = np.random.default_rng(92)
    e = rng.integers(-3, 4, size=H)                     # one power per head, all channels
    g = np.repeat(np.exp2(e.astype(np.float64))[:, None], d, axis=1).astype(F32)
    a = oq.prologue(Q, K, V, spec)
    b = oq.prologue(Q, K, V, spec, q_gain=g, k_gain=g)
    for k in ("Qc", "Kc", "Vc", "Vs", "q_rstd", "k_rstd"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    f = np.exp2(e.astype(np.float64))[None, :, None]
    np.testing.assert_array_equal(b["Qs"], (a["Qs"] * f).astype(F32))
    np.testing.assert_array_equal(b["Ks"], (a["Ks"] * f).astype(F32))


def test_unit_gain_equals_no_gain():
    Q, K, V, dO, gq, gk, spec = _gain_case(93)
    ones = np.ones_like(gq)
    a = oq.run(Q, K, V, dO, spec)
    b = oq.run(Q, K, V, dO, spec, q_gain=ones, k_gain=ones)
    for k in ("Qc", "Kc", "Qs", "Ks", "O", "dQ", "dK", "dV"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_gain_planted_mistake_is_caught(monkeypatch):
    """Dropping the gain from the RMSNorm backward (dn = dX^ instead of g o dX^) breaks the
    identity-quantiser pin."""
    Q, K, V, dO, gq, gk, spec = _gain_case(94)
    real = oq.rms_norm_backward
    calls = []

    def no_gain(dy, y, r):
        calls.append(1)
        return real(dy / np.broadcast_to(np.asarray(gq, np.float64), (Q.shape[0],) + gq.shape).reshape(-1, 1, gq.shape[-1])
                    if len(calls) == 1 else dy, y, r)
    monkeypatch.setattr(oq, "rms_norm_backward", no_gain)
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant, block_quant=oq.identity_block_quant,
                 q_gain=gq, k_gain=gk)
    ref = exact.attention(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64),
                          dO.astype(np.float64), causal=True, qk_norm=True, eps=spec.eps,
                          q_gain=gq.astype(np.float64), k_gain=gk.astype(np.float64))
    assert _rel(got["dQ"], ref["dQ"]) > 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_identity_quant_normed_grads(causal):
    """normed_grads with identity quantisers: the gradients with respect to Q^, K^ of exact
    attention (and the RMSNorm backward of them is the default output)."""
    rng = np.random.default_rng(111 + causal)
    B, H, N, d = 1, 2, 128, 32
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    spec = oq.Spec(N=N, d=d, blk=64, causal=causal, qk_norm=True, k_smooth=True, dtype="f64", normed_grads=True)
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant, block_quant=oq.identity_block_quant)
    ref = exact.attention(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), dO.astype(np.float64),
                          causal=causal, qk_norm=True, eps=spec.eps, normed_grads=True)
    for name in ("O", "dQ", "dK", "dV"):
        assert _rel(got[name], ref[name]) < 3e-6, name
    full = oq.run(Q, K, V, dO, oq.Spec(N=N, d=d, blk=64, causal=causal, qk_norm=True, k_smooth=True, dtype="f64"),
                  tile_quant=oq.identity_tile_quant, block_quant=oq.identity_block_quant)
    assert _rel(got["dQ"], full["dQ"]) > 1e-2     # the RMSNorm backward does change dQ


# ------------------------------------------------------------------- ragged N (N % blk != 0)

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,blk,tiles", [(100, 64, {}), (200, 128, dict(fwd_tk=64, bwd_tq=64, bwd_sk=64)),
                                         (65, 64, {})])
def test_identity_quant_ragged_n(causal, N, blk, tiles):
    """A last block holding N mod blk tokens: with identity quantisers the tiled path equals
    exact attention on the N tokens (the padding keys are masked, the padding queries take no
    part), with QK-norm and K-smoothing on."""
    rng = np.random.default_rng(121 + N + causal)
    B, H, d = 1, 2, 32
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    K = (K + 3 * rng.standard_normal((1, H, 1, d))).astype(F32)
    spec = oq.Spec(N=N, d=d, blk=blk, causal=causal, qk_norm=True, k_smooth=True, dtype="f64", **tiles)
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant, block_quant=oq.identity_block_quant)
    ref = _exact_all(Q, K, V, dO, spec)
    for name in ("O", "dQ", "dK", "dV"):
        assert got[name].shape == (B, H, N, d), name
        assert _rel(got[name], ref[name]) < 3e-6, name
    assert got["Qc"].shape == (B, H, spec.Np, d)


def test_ragged_block_quant_is_the_rule_on_valid_tokens():
    """The ragged last block's codes and scale are the INT8 rule over its valid tokens alone;
    the padding rows hold code 0; the K mean is over the N tokens and leaves the padding 0."""
    rng = np.random.default_rng(131)
    B, H, N, d, blk = 1, 2, 150, 16, 64
    Q, K, V = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(3))
    spec = oq.Spec(N=N, d=d, blk=blk, causal=True, qk_norm=True, k_smooth=True)
    pro = oq.prologue(Q, K, V, spec)
    Np = spec.Np
    assert Np == 192
    last = slice(128, N)
    qv, sv = oq.quant_rule_f32(V[:, :, last, :], axes=(2, 3))
    np.testing.assert_array_equal(pro["Vc"][:, :, last, :], qv)
    np.testing.assert_array_equal(pro["Vs"][:, :, 2], sv)
    assert not np.any(pro["Vc"][:, :, N:, :]) and not np.any(pro["Kc"][:, :, N:, :]) and not np.any(pro["Qc"][:, :, N:, :])
    kt = pro["Kc"].astype(np.float64) * np.repeat(pro["Ks"], blk, axis=-1)[..., None]
    # the smoothed keys average to ~0 over the valid tokens (up to the INT8 rounding)
    assert np.max(np.abs(kt[:, :, :N].mean(axis=2))) < 0.02
    kh = oq.rms_norm_f32(K, spec.eps)[0].astype(np.float64)
    assert np.allclose(pro["k_mean"], kh.mean(axis=2), atol=1e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_eps_zero(causal):
    """eps = 0 with a ragged last block: the zero padding tokens are not normalised (rstd 1,
    values 0), so no 0 * inf = NaN reaches the block sums, the K mean or any code; the
    identity-quantiser path still equals exact attention (eps = 0) on the N real tokens, and
    the INT8 path stays finite with the padding codes 0."""
    rng = np.random.default_rng(141 + causal)
    B, H, N, d, blk = 1, 2, 100, 32, 64
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(F32) for _ in range(4))
    K = (K + 2 * rng.standard_normal((1, H, 1, d))).astype(F32)
    spec = oq.Spec(N=N, d=d, blk=blk, causal=causal, qk_norm=True, k_smooth=True, dtype="f64", eps=0.0)
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant, block_quant=oq.identity_block_quant)
    ref = _exact_all(Q, K, V, dO, spec)
    for name in ("O", "dQ", "dK", "dV"):
        assert _rel(got[name], ref[name]) < 3e-6, name
    q = oq.run(Q, K, V, dO, oq.Spec(N=N, d=d, blk=blk, causal=causal, qk_norm=True, k_smooth=True, eps=0.0))
    for name in ("k_mean", "q_rstd", "k_rstd", "Qs", "Ks", "O", "dQ", "dK", "dV"):
        assert np.all(np.isfinite(q[name])), name
    assert np.all(q["q_rstd"][..., N:] == 1) and np.all(q["k_rstd"][..., N:] == 1)
    assert not np.any(q["Kc"][..., N:, :]) and not np.any(q["Qc"][..., N:, :])
    assert np.any(q["Kc"][..., :N, :])


# ------------------------------------------------------------------- FP8 (e4m3) recipe

def test_e4m3_matches_torch_conversion():
    """The oracle's own e4m3 encoding (written from the format's definition) equals torch's
    float8_e4m3fn conversion (round to nearest even) on every representable value, every
    midpoint between neighbours and random values across the whole range."""
    torch = pytest.importorskip("torch")
    vals = oq.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.unique(vals[np.isfinite(vals)])
    mids = (fin[:-1] + fin[1:]) / 2
    rng = np.random.default_rng(141)
    rnd = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-16, 1, 20000))
    x = np.concatenate([fin, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), rnd]).astype(F32)
    x = x[np.abs(x) <= 448]
    mine = oq.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch writes -0 for negative values rounding to zero, as the oracle does
    assert np.array_equal(mine, ref), int(np.sum(mine != ref))


def test_e4m3_round_trip_and_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # all but NaN
    assert np.array_equal(oq.e4m3_encode(oq.e4m3_decode(codes).astype(F32)), codes)
    assert oq.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert oq.e4m3_decode(np.array([0x01], np.uint8))[0] == 2.0 ** -9
    # ties go to the even mantissa: 17 -> 16, 19 -> 20, 2^-10 (half the smallest subnormal) -> 0
    got = oq.e4m3_decode(oq.e4m3_encode(np.array([17.0, 19.0, 2.0 ** -10, 3 * 2.0 ** -10], F32)))
    np.testing.assert_array_equal(got, [16.0, 20.0, 0.0, 2.0 ** -8])
    # an ulp above 448 (x * fl(448 / a) can land there) still rounds to 448; 464 is refused
    just_above = np.nextafter(F32(448.0), F32(np.inf))
    assert oq.e4m3_encode(np.array([just_above, -just_above], F32)).tolist() == [0x7E, 0xFE]
    with pytest.raises(ValueError):
        oq.e4m3_encode(np.array([464.0], F32))
    # signed zeros
    assert oq.e4m3_encode(np.array([0.0, -0.0], F32)).tolist() == [0x00, 0x80]


def test_fp8_rule_properties():
    """Every non-zero block has a code of magnitude 448 (the absmax element); each value is
    within half a step of the code's value times the scale."""
    rng = np.random.default_rng(143)
    x = (rng.standard_normal((2, 3, 256, 16)) * np.exp2(rng.integers(-8, 8, (2, 3, 1, 1)))).astype(F32)
    q, s = oq.quant_blocks_fp8_f32(x, 64)
    v = oq.e4m3_decode(q).reshape(2, 3, 4, 64, 16)
    assert np.all(np.max(np.abs(v), axis=(-2, -1)) == 448.0)
    deq = v * s[..., None, None]
    xb = x.reshape(2, 3, 4, 64, 16).astype(np.float64)
    # relative step of e4m3 is 2^-3 for normals; subnormals have an absolute step 2^-9 * s
    err = np.abs(deq - xb)
    bound = np.maximum(np.abs(xb) * 2.0 ** -4, 2.0 ** -10 * s[..., None, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_lossless_block_quant_equals_exact(causal):
    """Inputs that the FP8 rule represents exactly (e4m3 values times a per-block power of two,
    each block holding a +-448 element), identity tiles: the FP8 path equals exact attention,
    which pins the decode of the codes and which block scale multiplies which product."""
    rng = np.random.default_rng(145)
    shape, blk = (1, 2, 256, 16), 64
    vals = oq.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]

    def lossless(emin, emax):
        B, H, N, d = shape
        c = rng.choice(fin, size=shape)
        c.reshape(B, H, N // blk, blk * d)[..., 0] = 448.0 * rng.choice([-1, 1], (B, H, N // blk))
        e = rng.integers(emin, emax + 1, (B, H, N // blk))
        return (c * np.repeat(np.exp2(e.astype(np.float64)), blk, axis=-1)[..., None]).astype(F32), e
    Q, eq = lossless(-12, -10)
    K, _ = lossless(-12, -10)
    V, ev = lossless(-9, -6)
    dO, _ = lossless(-9, -6)
    spec = oq.Spec(N=256, d=16, blk=blk, causal=causal, qk_norm=False, k_smooth=False, dtype="f64", fmt="fp8")
    pro = oq.prologue(Q, K, V, spec, block_quant=oq.quant_blocks_fp8_f32)
    np.testing.assert_array_equal(pro["Qs"], np.exp2(eq).astype(F32))
    np.testing.assert_array_equal(pro["Vs"], np.exp2(ev).astype(F32))
    got = oq.run(Q, K, V, dO, spec, tile_quant=oq.identity_tile_quant)
    ref = _exact_all(Q, K, V, dO, spec)
    assert _rel(got["O"], ref["O"]) < 1e-12
    for name in ("dQ", "dK", "dV"):
        assert _rel(got[name], ref[name]) < 2e-6, name


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_close_to_exact(causal):
    """The FP8 recipe end to end stays close to exact attention (3 mantissa bits: looser than
    INT8's, still far from what an indexing error would give)."""
    rng = np.random.default_rng(147)
    B, H, N, d = 1, 2, 256, 64
    Q, K, V, dO = (rng.standard_normal((B, H, N, d)).astype(np.float16).astype(F32) for _ in range(4))
    spec = oq.Spec(N=N, d=d, blk=64, causal=causal, qk_norm=True, k_smooth=True, dtype="f64", fmt="fp8")
    got = oq.run(Q, K, V, dO, spec)
    assert got["Qc"].dtype == np.uint8
    ref = _exact_all(Q, K, V, dO, spec)

    def cos(a, b):
        a = a.ravel(); b = b.ravel()
        return a @ b / np.linalg.norm(a) / np.linalg.norm(b)
    assert cos(got["O"], ref["O"]) > 0.995
    for name in ("dQ", "dK", "dV"):
        assert cos(got[name], ref[name]) > 0.98, name
