"""Pins for the oracle's dQ_code_step / dK_code_step: the largest move of a dQ (dK) row that one
unit of one of its dS codes can cause.

An implementation whose dS differs from the oracle's in the last float32 bits (another exp, LSE
or summation order) decides a code at a near-tie the other way; the parity tests allow such a
change per row through this bound. The bound is checked here against the thing it bounds: one
code of one dS tile is changed by one unit in the oracle itself (a wrapped tile quantiser,
P tiles left alone) and the rows of the recomputed gradients are measured.

- one tile, no QK-norm: the moved dQ row and dK row equal the bound exactly (the unit is put at
  the query and key of largest code-row norm), every other row stays put, dV does not move;
- one tile with QK-norm and K-smoothing, small inputs (rstd near 20): the moved rows stay within
  the bound and reach most of it (a missing or doubled rstd factor fails one side);
- many tiles (causal, blk 128 with 64-key dS tiles, gains, with and without Q-smoothing): units
  planted in several tiles stay within the bound of their rows.
"""
import numpy as np
import pytest

from oracle import quant as oq

F32 = np.float32


class _Flip:
    """The INT8 tile quantiser, with one code of the n-th dS tile moved by one unit (towards
    zero at +-127, so the code stays in range)."""

    def __init__(self, tile, h, i, j):
        self.tile, self.h, self.i, self.j = tile, h, i, j
        self.calls = 0

    def __call__(self, x):
        q, s = oq.int8_tile_quant(x)
        if self.calls == self.tile:
            q = q.copy()
            q[self.h, self.i, self.j] += 1.0 if q[self.h, self.i, self.j] < 127 else -1.0
        self.calls += 1
        return q, s


def _stages(Q, K, V, dO, spec, gains=(None, None)):
    pro = oq.prologue(Q, K, V, spec, q_gain=gains[0], k_gain=gains[1])
    O, LSE = oq.forward(pro["Qc"], pro["Kc"], pro["Vc"], pro["Qs"], pro["Ks"], pro["Vs"], spec,
                        kbias=pro["kbias"] if spec.q_smooth else None)

    def bwd(tile_quant):
        return oq.backward(pro, Q, K, V, O, LSE, dO, spec, tile_quant=tile_quant,
                           p_quant=oq.int8_tile_quant)
    return pro, bwd


def _visits(spec):
    """(query tile, key tile) in the order the backward visits them: ascending query tile, then
    ascending key tile up to the diagonal when causal."""
    out = []
    for it in range(spec.Np // spec.bwd_tq):
        for jt in range(spec.Np // spec.sk):
            if spec.causal and jt * spec.sk > it * spec.bwd_tq + spec.bwd_tq - 1:
                break
            out.append((it, jt))
    return out


def _inputs(seed, N, d, scale=1.0, q_offset=0.0):
    rng = np.random.default_rng(seed)
    Q, K, V, dO = (rng.standard_normal((1, 2, N, d)) for _ in range(4))
    Q = Q + q_offset * rng.standard_normal((1, 2, 1, d))
    return tuple((scale * x).astype(F32) for x in (Q, K)) + (V.astype(F32), dO.astype(F32))


def _row_moves(a, b):
    return np.linalg.norm(np.asarray(a, np.float64) - np.asarray(b, np.float64), axis=-1)


def test_single_tile_move_equals_bound():
    N, d = 64, 32
    Q, K, V, dO = _inputs(301, N, d)
    spec = oq.Spec(N=N, d=d, blk=64, causal=False, qk_norm=False, k_smooth=False, dtype="f64",
                   bwd_tq=64, bwd_sk=64)
    pro, bwd = _stages(Q, K, V, dO, spec)
    h = 1  # the second head, so a head mix-up moves the wrong rows
    i = int(np.argmax(np.linalg.norm(pro["Qc"][0, h].astype(np.float64), axis=-1)))
    j = int(np.argmax(np.linalg.norm(pro["Kc"][0, h].astype(np.float64), axis=-1)))
    clean = bwd(oq.int8_tile_quant)
    moved = bwd(_Flip(0, h, i, j))
    mq = _row_moves(moved["dQ"], clean["dQ"])[0]
    mk = _row_moves(moved["dK"], clean["dK"])[0]
    np.testing.assert_allclose(mq[h, i], clean["dQ_code_step"][0, h, i], rtol=1e-9)
    np.testing.assert_allclose(mk[h, j], clean["dK_code_step"][0, h, j], rtol=1e-9)
    mq[h, i] = mk[h, j] = 0.0
    assert mq.max() < 1e-12 and mk.max() < 1e-12
    assert np.array_equal(moved["dV"], clean["dV"])
    # one tile: every row of a head carries the same bound
    assert np.all(clean["dQ_code_step"][0, h] == clean["dQ_code_step"][0, h, 0])


def test_single_tile_with_qk_norm_within_and_near_bound():
    N, d = 64, 32
    Q, K, V, dO = _inputs(302, N, d, scale=0.05)
    spec = oq.Spec(N=N, d=d, blk=64, causal=False, qk_norm=True, k_smooth=True, dtype="f64",
                   bwd_tq=64, bwd_sk=64)
    pro, bwd = _stages(Q, K, V, dO, spec)
    assert np.min(pro["q_rstd"]) > 10 and np.min(pro["k_rstd"]) > 10
    h = 0
    i = int(np.argmax(np.linalg.norm(pro["Qc"][0, h].astype(np.float64), axis=-1)))
    j = int(np.argmax(np.linalg.norm(pro["Kc"][0, h].astype(np.float64), axis=-1)))
    clean = bwd(oq.int8_tile_quant)
    moved = bwd(_Flip(0, h, i, j))
    rq = _row_moves(moved["dQ"], clean["dQ"])[0, h, i] / clean["dQ_code_step"][0, h, i]
    rk = _row_moves(moved["dK"], clean["dK"])[0, h, j] / clean["dK_code_step"][0, h, j]
    # the RMSNorm backward removes only the component along the normalised token
    assert 0.8 < rq <= 1.0 + 1e-9, rq
    assert 0.8 < rk <= 1.0 + 1e-9, rk


@pytest.mark.parametrize("q_smooth", [False, True])
def test_many_tiles_moves_within_bound(q_smooth):
    N, d = 384, 32
    Q, K, V, dO = _inputs(303 + q_smooth, N, d, q_offset=3.0)
    rng = np.random.default_rng(305 + q_smooth)
    gains = tuple((1.0 + 0.4 * rng.standard_normal((2, d))).astype(F32) for _ in range(2))
    spec = oq.Spec(N=N, d=d, blk=128, causal=True, qk_norm=True, k_smooth=True, q_smooth=q_smooth,
                   dtype="f64", bwd_tq=128, bwd_sk=64)
    pro, bwd = _stages(Q, K, V, dO, spec, gains)
    clean = bwd(oq.int8_tile_quant)
    visits = _visits(spec)
    ratios = []
    for t in (0, 4, len(visits) - 1):
        it, jt = visits[t]
        h, i, j = int(rng.integers(2)), int(rng.integers(spec.bwd_tq)), int(rng.integers(spec.sk))
        moved = bwd(_Flip(t, h, i, j))
        qi, kj = it * spec.bwd_tq + i, jt * spec.sk + j
        rq = _row_moves(moved["dQ"], clean["dQ"])[0, h, qi] / clean["dQ_code_step"][0, h, qi]
        rk = _row_moves(moved["dK"], clean["dK"])[0, h, kj] / clean["dK_code_step"][0, h, kj]
        ratios.append((rq, rk))
        assert 0.0 < rq <= 1.0 + 1e-9, (t, rq)
        assert 0.0 < rk <= 1.0 + 1e-9, (t, rk)
    print(f"[code step] q_smooth={q_smooth}: move / bound per planted unit {ratios}")
