"""Writes tile_placement_fixture.json: a hand-sized attention (4 tokens, d = 4, one 4-token
quantisation block) whose expected forward and backward outputs are derived here in exact
rational arithmetic, tile by tile, from the readings of where the in-kernel quantisers sit:

  forward : P~ is quantised on tiles of 2 query rows x 2 keys; the running max moves once per
            2-key tile; P~ = exp(s - running max); l sums P~ before quantisation
  backward: P = exp(s - LSE) is quantised on tiles of 2 query rows x 1 key (for dV), dS on
            tiles of 2 query rows x 2 keys (for dK and dQ)

with the per-block INT8 rule (scale absmax/127, nearest-even codes) on each tile. This script
imports nothing from the oracle or from the HIP path; the test runs the oracle on the same
inputs and compares, and runs it with other tile shapes, which must not match.

The inputs make every quantity rational: every block's absmax is 127 (scale 1, the codes are
the values), sm_scale = 2 ln 2, so exp(sm * S) = 4^S for the integer scores S, and the
softmax of a row is a ratio of powers of 4. Exact values stand in for the oracle's float32
scale rounding and float32 LSE (relative differences near 1e-7): the test compares with
rtol 1e-6 (forward) and 1e-5 (backward); other tilings move the outputs by 1e-3 and more.

Run: python tests/golden/make_tile_fixture.py  (rewrites the JSON next to this script)
"""
import json
import math
import os
from fractions import Fraction as F

N, D = 4, 4
# channel 2 of query 0 and channel 3 of key 0 carry the blocks' absmax (127) and meet only
# zeros on the other side, so the scores come from channels 0 and 1 alone
Q = [[1, 0, 127, 0], [0, 1, 0, 0], [-1, 0, 0, 0], [0, -1, 0, 0]]
K = [[2, 0, 0, 127], [1, 2, 0, 0], [0, 0, 0, 0], [1, 0, 0, 0]]
V = [[127 if i == j else 0 for j in range(D)] for i in range(N)]
dO = [[127, 0, 0, 0], [0, 0, 127, 0], [0, 127, 0, -127], [-127, 0, 127, 5]]
TQ, TK = 2, 2          # forward P~ tile
BTQ, BPK, BSK = 2, 1, 2  # backward P and dS tiles


def rne(x: F) -> int:
    """Nearest integer, ties to even; refuses values within 1e-4 of a tie (so the float32
    decisions of the oracle cannot differ)."""
    fl = math.floor(x)
    frac = x - fl
    assert abs(frac - F(1, 2)) > F(1, 10000), f"near tie {float(x)}"
    return fl + (1 if frac > F(1, 2) else 0)


def quant_tile(vals):
    """vals: dict (i, j) -> Fraction. INT8 rule on the tile: scale a/127, codes rne(x*127/a)."""
    a = max(abs(v) for v in vals.values())
    if a == 0:
        return {k: 0 for k in vals}, F(0)
    return {k: max(-127, min(127, rne(v * 127 / a))) for k, v in vals.items()}, a / 127


S = [[sum(Q[i][c] * K[j][c] for c in range(D)) for j in range(N)] for i in range(N)]
pow4 = lambda e: F(4) ** e

# ---------------------------------------------------------------- forward
O = [[F(0)] * D for _ in range(N)]
LSE_nat = [None] * N            # (m in units of S, l): LSE = sm * m + ln l
fwd_codes = {}
for it in range(N // TQ):
    rows = range(it * TQ, it * TQ + TQ)
    m = {i: None for i in rows}
    l = {i: F(0) for i in rows}
    acc = {i: [F(0)] * D for i in rows}
    for jt in range(N // TK):
        cols = range(jt * TK, jt * TK + TK)
        pt, alpha = {}, {}
        for i in rows:
            m_new = max(S[i][j] for j in cols) if m[i] is None else max(m[i], max(S[i][j] for j in cols))
            alpha[i] = F(0) if m[i] is None else pow4(m[i] - m_new)
            for j in cols:
                pt[(i, j)] = pow4(S[i][j] - m_new)
            m[i] = m_new
        codes, sP = quant_tile(pt)
        fwd_codes[f"q{it}k{jt}"] = [[codes[(i, j)] for j in cols] for i in rows]
        for i in rows:
            l[i] = l[i] * alpha[i] + sum(pt[(i, j)] for j in cols)
            acc[i] = [acc[i][c] * alpha[i] + sP * sum(codes[(i, j)] * V[j][c] for j in cols) for c in range(D)]
    for i in rows:
        O[i] = [acc[i][c] / l[i] for c in range(D)]
        LSE_nat[i] = (m[i], l[i])
sm = 2 * math.log(2)
LSE = [sm * mm + math.log(ll) for mm, ll in LSE_nat]

# ---------------------------------------------------------------- backward
# P = exp(s - LSE) is the row's softmax: 4^S / sum_j 4^S (exact)
P = [[pow4(S[i][j]) / sum(pow4(S[i][k]) for k in range(N)) for j in range(N)] for i in range(N)]
Dv = [sum(dO[i][c] * O[i][c] for c in range(D)) for i in range(N)]
dP = [[sum(dO[i][c] * V[j][c] for c in range(D)) for j in range(N)] for i in range(N)]
dS = [[P[i][j] * (dP[i][j] - Dv[i]) for j in range(N)] for i in range(N)]
dQ = [[F(0)] * D for _ in range(N)]
dK = [[F(0)] * D for _ in range(N)]
dV = [[F(0)] * D for _ in range(N)]
bwd_codes = {}
for it in range(N // BTQ):
    rows = range(it * BTQ, it * BTQ + BTQ)
    for jt in range(N // BSK):
        cols = range(jt * BSK, jt * BSK + BSK)
        dsc, sdS = quant_tile({(i, j): dS[i][j] for i in rows for j in cols})
        bwd_codes[f"dS_q{it}k{jt}"] = [[dsc[(i, j)] for j in cols] for i in rows]
        for p0 in range(jt * BSK, jt * BSK + BSK, BPK):
            pcols = range(p0, p0 + BPK)
            pc, sP = quant_tile({(i, j): P[i][j] for i in rows for j in pcols})
            bwd_codes[f"P_q{it}k{p0}"] = [[pc[(i, j)] for j in pcols] for i in rows]
            for j in pcols:
                for c in range(D):
                    dV[j][c] += sP * sum(pc[(i, j)] * dO[i][c] for i in rows)   # dO scale 1
        for j in cols:
            for c in range(D):
                dK[j][c] += sdS * sum(dsc[(i, j)] * Q[i][c] for i in rows)      # Q scale 1, x sm below
        for i in rows:
            for c in range(D):
                dQ[i][c] += sdS * sum(dsc[(i, j)] * K[j][c] for j in cols)      # K scale 1, x sm below


def fl(rows, scale=1.0):
    return [[float(v) * scale for v in r] for r in rows]


fixture = {
    "what": "Hand-sized attention whose forward and backward outputs are derived in exact rational "
            "arithmetic by tests/golden/make_tile_fixture.py (no oracle, no GPU code), to pin where "
            "the in-kernel quantisers sit: P~ on fwd_tq x fwd_tk = 2 x 2 tiles with the running max "
            "moving once per tile and l summing P~ before quantisation; P on bwd_tq x bwd_pk = 2 x 1 "
            "tiles; dS on bwd_tq x bwd_sk = 2 x 2 tiles (SageBwd article, per-block kernels paragraph "
            "and precision-split paragraph; the tile shapes are this build's reading of where the "
            "per-block rule applies inside the kernels).",
    "spec": {"N": N, "d": D, "blk": 4, "causal": False, "qk_norm": False, "k_smooth": False,
             "dtype": "f64", "sm_scale": sm, "fwd_tq": TQ, "fwd_tk": TK, "bwd_tq": BTQ, "bwd_pk": BPK,
             "bwd_sk": BSK},
    "inputs": {"Q": Q, "K": K, "V": V, "dO": dO},
    "derivation": {
        "scores_S": S,
        "note": "exp(sm*S) = 4^S. Query tile 0 (rows 0, 1): key tile 0 has P~ = [[1, 1/4], [1/16, 1]] "
                "(absmax 1: codes [[127, 32], [8, 127]]); key tile 1 keeps both running maxima, P~ = "
                "[[1/16, 1/4], [1/16, 1/16]] (absmax 1/4: codes [[32, 127], [32, 32]]); l = 25/16 and "
                "19/16. A per-row scale would give row 1 codes [127, 127] there; a 4-row tile would "
                "take row 2's P~ = 1 as the absmax (codes [[8, 32], [8, 8]]); l from the dequantised "
                "codes would give 795/508 instead of 25/16 for row 0. O = 127 * (dequantised P~) / l "
                "(V = 127 I): row 0 = [127, 32, 8, 31.75] * 16/25.",
        "forward_P~_codes": fwd_codes,
        "backward_codes": bwd_codes,
        "softmax_P": [[str(v) for v in r] for r in P],
        "D": [str(v) for v in Dv],
        "dS": [[str(v) for v in r] for r in dS],
    },
    "expected": {
        "O": fl(O),
        "LSE": LSE,
        "dQ": fl(dQ, sm),
        "dK": fl(dK, sm),
        "dV": fl(dV),
        "O_exact_fraction": [[str(v) for v in r] for r in O],
    },
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tile_placement_fixture.json")
with open(path, "w") as f:
    json.dump(fixture, f, indent=1)
print(f"wrote {path}")
