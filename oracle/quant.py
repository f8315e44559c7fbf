"""O-Q: the quantised SageBwd-style attention, written plainly (CPU, numpy).

Test infrastructure only (see oracle/__init__.py).

What is computed, in the order of the SageBwd article:
  1. QK-norm: RMSNorm of every token vector of Q and of K over the head dimension,
     times an optional learnable gain g [H, d] per head and channel (1 when absent;
     SageBwd article, QK-norm paragraph); the backward also returns the gains' gradients.
  2. K-smoothing: subtract from every key the mean key of its head, i.e. the
     per-channel mean over all N tokens, right before quantising (SageBwd article,
     K-smoothing paragraph; the axis follows from the Q-smoothing paragraph, whose
     bias term (dS^T 1) mu_Q^T needs mu to be a d-vector averaged over tokens).
  3. Per-block INT8 quantisation of Q^, K~, V (and dO in the backward): one float32
     scale per block of `blk` tokens x d channels, symmetric absmax/127, codes in
     [-127, 127], round to nearest even (SageBwd article, per-block kernels
     paragraph).
  4. A flash-style forward (TurboQuant blog, FlashAttention section: the T x T score
     matrix is processed block by block) whose QK^T and PV products are INT8 (SageBwd
     article, precision split paragraph). P~ is quantised on tiles of fwd_tq query
     rows x fwd_tk keys.
  5. The backward with recomputed QK^T, dP = dO V^T from the 16-bit dO and V,
     dS = P o (dP - D), and INT8 products dV = P^T dO, dK = dS^T Q, dQ = dS K (SageBwd
     article, precision split and gradient paragraphs). P is quantised on tiles of
     bwd_tq x bwd_pk, dS on tiles of bwd_tq x bwd_sk.
  6. Gradients are with respect to the raw Q, K handed to the prologue: the RMSNorm
     backward closes dQ and dK; K-smoothing contributes nothing, because every row of
     dS sums to zero.
  7. Optional Q-smoothing (Spec.q_smooth; SageBwd article, Q-smoothing paragraph, which
     names its bias term): the queries' per-channel mean mu_Q (taken like the keys') is
     subtracted before quantising; every score gets back the per-key bias
     b_k = (K mu_Q)_k (key_bias), and dK^ gets dK_bias = (dS^T 1) mu_Q^T
     (q_smooth_dk_bias); dQ is unchanged.
  8. Optional FP8 recipe (Spec.fmt = "fp8"). The SageBwd article's precision split names
     only INT8 and FP16; FP8 is named by the Full-Stack FP4 page (section 1, problem
     definition: attention is commonly kept in BF16 or FP8) and by the NVFP4 / Quartet 2
     page (block-scaled FP8 training; E4M3 as an FP8 format). The recipe keeps the
     article's split and swaps the format: every quantiser of steps 3-5 keeps its tile and
     its absmax rule but maps onto e4m3 (OCP float8 e4m3fn, largest finite 448) instead of
     [-127, 127]: scale a / 448, code e4m3_rne(x * 448 / a). The products are formed from
     the codes' values exactly as in the INT8 recipe.

  9. Optional Q-Attn precision split (Spec.split = "qattn"; Full-Stack FP4 page, section
     2.4, mixed-precision attention): the robust paths, QK^T (forward and recomputed) and
     the dS products dQ = dS K, dK = dS^T Q, stay low-bit (the codes of spec.fmt); the
     softmax-sensitive paths PV, P^T dO and dO V^T run in 16 bits: P~ and P are rounded to
     the inputs' 16-bit type (half_round_tile), and V and dO enter with their own 16-bit
     values (identity_block_quant), with float accumulation. The quantised views of Q and K
     are reused by both passes as before.

Precision: steps 1-3 are float32, one IEEE operation at a time, round to nearest
even, in the order written (sums run over channels, or over tokens, in ascending
index order). Everything after the prologue is float64, except that each in-kernel
quantisation (P~, P, dS) takes its decision in float32 exactly as in step 3 (the
value is rounded to float32 first), so the oracle and the kernels decide codes in
the same precision. Outputs are rounded to the 16-bit dtype, nearest even.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

F32 = np.float32


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape, flags and quantisation tiling of one attention call.

    fwd_tq x fwd_tk : tile on which P~ is quantised in the forward; fwd_tk is also
                      the online-softmax step (the running max moves once per tile).
    bwd_tq x bwd_pk : tile on which P is quantised in the backward (for dV).
    bwd_tq x bwd_sk : tile on which dS is quantised (for dK and dQ).
    Every tile lies inside one blk x blk block, so the block scales of Q, K, V and dO
    factor out of every integer product.
    """
    N: int
    d: int
    blk: int
    causal: bool
    qk_norm: bool
    k_smooth: bool
    dtype: str = "fp16"
    eps: float = 1e-6
    sm_scale: Optional[float] = None
    fwd_tq: int = 32
    fwd_tk: Optional[int] = None
    bwd_tq: int = 64
    bwd_pk: int = 16
    bwd_sk: Optional[int] = None
    q_smooth: bool = False
    normed_grads: bool = False   # dQ, dK with respect to Q^, K^ (no RMSNorm backward)
    fmt: str = "int8"            # encoding of the low-bit products' operands: "int8" | "fp8"
    split: str = "sagebwd"       # which products are low-bit: "sagebwd" (six of seven) | "qattn"

    def __post_init__(self):
        blk = self.blk
        fk = self.fwd_tk if self.fwd_tk is not None else blk
        sk = self.bwd_sk if self.bwd_sk is not None else blk
        for name, v in (("fwd_tq", self.fwd_tq), ("fwd_tk", fk), ("bwd_tq", self.bwd_tq),
                        ("bwd_pk", self.bwd_pk), ("bwd_sk", sk)):
            if v <= 0 or blk % v != 0:
                raise ValueError(f"{name}={v} must divide blk={blk}")
        if sk % self.bwd_pk != 0:
            raise ValueError("bwd_pk must divide bwd_sk")
        if self.N < 1:
            raise ValueError("N must be positive")
        if self.split not in ("sagebwd", "qattn"):
            raise ValueError(f"split={self.split!r}")

    @property
    def Np(self) -> int:
        """N rounded up to whole blocks: the last block of a head holds N - (Np - blk) tokens."""
        return -(-self.N // self.blk) * self.blk

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / np.sqrt(self.d)

    @property
    def tk(self) -> int:
        return self.fwd_tk if self.fwd_tk is not None else self.blk

    @property
    def sk(self) -> int:
        return self.bwd_sk if self.bwd_sk is not None else self.blk


# ----------------------------------------------------------------------------
# Output rounding to the 16-bit dtype (nearest even).
# ----------------------------------------------------------------------------

def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to fp16 or bf16 (nearest even); return them as float64.

    dtype "f64" leaves the values unrounded (used only by the oracle's own pins).
    fp16 is one rounding of the float64 value. bf16 goes through float32 first; the two
    roundings can only differ from one direct rounding on values within 2^-24 relative of
    a bf16 tie.
    Pinned by: test_oracle_tiles.py::test_round_to_dtype_matches_torch (torch's conversions,
    ties, subnormals, overflow, and a double-rounding case of each branch).
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":  # no rounding: used by the reduction pins
        return x
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
        lsb = (u >> np.uint64(16)) & np.uint64(1)
        r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
        return r.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Prologue, bit-specified in float32.
# ----------------------------------------------------------------------------

def tree_f32(s: np.ndarray) -> np.ndarray:
    """Sum over the last axis (a power of two long) by a pairwise tree over consecutive
    entries: (s0+s1), (s2+s3), ... then ((s0+s1)+(s2+s3)), ... down to one value, float32.
    Pinned by: test_oracle_quant.py::test_rms_norm_chunk_tree_order and
    test_k_smooth_group_tree_order (hand-derived 2^24 absorption cases)."""
    s = np.asarray(s, dtype=F32)
    n = s.shape[-1]
    assert n >= 1 and n & (n - 1) == 0
    while s.shape[-1] > 1:
        s = s[..., 0::2] + s[..., 1::2]
    return s[..., 0]


def rms_norm_f32(x: np.ndarray, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """QK-norm of each token vector (last axis), float32 op by op.

    The d channels (a power of two) form n = min(16, d) chunks of d/n consecutive channels;
    each chunk sum runs in ascending channel order, cs_j = fl(... fl(x_a*x_a +
    x_{a+1}*x_{a+1}) ...) (each x*x is exact for 16-bit x), and ss = tree(cs_0..cs_{n-1}),
    the pairwise tree of tree_f32. The pages fix no summation order;
    this one is the one a 16-lane row of the GPU computes (each lane one chunk, then a
    butterfly across the row).
    ms = fl(ss / d); rstd = fl(1 / fl(sqrt(fl(ms + eps)))); x^ = fl(x * rstd).
    This order is a frozen part of the bit-exact contract: it is specified here and kernels
    follow it, never the reverse.
    Returns (x^, rstd). SageBwd article, QK-norm paragraph (RMSNorm per token, gain 1).
    Pinned by: test_oracle_quant.py::test_rms_norm_* (hand example, order, error bound).
    """
    x = np.asarray(x, dtype=F32)
    d = x.shape[-1]
    n = min(16, d)
    cw = d // n
    assert cw * n == d and n & (n - 1) == 0
    xc = x.reshape(x.shape[:-1] + (n, cw))
    cs = np.zeros(x.shape[:-1] + (n,), dtype=F32)
    for i in range(cw):
        v = xc[..., i]
        cs = cs + v * v
    ss = tree_f32(cs)
    ms = ss / F32(d)
    rstd = F32(1.0) / np.sqrt(ms + F32(eps))
    return x * rstd[..., None], rstd


def k_smooth_f32(khat: np.ndarray, blk: int, n_valid: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """K-smoothing: K~ = K^ - mu, mu = per-channel mean of K^ over the N tokens of a head.

    Order: inside each block of blk tokens (a power of two), token t joins group t mod G,
    G = min(16, blk); each group sums its tokens in ascending order and part = tree of
    the G group sums (tree_f32); then tot = sum of the
    parts in ascending block order (from 0); mu = fl(tot / N); K~ = fl(K^ - mu). The
    pages fix no order; this is the one the GPU's 16 token slots per pass compute.
    Input [..., Np, d] with Np a multiple of blk; with n_valid < Np the rows from n_valid on
    are padding (zeros, which add nothing to the sums): mu = fl(tot / n_valid) and those
    rows of K~ are 0. Returns (K~, mu [..., d]). The order is frozen like rms_norm_f32's.
    SageBwd article, K-smoothing paragraph (axis: see module docstring).
    Pinned by: test_oracle_quant.py::test_k_smooth_* and the softmax-invariance tests.
    """
    khat = np.asarray(khat, dtype=F32)
    N, d = khat.shape[-2], khat.shape[-1]
    nb = N // blk
    G = min(16, blk)
    kb = khat.reshape(khat.shape[:-2] + (nb, blk // G, G, d))    # [..., block, pass, slot, d]
    gs = np.zeros(khat.shape[:-2] + (nb, G, d), dtype=F32)
    for p_ in range(blk // G):
        gs = gs + kb[..., p_, :, :]
    part = tree_f32(np.moveaxis(gs, -2, -1))                       # [..., nb, d]
    tot = np.zeros(khat.shape[:-2] + (d,), dtype=F32)
    for b in range(nb):
        tot = tot + part[..., b, :]
    nv = N if n_valid is None else n_valid
    mu = tot / F32(nv)
    kt = khat - mu[..., None, :]
    if nv < N:
        kt[..., nv:, :] = F32(0.0)
    return kt, mu


def quant_rule_f32(x32: np.ndarray, axes: Tuple[int, ...]) -> Tuple[np.ndarray, np.ndarray]:
    """The one INT8 rule used for every operand: symmetric absmax over `axes`.

    a = max |x|; if a == 0: scale 0, codes 0; else s = fl(a / 127), inv = fl(127 / a),
    code = clamp(rint_even(fl(x * inv)), -127, 127). Scales and inverses are correct
    divisions, never an approximate reciprocal (the NVFP4 page's insight list records
    training blowing up when an approximate reciprocal flushed subnormals).
    Returns (codes int8, scales float32 with `axes` removed).
    Pinned by: test_oracle_quant.py::test_quant_rule_*.
    """
    x32 = np.asarray(x32, dtype=F32)
    a = np.max(np.abs(x32), axis=axes, keepdims=True)
    zero = a == 0
    a_safe = np.where(zero, F32(1.0), a)
    s = np.where(zero, F32(0.0), a_safe / F32(127.0)).astype(F32)
    inv = np.where(zero, F32(0.0), F32(127.0) / a_safe).astype(F32)
    q = np.rint(x32 * inv)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, np.squeeze(s, axis=axes)


def quant_blocks_f32(x: np.ndarray, blk: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-block quantisation of [..., N, d]: one scale per blk tokens x d channels.

    SageBwd article, per-block kernels paragraph. Returns (codes [..., N, d] int8,
    scales [..., N // blk] float32).
    Pinned by: test_oracle_quant.py::test_lossless_block_quant_equals_exact (which block scale
    multiplies which product), test_ragged_block_quant_is_the_rule_on_valid_tokens and the
    hand-derived prologue fixtures.
    """
    x = np.asarray(x, dtype=F32)
    N, d = x.shape[-2], x.shape[-1]
    xb = x.reshape(x.shape[:-2] + (N // blk, blk, d))
    nd = xb.ndim
    q, s = quant_rule_f32(xb, axes=(nd - 2, nd - 1))
    return q.reshape(x.shape), s


# ----------------------------------------------------------------------------
# The FP8 recipe (e4m3, OCP "FN" variant: bias 7, 3 mantissa bits, max 448, no infinity).
# ----------------------------------------------------------------------------

FP8_MAX = 448.0


def e4m3_encode(x32: np.ndarray) -> np.ndarray:
    """float32 -> e4m3 bit patterns (uint8), round to nearest even, from the format's
    definition: normals (1 + m/8) * 2^(e - 7) for e = 1..15 (e = 15, m = 7 is NaN, so the
    largest finite value is 1.75 * 2^8 = 448), subnormals m/8 * 2^-6; the sign is kept (also
    on zero). |x| must stay below 464, the midpoint between 448 and the next step (the NaN
    pattern): fl(x * fl(448 / a)) can exceed 448 by an ulp, and rounds to 448.
    Pinned by: test_oracle_quant.py::test_e4m3_* (torch's float8_e4m3fn conversion, round
    trips of every finite code, hand-made ties)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    if np.any(np.abs(x) >= 464.0):
        raise ValueError("e4m3 input at or beyond 464 (overflows 448)")
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x)
    f, E = np.frexp(a)                       # a = f * 2^E, f in [0.5, 1)
    e = E - 1                                # a = (2f) * 2^e, 2f in [1, 2)
    normal = (a > 0) & (e >= -6)             # zero (frexp exponent 0) takes the subnormal path
    # normals: mantissa steps of 2^(e-3); subnormals: steps of 2^-9
    step = np.where(normal, np.exp2(e - 3.0), 2.0 ** -9)
    q = np.rint(a / step)                    # exact division by a power of two; RNE
    code = np.zeros(x.shape, dtype=np.int64)
    # normal: q in [8, 16]; q == 16 rounds up into the next binade
    qn = q.astype(np.int64)
    en = np.where(qn >= 16, e + 1, e)
    mn = np.where(qn >= 16, 0, qn - 8)
    code = np.where(normal, ((en + 7) << 3) | mn, qn)   # subnormal: q in [0, 8] (8 = min normal)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """e4m3 bit patterns -> float64 values.
    Pinned by: test_oracle_quant.py::test_e4m3_round_trip_and_ties (every finite code) and
    test_e4m3_matches_torch_conversion."""
    c = np.asarray(code).astype(np.int64) & 0xFF
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    v = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


def quant_rule_fp8_f32(x32: np.ndarray, axes: Tuple[int, ...]) -> Tuple[np.ndarray, np.ndarray]:
    """The FP8 rule: symmetric absmax over `axes`, scale s = fl(a / 448), inv = fl(448 / a),
    code = e4m3_rne(fl(x * inv)) (an all-zero block: scale 0, codes 0). Returns (codes as
    uint8 e4m3 bit patterns, scales float32 with `axes` removed).
    Pinned by: test_oracle_quant.py::test_fp8_rule_properties and
    test_fp8_lossless_block_quant_equals_exact."""
    x32 = np.asarray(x32, dtype=F32)
    a = np.max(np.abs(x32), axis=axes, keepdims=True)
    zero = a == 0
    a_safe = np.where(zero, F32(1.0), a)
    s = np.where(zero, F32(0.0), a_safe / F32(FP8_MAX)).astype(F32)
    inv = np.where(zero, F32(0.0), F32(FP8_MAX) / a_safe).astype(F32)
    return e4m3_encode((x32 * inv).astype(F32)), np.squeeze(s, axis=axes)


def quant_blocks_fp8_f32(x: np.ndarray, blk: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-block FP8 quantisation of [..., N, d]: one scale per blk tokens x d channels.
    Pinned by: test_oracle_quant.py::test_fp8_lossless_block_quant_equals_exact."""
    x = np.asarray(x, dtype=F32)
    N, d = x.shape[-2], x.shape[-1]
    xb = x.reshape(x.shape[:-2] + (N // blk, blk, d))
    nd = xb.ndim
    q, s = quant_rule_fp8_f32(xb, axes=(nd - 2, nd - 1))
    return q.reshape(x.shape), s


def code_values(codes: np.ndarray) -> np.ndarray:
    """Values of codes as float64: e4m3 bit patterns (uint8) are decoded, INT8 codes and
    identity "codes" are taken as they are. Pinned by the lossless reductions of both
    formats (test_oracle_quant.py::test_lossless_block_quant_equals_exact, _fp8_)."""
    codes = np.asarray(codes)
    if codes.dtype == np.uint8:
        return e4m3_decode(codes)
    return codes.astype(np.float64)


BlockQuant = Callable[[np.ndarray, int], Tuple[np.ndarray, np.ndarray]]


def identity_block_quant(x: np.ndarray, blk: int) -> Tuple[np.ndarray, np.ndarray]:
    """No quantisation: values pass through as float64 "codes" with block scales 1.
    Pinned by: test_oracle_quant.py::test_identity_quant_equals_exact (any change to the
    values breaks the reduction to exact attention)."""
    x = np.asarray(x, dtype=np.float64)
    return x, np.ones(x.shape[:-2] + (x.shape[-2] // blk,), dtype=np.float64)


def _pad_rows(x: np.ndarray, Np: int, value: float = 0.0) -> np.ndarray:
    """x [..., n, ...] (rows on axis -2 for 4-d tensors, the last axis for [B,H,n]) padded
    with `value` to Np rows. Pinned by: test_oracle_quant.py::test_identity_quant_ragged_n."""
    axis = -2 if x.ndim == 4 else -1
    n = x.shape[axis]
    if n == Np:
        return x
    width = [(0, 0)] * x.ndim
    width[axis] = (0, Np - n)
    return np.pad(x, width, constant_values=value)


def apply_gain_f32(xn: np.ndarray, g: Optional[np.ndarray]) -> np.ndarray:
    """The QK-norm gain: x^ = fl(n * g[h, c]) for n [B,H,N,d] (the normalised tokens) and
    g [H, d] float32 (one IEEE product per element); g None leaves n unchanged (gain 1).
    Pinned by: test_oracle_quant.py::test_gain_prologue_power_of_two_exact and
    test_identity_quant_with_gains."""
    if g is None:
        return xn
    return (xn * np.asarray(g, dtype=F32)[None, :, None, :]).astype(F32)


def prologue(Q: np.ndarray, K: np.ndarray, V: np.ndarray, spec: Spec,
             block_quant: BlockQuant = quant_blocks_f32, q_gain: Optional[np.ndarray] = None,
             k_gain: Optional[np.ndarray] = None,
             v_block_quant: Optional[BlockQuant] = None) -> Dict[str, np.ndarray]:
    """QK-norm (with optional gains [H, d]) -> K-smoothing -> per-block INT8 quantisation
    of Q^, K~, V.

    Inputs: float32 arrays [B,H,N,d] holding the exact values of the 16-bit inputs.
    Returns codes Qc, Kc, Vc (int8 [B,H,N,d], V in natural token-major layout),
    scales Qs, Ks, Vs (float32 [B,H,N/blk]), q_rstd, k_rstd (float32 [B,H,N], 1 when
    QK-norm is off), k_mean (float32 [B,H,d], 0 when smoothing is off), the normalised
    tokens before the gain Qn, Kn and after it Qhat, Khat (float32), which the RMSNorm
    backward and the gains' gradients need, and the gains (q_gain, k_gain; None = 1).
    Pinned by: its steps' pins (rms_norm_f32, k_smooth_f32, quant_blocks_f32), the
    hand-derived prologue fixtures, test_ragged_eps_zero and the reductions to exact
    attention with norm, smoothing and gains on.
    """
    # a ragged last block: pad every head to Np rows with zero tokens, which change no block
    # absmax and no sum; the means divide by the N valid tokens (k_smooth_f32)
    Q, K, V = (_pad_rows(np.asarray(x, dtype=F32), spec.Np) for x in (Q, K, V))
    if spec.qk_norm:
        # (with eps = 0 the zero padding rows divide by zero here; they are replaced just below)
        with np.errstate(divide="ignore", invalid="ignore"):
            Qn, q_rstd = rms_norm_f32(Q, spec.eps)
            Kn, k_rstd = rms_norm_f32(K, spec.eps)
        if spec.N < spec.Np:
            # padding tokens are not normalised: rstd 1, values 0 (with eps = 0 their rstd
            # would be 1/sqrt(0) and 0 * inf would put NaN into every sum over the block)
            for xn, r in ((Qn, q_rstd), (Kn, k_rstd)):
                r[..., spec.N:] = F32(1.0)
                xn[..., spec.N:, :] = F32(0.0)
        Qh, Kh = apply_gain_f32(Qn, q_gain), apply_gain_f32(Kn, k_gain)
    else:
        if q_gain is not None or k_gain is not None:
            raise ValueError("QK-norm gains need qk_norm")
        Qh, q_rstd = Q, np.ones(Q.shape[:-1], dtype=F32)
        Kh, k_rstd = K, np.ones(K.shape[:-1], dtype=F32)
        Qn, Kn = Qh, Kh
    if spec.k_smooth:
        Kt, mu = k_smooth_f32(Kh, spec.blk, spec.N)
    else:
        Kt, mu = Kh, np.zeros(K.shape[:-2] + (K.shape[-1],), dtype=F32)
    if spec.q_smooth:
        # Q-smoothing (SageBwd article, Q-smoothing paragraph): the queries' per-channel mean,
        # taken like the keys' (same order), is subtracted before quantising
        Qt, mu_q = k_smooth_f32(Qh, spec.blk, spec.N)
    else:
        Qt, mu_q = Qh, np.zeros(Q.shape[:-2] + (Q.shape[-1],), dtype=F32)
    Qc, Qs = block_quant(Qt, spec.blk)
    Kc, Ks = block_quant(Kt, spec.blk)
    Vc, Vs = (block_quant if v_block_quant is None else v_block_quant)(V, spec.blk)
    out = dict(Qc=Qc, Kc=Kc, Vc=Vc, Qs=Qs, Ks=Ks, Vs=Vs, q_rstd=q_rstd, k_rstd=k_rstd,
               k_mean=mu, q_mean=mu_q, Qhat=Qh, Khat=Kh, Qn=Qn, Kn=Kn, q_gain=q_gain, k_gain=k_gain)
    out["kbias"] = key_bias(Kc, Ks, mu_q, spec.blk) if spec.q_smooth else np.zeros(K.shape[:-1])
    return out


def key_bias(Kc, Ks, mu_q, blk: int) -> np.ndarray:
    """The per-key score bias Q-smoothing adds back: b_k = sK(block of k) * (Kc_k . mu_Q).

    With Q^ = Q~ + mu_Q, Q^ K^T = Q~ K^T + 1 (K mu_Q)^T (SageBwd article, Q-smoothing
    paragraph); the keys enter as their dequantised codes, the same K the INT8 product uses.
    float64 (it is computed after the codes, like everything past the prologue's float32
    steps). Kc [..., N, d] codes (or identity values), Ks [..., N/blk], mu_q [..., d].
    Returns [..., N] float64.
    Pinned by: test_oracle_quant.py::test_q_smooth_identity_reduction (with identity
    quantisation the smoothed scores equal the unsmoothed ones).
    """
    kc = np.asarray(Kc, dtype=np.float64)
    ks = np.repeat(np.asarray(Ks, dtype=np.float64), blk, axis=-1)
    return ks * np.einsum("...nd,...d->...n", kc, np.asarray(mu_q, dtype=np.float64))


# ----------------------------------------------------------------------------
# In-kernel tile quantiser (P~, P, dS).
# ----------------------------------------------------------------------------

TileQuant = Callable[[np.ndarray], Tuple[np.ndarray, np.ndarray]]


def fp8_tile_quant(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise each tile x[h] with the FP8 rule, deciding in float32; codes returned as their
    float64 values, scales as float64 [BH].
    Pinned by: test_oracle_quant.py::test_fp8_close_to_exact (and the rule's own pins)."""
    x32 = np.asarray(x, dtype=np.float64).astype(F32)
    axes = tuple(range(1, x32.ndim))
    q, s = quant_rule_fp8_f32(x32, axes)
    return e4m3_decode(q), s.astype(np.float64)


def int8_tile_quant(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise each tile x[h] (leading axis = head) with the INT8 rule, deciding in float32.

    Returns (codes as float64, scales as float64 [BH]).
    Pinned by: test_oracle_tiles.py (the exact-rational fixture's codes) and
    test_oracle_quant.py::test_int8_close_to_exact.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(F32)
    axes = tuple(range(1, x32.ndim))
    q, s = quant_rule_f32(x32, axes)
    return q.astype(np.float64), s.astype(np.float64)


def half_round_tile(dtype: str) -> TileQuant:
    """The Q-Attn split's 16-bit operand for P~ and P: every value rounded to the 16-bit type
    dtype (nearest even) after rounding to float32, the precision the kernels hold P in; scale
    1 (no tile scale: P <= 1 fits both 16-bit types). dtype "f64" keeps the values (for pins).
    Pinned by: test_oracle_qattn.py (reduction to exact attention on the dequantised Q, K;
    rounding on vs off) and round_to_dtype's pins."""
    def q(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        x = np.asarray(x, dtype=np.float64)
        if dtype != "f64":
            x = round_to_dtype(x.astype(F32).astype(np.float64), dtype)
        return x, np.ones(x.shape[0], dtype=np.float64)
    return q


def identity_tile_quant(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """No quantisation: values pass through with scale 1 (used to pin the tiling logic).
    Pinned by: test_oracle_quant.py::test_identity_quant_equals_exact."""
    x = np.asarray(x, dtype=np.float64)
    return x, np.ones(x.shape[0], dtype=np.float64)


# ----------------------------------------------------------------------------
# Forward and backward (float64 after the prologue).
# ----------------------------------------------------------------------------

def lowbit_product(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The product of two code operands (batched matmul, float64). INT8 code products are
    exact integers and FP8 code products exact in float64, so this is the plain product; it
    is one function so that a test can model a matrix core's inexact accumulation in its
    place (tests/test_oracle_fp8_model.py). Used for QK^T (both passes), PV, dV, dK and dQ.
    Pinned by: the lossless reductions (test_lossless_block_quant_equals_exact, _fp8_)."""
    return a @ b


def _flat(a: np.ndarray, nlead: int = 2) -> np.ndarray:
    """Merge the first nlead axes into one (a reshape: no arithmetic, nothing to pin)."""
    return a.reshape((-1,) + a.shape[nlead:])


def forward(Qc, Kc, Vc, Qs, Ks, Vs, spec: Spec, tile_quant: TileQuant = int8_tile_quant,
            q_tiles: Optional[Sequence[int]] = None, kbias: Optional[np.ndarray] = None):
    """Flash-style forward with INT8 QK^T and PV (SageBwd article, precision split).

    Per head, per query tile I of fwd_tq rows: m = -inf, l = 0, acc = 0; for key tiles J
    of fwd_tk keys in ascending order, skipping tiles wholly above the causal diagonal:
      S   = Qc_I . Kc_J^T (exact integers),  s = S * sQ(I) * sK(J) * sm_scale
            (+ kbias_J * sm_scale with Q-smoothing: key_bias), masked (key > query)
            -> -inf when causal
      m'  = max(m, rowmax s);  P~ = exp(s - m');  alpha = exp(m - m')
      l   = l * alpha + rowsum P~                     (P~ before quantisation)
      qP, sP = quantise P~ on the tile                (INT8 rule, decided in float32)
      acc = acc * alpha + sP * sV(J) * (qP . Vc_J)    (exact integer product)
      m   = m'
    then O = acc / l (rounded to the dtype) and LSE = m + ln l (natural log, float32).
    Codes may be given as integers or, with identity_tile_quant, as real values.
    With a ragged last block (spec.N < Np rows of codes) keys from N on are masked and the
    padding query rows take no part in any tile (their P~ is 0).
    Returns (O [B,H,N,d] float64 of dtype-rounded values, LSE [B,H,N] float32); with
    q_tiles only those query tiles are computed (rows of other tiles are NaN).
    Pinned by: test_oracle_quant.py identity and lossless reductions to oracle.exact; the
    tile placement (P~ tile shape, running max per key tile, l before quantisation) by
    test_oracle_tiles.py (an exact-rational two-tile fixture that other tilings miss, a spy
    on the quantised tiles, LSE independent of the P~ quantiser).
    """
    B, H, N, d = Qc.shape
    blk, tq, tk = spec.blk, spec.fwd_tq, spec.tk
    sm = spec.scale
    nv = spec.N
    q = code_values(_flat(Qc))
    k = code_values(_flat(Kc))
    v = code_values(_flat(Vc))
    qs = _flat(np.asarray(Qs, dtype=np.float64))
    ks = _flat(np.asarray(Ks, dtype=np.float64))
    vs = _flat(np.asarray(Vs, dtype=np.float64))
    kb = None if kbias is None else _flat(np.asarray(kbias, dtype=np.float64), 2)
    BH = q.shape[0]
    O = np.full((BH, N, d), np.nan)
    LSE = np.full((BH, N), np.nan)
    tiles = range(N // tq) if q_tiles is None else q_tiles
    for it in tiles:
        i0 = it * tq
        rows = np.arange(i0, i0 + tq)
        qi = q[:, i0:i0 + tq, :]
        sq = qs[:, i0 // blk]
        m = np.full((BH, tq), -np.inf)
        l = np.zeros((BH, tq))
        acc = np.zeros((BH, tq, d))
        for j0 in range(0, N, tk):
            if spec.causal and j0 > i0 + tq - 1:
                break
            cols = np.arange(j0, j0 + tk)
            S = lowbit_product(qi, k[:, j0:j0 + tk, :].transpose(0, 2, 1))
            s = S * (sq * ks[:, j0 // blk] * sm)[:, None, None]
            if kb is not None:
                s = s + sm * kb[:, None, j0:j0 + tk]
            if spec.causal:
                s = np.where(cols[None, None, :] > rows[None, :, None], -np.inf, s)
            s = np.where(cols[None, None, :] >= nv, -np.inf, s)
            m_new = np.maximum(m, s.max(axis=-1))
            Pt = np.exp(s - m_new[..., None])
            Pt = np.where(rows[None, :, None] < nv, Pt, 0.0)
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
            l = l * alpha + Pt.sum(axis=-1)
            qP, sP = tile_quant(Pt)
            pv = lowbit_product(qP, v[:, j0:j0 + tk, :])
            acc = acc * alpha[..., None] + (sP * vs[:, j0 // blk])[:, None, None] * pv
            m = m_new
        with np.errstate(divide="ignore", invalid="ignore"):   # padding rows: l = 0, dropped below
            O[:, i0:i0 + tq, :] = acc / l[..., None]
            LSE[:, i0:i0 + tq] = m + np.log(l)
    O = round_to_dtype(O, spec.dtype)
    return O.reshape(B, H, N, d)[:, :, :nv], LSE.astype(F32).reshape(B, H, N)[:, :, :nv]


def backward_pre(O, dO, spec: Spec, block_quant: BlockQuant = quant_blocks_f32):
    """D = rowsum(dO o O) (float64, O as stored in the dtype) and the per-block INT8 dO.

    Returns (D [B,H,N] float64, dOc int8 [B,H,N,d], dOs float32 [B,H,N/blk]).
    Pinned by: the identity reduction of the backward to exact attention (D enters every dS)
    and the planted mistake "ds_drop_D" (test_oracle_quant.py).
    """
    O = np.asarray(O, dtype=np.float64)
    dO32 = np.asarray(dO, dtype=F32)
    D = np.sum(dO32.astype(np.float64) * O, axis=-1)
    dOc, dOs = block_quant(dO32, spec.blk)
    return D, dOc, dOs


def rms_norm_backward(dy: np.ndarray, y: np.ndarray, rstd: np.ndarray) -> np.ndarray:
    """Backward of y = x * rstd(x) with rstd = (mean_c x^2 + eps)^-1/2 (float64):
    dx = rstd * (dy - y * mean_c(dy * y)). Pinned by the finite-difference tests."""
    dy = np.asarray(dy, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(rstd, dtype=np.float64)[..., None]
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def backward(pro: Dict[str, np.ndarray], Q, K, V, O, LSE, dO, spec: Spec,
             tile_quant: TileQuant = int8_tile_quant,
             block_quant: BlockQuant = quant_blocks_f32,
             q_tiles: Optional[Sequence[int]] = None,
             k_tiles: Optional[Sequence[int]] = None,
             p_quant: Optional[TileQuant] = None,
             do_quant: Optional[BlockQuant] = None):
    """Backward with recomputed INT8 QK^T, FP dP = dO V^T and INT8 dV, dK, dQ.

    pro: the prologue's dict (codes, scales, rstd, Qhat, Khat). Q, K, V, dO: float32
    exact 16-bit values; O: the forward's output as stored (dtype values); LSE float32.
    Per head, for every visible pair of query tile I (bwd_tq rows) and key tile J
    (bwd_sk keys), in ascending I then J:
      s  = (Qc_I . Kc_J^T) * sQ(I) * sK(J) * sm_scale (+ kbias_J * sm_scale with
           Q-smoothing) (masked -> -inf); P = exp(s - LSE_I)
      dP = dO_I . V_J^T   (the 16-bit dO and V, never quantised; SageBwd article,
                           precision split: this product alone stays 16-bit)
      dS = P o (dP - D_I)
      qdS, sdS = quantise dS on the tile
      for each key sub-tile J' of bwd_pk keys: qP, sP = quantise P_{I,J'};
           dV_J' += sP * sdO(I) * (qP^T . dOc_I)
      dK_J += sm * sdS * sQ(I) * (qdS^T . Qc_I)
              (+ sm * sdS * (qdS^T 1) mu_Q^T with Q-smoothing: Q^ = Q~ + mu_Q, so
               dS^T Q^ = dS^T Q~ + (dS^T 1) mu_Q^T, the pages' dK_bias term)
      dQ_I += sm * sdS * sK(J) * (qdS . Kc_J)          (Kc: the smoothed K codes)
    Epilogue: dQ = RMSNorm-backward(g_Q o dQ^, Qn, q_rstd), dK = RMSNorm-backward(g_K o dK^,
    Kn, k_rstd) when QK-norm is on (Qn, Kn: the normalised tokens before the gains, K before
    smoothing; smoothing adds no term because every dS row sums to zero), then all three are
    rounded to the dtype. With gains, dq_gain = sum over batch and tokens of dQ^ o Qn (and
    likewise dk_gain), float64 [H, d]. With spec.normed_grads the epilogue stops at dQ^, dK^
    (the gradients with respect to the normalised tokens).
    With q_tiles / k_tiles only pairs whose I is in q_tiles (bwd_tq units) or whose J
    is in k_tiles (bwd_sk units) are visited: dQ is then exact for those query tiles,
    dK and dV for those key tiles, and NaN elsewhere.
    p_quant (default tile_quant) quantises the P tiles of dV and do_quant (default
    block_quant) the dO blocks: the Q-Attn split passes the 16-bit rounding and the
    identity, so dV = round16(P)^T dO.
    Returns dict dQ, dK, dV ([B,H,N,d] float64 of dtype-rounded values) plus D, dOc, dOs, and
    dQ_code_step, dK_code_step ([B,H,N] float64): for each row of dQ (dK), an upper bound on
    how far one unit of one of its dS codes moves that row (L2), in the row's own units. A dS
    code is decided by rounding a float at a grid point, so an implementation whose dS differs
    from this one in the last float32 bits (another exp, LSE or summation order) may land on
    the neighbouring code at a near-tie; for integer codes one unit is one such step. Per tile,
    one unit at (i, j) adds sm * sdS * sK(J) * Kc_j to dQ^_i and sm * sdS * (sQ(I) * Qc_i
    (+ mu_Q with Q-smoothing)) to dK^_j; the bound takes the largest key (query) row norm of the
    tile and the largest over the row's tiles, then the RMSNorm backward's factor rstd * max|g|
    (its map is rstd times a contraction, mean(y^2) <= 1, applied to g o dX^).
    Pinned by: test_oracle_code_step.py (a planted one-unit code change is matched exactly on
    a single tile and stays within the bound on many tiles, with and without QK-norm, gains and
    Q-smoothing); test_oracle_quant.py (identity and lossless reductions to oracle.exact,
    finite-difference-pinned exact gradients, planted mistakes) and, for the P and dS tile
    placement, test_oracle_tiles.py (exact-rational fixture that other tilings miss, spy).
    """
    B, H, N, d = pro["Qc"].shape
    blk, tq, sk, pk = spec.blk, spec.bwd_tq, spec.sk, spec.bwd_pk
    sm = spec.scale
    # a ragged last block: the padding rows (from spec.N on) are zero tokens with LSE = +inf,
    # so their P is 0, and keys from spec.N on are masked
    nv = spec.N
    V, dO, O = (_pad_rows(np.asarray(x), N) for x in (V, dO, O))
    LSE = _pad_rows(np.asarray(LSE, dtype=F32), N, np.inf)
    D, dOc, dOs = backward_pre(O, dO, spec, block_quant=block_quant if do_quant is None else do_quant)
    if p_quant is None:
        p_quant = tile_quant
    qc = code_values(_flat(pro["Qc"]))
    kc = code_values(_flat(pro["Kc"]))
    qs = _flat(np.asarray(pro["Qs"], dtype=np.float64))
    ks = _flat(np.asarray(pro["Ks"], dtype=np.float64))
    doc = code_values(_flat(dOc))
    dos = _flat(np.asarray(dOs, dtype=np.float64))
    do = _flat(np.asarray(dO, dtype=F32)).astype(np.float64)
    vf = _flat(np.asarray(V, dtype=F32)).astype(np.float64)
    lse = _flat(np.asarray(LSE, dtype=F32)).astype(np.float64)
    Df = _flat(D)
    qsm = spec.q_smooth
    kb = _flat(np.asarray(pro["kbias"], dtype=np.float64), 2) if qsm else None
    muq = _flat(np.asarray(pro["q_mean"], dtype=np.float64)) if qsm else None
    BH = qc.shape[0]
    dQh = np.zeros((BH, N, d))
    dKh = np.zeros((BH, N, d))
    dV = np.zeros((BH, N, d))
    stepQ = np.zeros((BH, N))
    stepK = np.zeros((BH, N))
    qsel = None if q_tiles is None else set(q_tiles)
    ksel = None if k_tiles is None else set(k_tiles)
    for it in range(N // tq):
        i0 = it * tq
        rows = np.arange(i0, i0 + tq)
        for jt in range(N // sk):
            j0 = jt * sk
            if spec.causal and j0 > i0 + tq - 1:
                break
            if qsel is not None or ksel is not None:
                if not ((qsel is not None and it in qsel) or (ksel is not None and jt in ksel)):
                    continue
            cols = np.arange(j0, j0 + sk)
            S = lowbit_product(qc[:, i0:i0 + tq, :], kc[:, j0:j0 + sk, :].transpose(0, 2, 1))
            s = S * (qs[:, i0 // blk] * ks[:, j0 // blk] * sm)[:, None, None]
            if qsm:
                s = s + sm * kb[:, None, j0:j0 + sk]
            if spec.causal:
                s = np.where(cols[None, None, :] > rows[None, :, None], -np.inf, s)
            s = np.where(cols[None, None, :] >= nv, -np.inf, s)
            P = np.exp(s - lse[:, i0:i0 + tq, None])
            dP = do[:, i0:i0 + tq, :] @ vf[:, j0:j0 + sk, :].transpose(0, 2, 1)
            dS = P * (dP - Df[:, i0:i0 + tq, None])
            qdS, sdS = tile_quant(dS)
            kmax = np.linalg.norm(kc[:, j0:j0 + sk, :], axis=2).max(axis=1)
            qrow = qs[:, i0 // blk][:, None, None] * qc[:, i0:i0 + tq, :]
            if qsm:
                qrow = qrow + muq[:, None, :]
            qmax = np.linalg.norm(qrow, axis=2).max(axis=1)
            stepQ[:, i0:i0 + tq] = np.maximum(stepQ[:, i0:i0 + tq], (sm * sdS * ks[:, j0 // blk] * kmax)[:, None])
            stepK[:, j0:j0 + sk] = np.maximum(stepK[:, j0:j0 + sk], (sm * sdS * qmax)[:, None])
            for p0 in range(0, sk, pk):
                qP, sP = p_quant(P[:, :, p0:p0 + pk])
                dV[:, j0 + p0:j0 + p0 + pk, :] += (sP * dos[:, i0 // blk])[:, None, None] * (
                    lowbit_product(qP.transpose(0, 2, 1), doc[:, i0:i0 + tq, :]))
            dKh[:, j0:j0 + sk, :] += (sm * sdS * qs[:, i0 // blk])[:, None, None] * (
                lowbit_product(qdS.transpose(0, 2, 1), qc[:, i0:i0 + tq, :]))
            if qsm:
                dKh[:, j0:j0 + sk, :] += q_smooth_dk_bias(qdS, sdS, muq, sm)
            dQh[:, i0:i0 + tq, :] += (sm * sdS * ks[:, j0 // blk])[:, None, None] * (
                lowbit_product(qdS, kc[:, j0:j0 + sk, :]))
    gains = {}
    if spec.qk_norm and spec.normed_grads:
        dQ, dK = dQh, dKh   # gradients with respect to Q^ = g o n and K^ (before smoothing)
    elif spec.qk_norm:
        # with gains g: X^ = g o n, so dn = g o dX^ and dg = sum over batch and tokens of dX^ o n
        qg, kg = pro.get("q_gain"), pro.get("k_gain")
        Qn, Kn = _flat(pro.get("Qn", pro["Qhat"])), _flat(pro.get("Kn", pro["Khat"]))
        gq = np.ones((1, 1, d)) if qg is None else np.broadcast_to(
            np.asarray(qg, np.float64), (B, H, d)).reshape(B * H, 1, d)
        gk = np.ones((1, 1, d)) if kg is None else np.broadcast_to(
            np.asarray(kg, np.float64), (B, H, d)).reshape(B * H, 1, d)
        dQ = rms_norm_backward(dQh * gq, Qn, _flat(pro["q_rstd"]))
        dK = rms_norm_backward(dKh * gk, Kn, _flat(pro["k_rstd"]))
        stepQ = stepQ * _flat(np.asarray(pro["q_rstd"], np.float64)) * np.abs(gq).max(axis=2)
        stepK = stepK * _flat(np.asarray(pro["k_rstd"], np.float64)) * np.abs(gk).max(axis=2)
        if qg is not None or kg is not None:
            gains = dict(dq_gain=(dQh * Qn).reshape(B, H, N, d).sum(axis=(0, 2)),
                         dk_gain=(dKh * Kn).reshape(B, H, N, d).sum(axis=(0, 2)))
    else:
        dQ, dK = dQh, dKh
    if qsel is not None or ksel is not None:
        qmask = np.zeros(N, dtype=bool)
        kmask = np.zeros(N, dtype=bool)
        for it in (qsel or ()):
            qmask[it * tq:(it + 1) * tq] = True
        for jt in (ksel or ()):
            kmask[jt * sk:(jt + 1) * sk] = True
        dQ = np.where(qmask[None, :, None], dQ, np.nan)
        dK = np.where(kmask[None, :, None], dK, np.nan)
        dV = np.where(kmask[None, :, None], dV, np.nan)
    out = dict(
        dQ=round_to_dtype(dQ, spec.dtype).reshape(B, H, N, d)[:, :, :nv],
        dK=round_to_dtype(dK, spec.dtype).reshape(B, H, N, d)[:, :, :nv],
        dV=round_to_dtype(dV, spec.dtype).reshape(B, H, N, d)[:, :, :nv],
        D=D, dOc=dOc, dOs=dOs,
        dQ_code_step=stepQ.reshape(B, H, N)[:, :, :nv],
        dK_code_step=stepK.reshape(B, H, N)[:, :, :nv],
    )
    out.update(gains)
    return out


def q_smooth_dk_bias(qdS, sdS, mu_q, sm: float) -> np.ndarray:
    """Q-smoothing's dK_bias on one tile: sm * (dS^T 1) mu_Q^T (SageBwd article, Q-smoothing
    paragraph), with dS the tile's dequantised codes (sdS * qdS, the dS the INT8 dK product
    uses) summed over the tile's queries. qdS [BH, tq, sk], sdS [BH], mu_q [BH, d].
    Returns the [BH, sk, d] increment of dK^ (float64).
    Pinned by: test_oracle_quant.py::test_identity_quant_with_q_smoothing and the planted
    mistake "qs_drop_dk_bias".
    """
    csum = np.asarray(sdS, np.float64)[:, None] * np.asarray(qdS, np.float64).sum(axis=1)
    return sm * csum[:, :, None] * np.asarray(mu_q, np.float64)[:, None, :]


def run(Q, K, V, dO, spec: Spec, tile_quant: Optional[TileQuant] = None,
        block_quant: Optional[BlockQuant] = None, q_gain: Optional[np.ndarray] = None,
        k_gain: Optional[np.ndarray] = None):
    """Prologue -> forward -> backward on whole tensors. Returns one dict of everything
    (with gains [H, d] also their gradients dq_gain, dk_gain). The quantisers default to the
    recipe of spec.fmt: the INT8 rule, or the FP8 (e4m3) rule with absmax/448 scales.
    Pinned by: the pins of its three steps (prologue, forward, backward)."""
    fp8 = spec.fmt == "fp8"
    if tile_quant is None:
        tile_quant = fp8_tile_quant if fp8 else int8_tile_quant
    if block_quant is None:
        block_quant = quant_blocks_fp8_f32 if fp8 else quant_blocks_f32
    qattn = spec.split == "qattn"
    # Q-Attn: PV, P^T dO in 16 bits (P~, P rounded to the dtype; V, dO their own values)
    half = half_round_tile(spec.dtype) if qattn else None
    pro = prologue(Q, K, V, spec, block_quant=block_quant, q_gain=q_gain, k_gain=k_gain,
                   v_block_quant=identity_block_quant if qattn else None)
    O, LSE = forward(pro["Qc"], pro["Kc"], pro["Vc"], pro["Qs"], pro["Ks"], pro["Vs"], spec,
                     tile_quant=half if qattn else tile_quant,
                     kbias=pro["kbias"] if spec.q_smooth else None)
    g = backward(pro, Q, K, V, O, LSE, dO, spec, tile_quant=tile_quant, block_quant=block_quant,
                 p_quant=half if qattn else None, do_quant=identity_block_quant if qattn else None)
    out = dict(pro)
    out.update(O=O, LSE=LSE)
    out.update(g)
    return out
