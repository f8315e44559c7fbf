"""O-X: full-precision float64 attention with QK-norm, forward and backward (CPU, numpy).

Test infrastructure only (see oracle/__init__.py). No quantisation anywhere.

Forward:  Q^ = g_Q o RMSNorm(Q), K^ = g_K o RMSNorm(K) per token over d (when QK-norm is on;
          SageBwd article, QK-norm paragraph; the gains g [H, d] default to 1 and are
          learnable, their gradients dg = sum over batch and tokens of dX^ o RMSNorm(X));
          S = sm * Q^ K^T, masked above the
          diagonal when causal; P = softmax_rows(S); O = P V; LSE = ln sum_j exp(S_ij).
Backward: dV = P^T dO; dP = dO V^T; D = rowsum(dO o O); dS = P o (dP - D);
          dQ^ = sm * dS K^; dK^ = sm * dS^T Q^ (SageBwd article, gradient paragraph);
          dQ, dK = RMSNorm backward of g o dQ^, g o dK^.
K-smoothing is left out: subtracting any fixed vector from every key adds a per-row
constant to S, which softmax ignores (pinned by test_oracle_exact.py).

Rows are processed in blocks of query rows so that long sequences never hold the
N x N matrix; each row of the softmax is computed whole, as the definition says.
Pinned by: central finite differences (test_oracle_exact.py::test_grad_fd,
test_gain_grad_fd), torch's float64 RMSNorm and attention routine under autograd
(test_matches_torch_autograd, test_gain_matches_torch_autograd), closed forms (identical
keys, single key), and the dS structure (row sums zero, RMS(dS) bound).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def rms_norm(x: np.ndarray, eps: float):
    """y = x / sqrt(mean_c x^2 + eps); returns (y, rstd) in float64.
    Pinned by: torch's rms_norm in test_matches_torch_autograd (qk_norm on: O and LSE to
    1e-11)."""
    x = np.asarray(x, dtype=np.float64)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * rstd[..., None], rstd


def rms_norm_backward(dy: np.ndarray, y: np.ndarray, rstd: np.ndarray) -> np.ndarray:
    """Backward of y = x * rstd(x): dx = rstd * (dy - y * mean_c(dy * y)).
    Pinned by: finite differences of dQ, dK with qk_norm on (test_grad_fd) and torch
    autograd through rms_norm (test_matches_torch_autograd)."""
    r = rstd[..., None]
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def _gain_rows(g, lead, BH: int, d: int) -> np.ndarray:
    """A gain [H, d] (or None -> ones) as [BH, 1, d] for inputs with leading dims (.., H).
    Pinned by: test_gain_grad_fd, test_gain_matches_torch_autograd (per-head gains on H = 2
    and 3) and test_unit_gain_is_no_gain."""
    if g is None:
        return np.ones((BH, 1, d))
    g = np.asarray(g, dtype=np.float64)
    return np.broadcast_to(g, tuple(lead[:-1]) + g.shape).reshape(BH, 1, d)


def attention(Q, K, V, dO=None, *, causal: bool, qk_norm: bool, eps: float = 1e-6,
              sm_scale: Optional[float] = None, k_shift: Optional[np.ndarray] = None,
              row_block: int = 512, want_ds_stats: bool = False,
              q_gain: Optional[np.ndarray] = None, k_gain: Optional[np.ndarray] = None,
              normed_grads: bool = False) -> Dict[str, np.ndarray]:
    """Exact attention on [..., N, d] float64 inputs; the backward runs when dO is given.

    normed_grads: dQ, dK are the gradients with respect to the normalised Q^, K^ (the RMSNorm
    backward is left to the caller).

    q_gain, k_gain: optional QK-norm gains [H, d] (the last leading axis of the inputs is H);
    with them the backward also returns dq_gain, dk_gain [H, d].

    k_shift: optional vector (broadcast to [..., d]) subtracted from every normalised key
    before the scores (used only to check that K-smoothing leaves the output unchanged).
    want_ds_stats: also return, per query row, sqrt(mean_j dS_ij^2) over the row's
    visible keys ("ds_rms"), sqrt(sum_j dS_ij^2) ("ds_l2"), max_j |dP_ij| ("dp_max"),
    the row sum of dS ("ds_rowsum") and max_j |dS_ij| ("ds_max").

    Pinned by: test_grad_fd (every gradient against central differences of loss(), both
    masks, QK-norm on and off), test_matches_torch_autograd (O, LSE, dQ, dK, dV against
    torch's float64 attention), test_closed_form_identical_keys / _single_key,
    test_k_smoothing_invariance (k_shift), test_ds_structure and test_ds_rms_falls_with_sqrt_n
    (want_ds_stats), test_gain_* (gains), test_normed_grads_equal_attention_on_normalised_inputs.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    lead = Q.shape[:-2]
    N, d = Q.shape[-2], Q.shape[-1]
    q = Q.reshape((-1, N, d))
    k = K.reshape((-1, N, d))
    v = V.reshape((-1, N, d))
    BH = q.shape[0]
    sm = sm_scale if sm_scale is not None else 1.0 / np.sqrt(d)
    gq = _gain_rows(q_gain, lead, BH, d)
    gk = _gain_rows(k_gain, lead, BH, d)
    if qk_norm:
        qn, rq = rms_norm(q, eps)
        kn, rk = rms_norm(k, eps)
        qh, kh = qn * gq, kn * gk
    else:
        qh, rq = q, np.ones((BH, N))
        kh, rk = k, np.ones((BH, N))
    ks = kh if k_shift is None else kh - np.broadcast_to(np.asarray(k_shift, np.float64),
                                                         lead + (d,)).reshape(BH, 1, d)
    O = np.empty((BH, N, d))
    LSE = np.empty((BH, N))
    have_bwd = dO is not None
    if have_bwd:
        do = np.asarray(dO, dtype=np.float64).reshape((-1, N, d))
        dqh = np.empty((BH, N, d))
        dkh = np.zeros((BH, N, d))
        dv = np.zeros((BH, N, d))
    stats = {name: np.empty((BH, N)) for name in ("ds_rms", "ds_l2", "dp_max", "ds_rowsum", "ds_max")}
    cols = np.arange(N)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        rows = np.arange(r0, r1)
        S = sm * (qh[:, r0:r1, :] @ ks.transpose(0, 2, 1))
        if causal:
            S = np.where(cols[None, None, :] > rows[None, :, None], -np.inf, S)
        m = S.max(axis=-1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=-1, keepdims=True)
        P = E / l
        O[:, r0:r1, :] = P @ v
        LSE[:, r0:r1] = (m + np.log(l))[..., 0]
        if have_bwd:
            dv += P.transpose(0, 2, 1) @ do[:, r0:r1, :]
            dP = do[:, r0:r1, :] @ v.transpose(0, 2, 1)
            D = np.sum(do[:, r0:r1, :] * O[:, r0:r1, :], axis=-1, keepdims=True)
            dS = P * (dP - D)
            dqh[:, r0:r1, :] = sm * (dS @ kh)
            dkh += sm * (dS.transpose(0, 2, 1) @ qh[:, r0:r1, :])
            if want_ds_stats:
                nvis = (rows + 1).astype(np.float64) if causal else np.full(r1 - r0, float(N))
                vis = np.ones_like(dS, dtype=bool)
                if causal:
                    vis = np.broadcast_to(cols[None, None, :] <= rows[None, :, None], dS.shape)
                sq = np.sum(dS * dS, axis=-1)
                stats["ds_l2"][:, r0:r1] = np.sqrt(sq)
                stats["ds_rms"][:, r0:r1] = np.sqrt(sq / nvis[None, :])
                stats["dp_max"][:, r0:r1] = np.max(np.where(vis, np.abs(dP), 0.0), axis=-1)
                stats["ds_rowsum"][:, r0:r1] = dS.sum(axis=-1)
                stats["ds_max"][:, r0:r1] = np.abs(dS).max(axis=-1)
    out = dict(O=O.reshape(lead + (N, d)), LSE=LSE.reshape(lead + (N,)))
    if have_bwd:
        if qk_norm and normed_grads:
            dq, dk = dqh, dkh
        elif qk_norm:
            dq = rms_norm_backward(dqh * gq, qn, rq)
            dk = rms_norm_backward(dkh * gk, kn, rk)
            if q_gain is not None or k_gain is not None:
                H = lead[-1]
                out.update(dq_gain=(dqh * qn).reshape((-1, H, N, d)).sum(axis=(0, 2)),
                           dk_gain=(dkh * kn).reshape((-1, H, N, d)).sum(axis=(0, 2)))
        else:
            dq, dk = dqh, dkh
        out.update(dQ=dq.reshape(lead + (N, d)), dK=dk.reshape(lead + (N, d)),
                   dV=dv.reshape(lead + (N, d)))
        if want_ds_stats:
            out.update({k_: v_.reshape(lead + (N,)) for k_, v_ in stats.items()})
    return out


def loss(Q, K, V, dO, **kw) -> float:
    """L = sum(dO o O): its gradient w.r.t. (Q, K, V) is what attention(..., dO) returns.
    Pinned by: test_matches_torch_autograd (O itself against torch); the finite differences
    in test_grad_fd difference this function."""
    out = attention(Q, K, V, None, **kw)
    return float(np.sum(np.asarray(dO, np.float64) * out["O"]))
