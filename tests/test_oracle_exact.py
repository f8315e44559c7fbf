"""Pins for the exact float64 oracle (oracle.exact) against things other than itself.

- central finite differences of L = sum(dO o O) (gradients),
- torch's own attention and RMSNorm routines with autograd, in float64 on the CPU,
- closed forms (identical keys -> uniform softmax; one key -> O = V),
- the dS structure the SageBwd article relies on (row sums zero; RMS(dS) bounded by
  2 max|dP| / sqrt(N) and falling at least like 1/sqrt(N); article paragraph on the
  dS magnitude bound),
- K-smoothing invariance (article, K-smoothing paragraph): subtracting a fixed vector
  from all keys leaves the attention output unchanged.
"""
import numpy as np
import pytest

from oracle import exact

pytestmark = []


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("qk_norm", [False, True])
@pytest.mark.parametrize("N,d", [(4, 4), (8, 8), (5, 3)])
def test_grad_fd(causal, qk_norm, N, d):
    rng = np.random.default_rng(7 + N * 10 + d + 100 * causal + 1000 * qk_norm)
    Q, K, V, dO = (_rand(rng, 1, 1, N, d) for _ in range(4))
    kw = dict(causal=causal, qk_norm=qk_norm, eps=1e-6)
    out = exact.attention(Q, K, V, dO, **kw)
    h = 1e-6
    for name, X, G in (("Q", Q, out["dQ"]), ("K", K, out["dK"]), ("V", V, out["dV"])):
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp = X.copy(); Xp[idx] += h
            Xm = X.copy(); Xm[idx] -= h
            args = {"Q": Q, "K": K, "V": V}
            args[name] = Xp
            lp = exact.loss(args["Q"], args["K"], args["V"], dO, **kw)
            args[name] = Xm
            lm = exact.loss(args["Q"], args["K"], args["V"], dO, **kw)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(G - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("qk_norm", [False, True])
def test_matches_torch_autograd(causal, qk_norm):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(11 + causal + 2 * qk_norm)
    B, H, N, d = 2, 3, 37, 16
    Q, K, V, dO = (_rand(rng, B, H, N, d) for _ in range(4))
    eps = 1e-6
    out = exact.attention(Q, K, V, dO, causal=causal, qk_norm=qk_norm, eps=eps, row_block=8)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    a, b = tq, tk
    if qk_norm:
        a = F.rms_norm(tq, (d,), eps=eps)
        b = F.rms_norm(tk, (d,), eps=eps)
    o = F.scaled_dot_product_attention(a, b, tv, is_causal=causal)
    o.backward(torch.tensor(dO))
    np.testing.assert_allclose(out["O"], o.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(out["dQ"], tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(out["dK"], tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(out["dV"], tv.grad.numpy(), rtol=1e-9, atol=1e-11)
    # LSE against the library's logsumexp of the masked scores
    s = (a @ b.transpose(-1, -2)) / np.sqrt(d)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(out["LSE"], torch.logsumexp(s, -1).detach().numpy(), rtol=1e-12)


def test_closed_form_identical_keys():
    rng = np.random.default_rng(3)
    N, d = 9, 4
    Q = _rand(rng, N, d)
    K = np.tile(_rand(rng, 1, d), (N, 1))
    V = _rand(rng, N, d)
    for causal in (False, True):
        out = exact.attention(Q, K, V, causal=causal, qk_norm=False)
        for i in range(N):
            n = i + 1 if causal else N
            np.testing.assert_allclose(out["O"][i], V[:n].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_closed_form_single_key():
    rng = np.random.default_rng(4)
    Q, K, V = (_rand(rng, 1, 5) for _ in range(3))
    out = exact.attention(Q, K, V, causal=True, qk_norm=True)
    np.testing.assert_allclose(out["O"], V, rtol=0, atol=0)
    s = np.sum(exact.rms_norm(Q, 1e-6)[0] * exact.rms_norm(K, 1e-6)[0]) / np.sqrt(5)
    np.testing.assert_allclose(out["LSE"], [s], rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_k_smoothing_invariance(causal):
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 40, 8
    Q, K, V = (_rand(rng, B, H, N, d) for _ in range(3))
    K = K + 3.0 * _rand(rng, 1, H, 1, d)  # channel bias, the case smoothing targets
    base = exact.attention(Q, K, V, causal=causal, qk_norm=True)
    mu = exact.rms_norm(K, 1e-6)[0].mean(axis=-2)  # per-channel mean over tokens
    sm = exact.attention(Q, K, V, causal=causal, qk_norm=True, k_shift=mu)
    np.testing.assert_allclose(sm["O"], base["O"], rtol=1e-12, atol=1e-13)
    # whereas a per-token mean (the other axis) is not invariant
    Kh = exact.rms_norm(K, 1e-6)[0]
    tok = Kh - Kh.mean(axis=-1, keepdims=True)
    # apply by passing normalised-and-shifted keys with QK-norm off on both sides
    Qh = exact.rms_norm(Q, 1e-6)[0]
    a = exact.attention(Qh, Kh, V, causal=causal, qk_norm=False)["O"]
    b = exact.attention(Qh, tok, V, causal=causal, qk_norm=False)["O"]
    assert np.max(np.abs(a - b)) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_ds_structure(causal):
    rng = np.random.default_rng(6)
    Q, K, V, dO = (_rand(rng, 1, 2, 64, 16) for _ in range(4))
    out = exact.attention(Q, K, V, dO, causal=causal, qk_norm=True, want_ds_stats=True, row_block=16)
    # every row of dS sums to zero (P sums to 1 and D = sum_j P_ij dP_ij)
    assert np.max(np.abs(out["ds_rowsum"])) <= 1e-12 * max(1.0, np.max(out["ds_max"]))
    # the per-row bound: sqrt(mean_j dS^2) <= 2 max|dP| / sqrt(n_visible)
    n = (np.arange(64) + 1.0) if causal else np.full(64, 64.0)
    assert np.all(out["ds_rms"] <= 2 * out["dp_max"] / np.sqrt(n)[None, None, :] + 1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_ds_rms_falls_with_sqrt_n(causal):
    """RMS(dS) falls at least like 1/sqrt(N) on random inputs (article, dS bound paragraph)."""
    Ns = [128, 256, 512, 1024]
    rms = []
    for N in Ns:
        rng = np.random.default_rng(1000 + N)
        Q, K, V, dO = (_rand(rng, 1, 2, N, 32).astype(np.float32).astype(np.float64) for _ in range(4))
        out = exact.attention(Q, K, V, dO, causal=causal, qk_norm=True, want_ds_stats=True, row_block=256)
        n = (np.arange(N) + 1.0) if causal else np.full(N, float(N))
        assert np.all(out["ds_rms"] <= 2 * out["dp_max"] / np.sqrt(n)[None, None, :] + 1e-15)
        rows = slice(N // 2, N) if causal else slice(0, N)  # causal: rows that see >= N/2 keys
        rms.append(np.sqrt(np.mean(out["ds_rms"][..., rows] ** 2)))
    slope = np.polyfit(np.log(Ns), np.log(rms), 1)[0]
    assert slope <= -0.5 + 0.1, slope


# ---------------------------------------------------------------- learnable QK-norm gains

@pytest.mark.parametrize("causal", [False, True])
def test_gain_grad_fd(causal):
    """Gradients with respect to Q, K, V and the two gains [H, d] against central finite
    differences of L = sum(dO o O)."""
    rng = np.random.default_rng(51 + causal)
    B, H, N, d = 1, 2, 5, 4
    Q, K, V, dO = (_rand(rng, B, H, N, d) for _ in range(4))
    gq = 1.0 + 0.3 * _rand(rng, H, d)
    gk = 1.0 + 0.3 * _rand(rng, H, d)
    kw = dict(causal=causal, qk_norm=True, eps=1e-6)
    out = exact.attention(Q, K, V, dO, q_gain=gq, k_gain=gk, **kw)
    h = 1e-6
    args = {"Q": Q, "K": K, "V": V, "gq": gq, "gk": gk}

    def L(a):
        return exact.loss(a["Q"], a["K"], a["V"], dO, q_gain=a["gq"], k_gain=a["gk"], **kw)

    for name, G in (("Q", out["dQ"]), ("K", out["dK"]), ("V", out["dV"]), ("gq", out["dq_gain"]),
                    ("gk", out["dk_gain"])):
        X = args[name]
        fd = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            ap, am = dict(args), dict(args)
            ap[name] = X.copy(); ap[name][idx] += h
            am[name] = X.copy(); am[name][idx] -= h
            fd[idx] = (L(ap) - L(am)) / (2 * h)
        err = np.linalg.norm(G - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err < 1e-6, (name, err)


def test_gain_matches_torch_autograd():
    """torch's RMSNorm with a weight and its attention routine, autograd in float64."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(61)
    B, H, N, d = 2, 3, 23, 8
    Q, K, V, dO = (_rand(rng, B, H, N, d) for _ in range(4))
    gq = 1.0 + 0.5 * _rand(rng, H, d)
    gk = 1.0 + 0.5 * _rand(rng, H, d)
    eps = 1e-6
    out = exact.attention(Q, K, V, dO, causal=True, qk_norm=True, eps=eps, row_block=8, q_gain=gq, k_gain=gk)
    tq, tk, tv, tgq, tgk = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V, gq, gk))
    a = F.rms_norm(tq, (d,), eps=eps) * tgq[None, :, None, :]
    b = F.rms_norm(tk, (d,), eps=eps) * tgk[None, :, None, :]
    o = F.scaled_dot_product_attention(a, b, tv, is_causal=True)
    o.backward(torch.tensor(dO))
    assert np.allclose(out["O"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    for mine, ref in ((out["dQ"], tq), (out["dK"], tk), (out["dV"], tv), (out["dq_gain"], tgq),
                      (out["dk_gain"], tgk)):
        assert np.allclose(mine, ref.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_unit_gain_is_no_gain():
    rng = np.random.default_rng(71)
    Q, K, V, dO = (_rand(rng, 1, 2, 9, 8) for _ in range(4))
    a = exact.attention(Q, K, V, dO, causal=True, qk_norm=True)
    b = exact.attention(Q, K, V, dO, causal=True, qk_norm=True, q_gain=np.ones((2, 8)), k_gain=np.ones((2, 8)))
    for k in ("O", "dQ", "dK", "dV"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("causal", [False, True])
def test_normed_grads_equal_attention_on_normalised_inputs(causal):
    """The gradients with respect to Q^ = RMSNorm(Q), K^ (normed_grads) are those of plain
    attention (QK-norm off, itself pinned by finite differences) applied to Q^, K^."""
    rng = np.random.default_rng(101 + causal)
    Q, K, V, dO = (_rand(rng, 1, 2, 11, 8) for _ in range(4))
    a = exact.attention(Q, K, V, dO, causal=causal, qk_norm=True, normed_grads=True)
    qh, kh = exact.rms_norm(Q, 1e-6)[0], exact.rms_norm(K, 1e-6)[0]
    b = exact.attention(qh, kh, V, dO, causal=causal, qk_norm=False)
    for k in ("O", "dQ", "dK", "dV"):
        assert np.allclose(a[k], b[k], rtol=1e-12, atol=1e-14), k
