"""Pins of the E2-TTT oracle (CPU only): the closed form against the per-token
recursion, and the special cases the page states."""
import numpy as np
import pytest

import synth
from oracle import e2ttt as E


def _inputs(H=2, T=96, D=8, seed=11, M0=False):
    g = synth.gen_e2(H, T, D, seed)
    k, v = g["k"].float().numpy(), g["v"].float().numpy()
    eta, beta, gamma = g["eta"].numpy(), g["beta"].numpy(), g["gamma"].numpy()
    W = g["W"].numpy()
    M = np.random.default_rng(seed).standard_normal(W.shape) * 0.01 if M0 else g["M"].numpy()
    return k, v, eta, beta, gamma, W, M


@pytest.mark.parametrize("sign", [1.0, -1.0])
@pytest.mark.parametrize("M0", [False, True])
@pytest.mark.parametrize("C", [32, 40, 96])
def test_closed_form_equals_sequential(sign, M0, C):
    k, v, eta, beta, gamma, W, M = _inputs(M0=M0)
    Ws, Ms = E.e2_sequential(k, v, eta, beta, gamma, W, M, C, sign)
    Wc, Mc = E.e2_closed_form(k, v, eta, beta, gamma, W, M, C, sign)
    assert np.max(np.abs(Wc - Ws)) <= 1e-12 * np.max(np.abs(Ws))
    assert np.max(np.abs(Mc - Ms)) <= 1e-12 * np.max(np.abs(Ms))


def test_unit_retention_gives_linear_ratio_sum():
    """beta = gamma = 1: R_t = C - t + 1 and
    W_C = W0 + C M0 + sum_t eta_t (C - t + 1) G_t."""
    C, D = 24, 6
    k, v, eta, _, _, W, M = _inputs(H=1, T=C, D=D, M0=True)
    eta = eta.astype(np.float64)
    one = np.ones_like(eta)
    bt, gt, R, KM, KW = E.chunk_scalars(eta[0], one[0], one[0])
    t = np.arange(1, C + 1)
    np.testing.assert_allclose(R[1:], C - t + 1, rtol=0, atol=0)
    Wc, Mc = E.e2_closed_form(k, v, eta, one, one, W, M, C)
    kk, vv = k[0].astype(np.float64), v[0].astype(np.float64)
    G = [np.outer(W[0] @ kk[i] - vv[i], kk[i]) for i in range(C)]
    ref = W[0] + C * M[0] + sum(eta[0, i] * (C - i) * G[i] for i in range(C))
    np.testing.assert_allclose(Wc[0], ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(Mc[0], M[0] + sum(eta[0, i] * G[i] for i in range(C)), rtol=1e-12, atol=1e-15)


def test_chunk_of_one_token():
    """C = 1: W_1 = gamma_1 W0 + beta_1 M0 + eta_1 G_1, M_1 = beta_1 M0 + eta_1 G_1."""
    k, v, eta, beta, gamma, W, M = (np.asarray(x, np.float64) for x in _inputs(H=1, T=1, D=5, M0=True))
    Wc, Mc = E.e2_closed_form(k, v, eta, beta, gamma, W, M, 1)
    G = np.outer(W[0] @ k[0, 0] - v[0, 0], k[0, 0])
    np.testing.assert_allclose(Wc[0], gamma[0, 0] * W[0] + beta[0, 0] * M[0] + eta[0, 0] * G, rtol=1e-13)
    np.testing.assert_allclose(Mc[0], beta[0, 0] * M[0] + eta[0, 0] * G, rtol=1e-13)


def test_kernel_bound_and_underflow_scale():
    """beta, gamma in (0.9, 1): the weight kernel K^W_t = eta_t beta~_t R_t is
    bounded by eta_max * C (stability remark), while beta~_0 underflows fp32 at
    C = 2048 -- the reason a division-free form is needed in fp32."""
    g = synth.gen_e2(1, 2048, 4, 5)
    eta, beta, gamma = (g[x][0].numpy().astype(np.float64) for x in ("eta", "beta", "gamma"))
    bt, gt, R, KM, KW = E.chunk_scalars(eta, beta, gamma)
    assert np.all(KW <= eta.max() * 2048) and np.all(KW >= 0)
    assert bt[0] < 1.4e-45 * 1e3  # far below fp32's normal range


# ---------------------------------------------------------------- LaCT baseline
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_lact_with_one_token_chunks_is_the_per_token_recursion_without_decay(sign):
    """C = 1: the chunk mean of beta is beta_t itself and G = eta_t G_t, so the
    chunk rule is the per-token recursion with gamma = 1."""
    k, v, eta, beta, gamma, W, M = _inputs(H=2, T=23, D=6, M0=True)
    Wl, Ml = E.lact_chunked(k, v, eta, beta, W, M, 1, sign)
    Ws, Ms = E.e2_sequential(k, v, eta, beta, np.ones_like(gamma), W, M, 1, sign)
    np.testing.assert_allclose(Wl, Ws, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(Ml, Ms, rtol=1e-12, atol=1e-15)


def test_lact_update_direction_is_the_gradient_of_the_weighted_chunk_loss():
    """One chunk from M0 = 0: M_C = G = gradient at W0 of
    sum_t eta_t 1/2 ||W k_t - v_t||^2, checked entry by entry against central
    finite differences of that loss."""
    k, v, eta, beta, gamma, W, M = (np.asarray(x, np.float64) for x in _inputs(H=1, T=12, D=4))
    C = 12
    _, Mc = E.lact_chunked(k, v, eta, beta, W, np.zeros_like(W), C)

    def loss(Wm):
        r = k[0] @ Wm.T - v[0]
        return 0.5 * np.sum(eta[0][:, None] * r * r)
    eps = 1e-6
    fd = np.zeros((4, 4))
    for i in range(4):
        for j in range(4):
            dW = np.zeros((4, 4))
            dW[i, j] = eps
            fd[i, j] = (loss(W[0] + dW) - loss(W[0] - dW)) / (2 * eps)
    np.testing.assert_allclose(Mc[0], fd, rtol=1e-6, atol=1e-12)


def test_lact_without_learning_rate_is_a_geometric_series():
    """eta = 0 and a constant beta = b: M_r = b^r M0 and
    W_r = W0 + M0 (b - b^(r+1)) / (1 - b) after r chunks."""
    k, v, eta, beta, gamma, W, M = (np.asarray(x, np.float64) for x in _inputs(H=1, T=70, D=5, M0=True))
    b, C, r = 0.93, 16, 5   # 70 tokens: 4 full chunks and a ragged one
    Wl, Ml = E.lact_chunked(k, v, np.zeros_like(eta), np.full_like(beta, b), W, M, C)
    np.testing.assert_allclose(Ml[0], b ** r * M[0], rtol=1e-12)
    np.testing.assert_allclose(Wl[0], W[0] + M[0] * (b - b ** (r + 1)) / (1 - b), rtol=1e-12, atol=1e-15)


def test_lact_depends_on_beta_only_through_its_chunk_mean():
    """Permuting beta inside each chunk leaves the chunk rule unchanged (the
    per-token recursion does change), and a chunk whose beta are all b uses b."""
    k, v, eta, beta, gamma, W, M = (np.asarray(x, np.float64) for x in _inputs(H=2, T=64, D=5, M0=True))
    C = 16
    perm = np.concatenate([a + np.random.default_rng(3).permutation(C) for a in range(0, 64, C)])
    W1, M1 = E.lact_chunked(k, v, eta, beta, W, M, C)
    W2, M2 = E.lact_chunked(k, v, eta, beta[:, perm], W, M, C)
    np.testing.assert_allclose(W1, W2, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(M1, M2, rtol=1e-13, atol=1e-16)
    Ws1, _ = E.e2_sequential(k, v, eta, beta, np.ones_like(gamma), W, M, C)
    Ws2, _ = E.e2_sequential(k, v, eta, beta[:, perm], np.ones_like(gamma), W, M, C)
    assert np.max(np.abs(Ws1 - Ws2)) > 1e-6 * np.max(np.abs(Ws1))


# ---------------------------------------------------------------- token mixer
def _mixer_case(T=96, H=2, D=8, dm=12, seed=5):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, dm))
    wqkv = g.standard_normal((3 * H * D + 3 * H, dm)) / np.sqrt(dm)
    wqkv[2 * H * D:3 * H * D] /= np.sqrt(D)
    bias = np.concatenate([np.zeros(H), np.full(H, 3.0), np.zeros(H)])
    W = g.standard_normal((H, D, D)) * 0.02
    M = g.standard_normal((H, D, D)) * 0.01
    return x, wqkv, bias, W, M


def test_mixer_scalars_and_normalised_queries():
    """q, k have unit norm per head (up to their bf16 rounding); eta in
    (0, eta_base), beta in (0, 1) and closer to 1 than the plain sigmoid,
    gamma = 1 - eta alpha in (0, 1]."""
    x, wqkv, bias, W, M = _mixer_case()
    q, k, v, eta, beta, gamma = E.mixer_inputs(x, wqkv, bias, 0.1, 0.5, 4.0, 2, 8)
    for a in (q, k):
        np.testing.assert_allclose(np.linalg.norm(a, axis=-1), 1.0, atol=8e-3)
    assert np.all((eta > 0) & (eta < 0.1)) and np.all((beta > 0) & (beta < 1)) and np.all((gamma > 0) & (gamma <= 1))
    _, _, _, _, beta1, _ = E.mixer_inputs(x, wqkv, bias, 0.1, 0.5, 1.0, 2, 8)
    assert np.all(beta >= beta1)


def test_mixer_without_learning_keeps_the_initial_weights():
    """eta_base = 0 and M0 = 0: gamma = 1 and no gradient, so the state never
    changes and every output is W0 q_t."""
    x, wqkv, bias, W, M = _mixer_case()
    out, Wf, Mf = E.e2_mixer(x, wqkv, bias, 0.0, 0.5, 4.0, W, np.zeros_like(M), 2, 8, 32)
    q, *_ = E.mixer_inputs(x, wqkv, bias, 0.0, 0.5, 4.0, 2, 8)
    np.testing.assert_allclose(Wf, W, rtol=0, atol=0)
    np.testing.assert_allclose(out, np.einsum("htj,hij->thi", q, W), rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("C", [16, 40])
def test_mixer_outputs_use_the_state_at_the_start_of_their_chunk(C):
    """Outputs of chunk r equal W_r q_t, where W_r is the per-token
    recursion's state after the first r chunks (e2_sequential, an
    independent path)."""
    x, wqkv, bias, W, M = _mixer_case()
    H, D, T = 2, 8, 96
    out, Wf, Mf = E.e2_mixer(x, wqkv, bias, 0.1, 0.5, 4.0, W, M, H, D, C)
    q, k, v, eta, beta, gamma = E.mixer_inputs(x, wqkv, bias, 0.1, 0.5, 4.0, H, D)
    for a in range(0, T, C):
        Wa, _ = (E.e2_sequential(k[:, :a], v[:, :a], eta[:, :a], beta[:, :a], gamma[:, :a], W, M, C, -1.0)
                 if a else (W, M))
        e = min(T, a + C)
        np.testing.assert_allclose(out[a:e], np.einsum("htj,hij->thi", q[:, a:e], Wa), rtol=1e-10, atol=1e-13)
    Ws, Ms = E.e2_sequential(k, v, eta, beta, gamma, W, M, C, -1.0)
    np.testing.assert_allclose(Wf, Ws, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(Mf, Ms, rtol=1e-10, atol=1e-14)
