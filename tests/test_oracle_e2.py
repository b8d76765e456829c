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
