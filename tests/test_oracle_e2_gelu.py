"""Pins of the GELU fast-weight E2-TTT oracle (CPU only): GELU and its
derivative against the library's exact GELU and autograd, the per-token
gradients against finite differences of the loss, the chunk-end closed form
against the per-token recursion, and the special cases the formula fixes."""
import numpy as np
import pytest
import torch

import synth
from oracle import e2ttt_gelu as G


def _W(rng, D, Dh, w2_scale=None):
    s2 = 1.0 / np.sqrt(Dh) if w2_scale is None else w2_scale
    return {"w1": rng.normal(size=(Dh, D)), "w2": rng.normal(size=(D, Dh)) * s2}


def _fd(W, k, v, m, eps=1e-6):
    fd = np.zeros_like(W[m])
    for i in range(W[m].shape[0]):
        for j in range(W[m].shape[1]):
            Wp = {a: b.copy() for a, b in W.items()}
            Wm = {a: b.copy() for a, b in W.items()}
            Wp[m][i, j] += eps
            Wm[m][i, j] -= eps
            fd[i, j] = (G.fw_loss(Wp, k, v) - G.fw_loss(Wm, k, v)) / (2 * eps)
    return fd


def test_gelu_and_its_derivative_match_the_library():
    u = np.linspace(-6.0, 6.0, 241)
    ut = torch.from_numpy(u).requires_grad_(True)
    y = torch.nn.functional.gelu(ut, approximate="none")
    assert np.max(np.abs(G.gelu(u) - y.detach().numpy())) < 1e-14
    y.sum().backward()
    assert np.max(np.abs(G.gelu_grad(u) - ut.grad.numpy())) < 1e-14


@pytest.mark.parametrize("m", G.MATS)
def test_gradients_match_finite_differences(m):
    rng = np.random.default_rng(13)
    W = _W(rng, 4, 6)
    k, v = rng.normal(size=(5, 4)), rng.normal(size=(5, 4))
    l, r = G._grads(W, k, v)[m]
    fd = _fd(W, k, v, m)
    assert np.max(np.abs(l.T @ r - fd)) <= 1e-7 * np.max(np.abs(fd))


def test_planted_mistake_in_gelu_derivative_fails_the_pin(monkeypatch):
    """Keeping only Phi(u) of GELU' (dropping u phi(u), a plausible slip)
    breaks the finite-difference agreement of grad_{w1}."""
    from scipy.special import erf
    monkeypatch.setattr(G, "gelu_grad", lambda u: 0.5 * (1.0 + erf(u / np.sqrt(2.0))))
    rng = np.random.default_rng(13)
    W = _W(rng, 4, 6)
    k, v = rng.normal(size=(5, 4)), rng.normal(size=(5, 4))
    l, r = G._grads(W, k, v)["w1"]
    fd = _fd(W, k, v, "w1")
    assert np.max(np.abs(l.T @ r - fd)) > 1e-3 * np.max(np.abs(fd))


def _state(rng, H, D, Dh, M0):
    W = [_W(rng, D, Dh) for _ in range(H)]
    M = [{m: (rng.normal(size=W[0][m].shape) * 0.01 if M0 else np.zeros(W[0][m].shape)) for m in G.MATS}
         for _ in range(H)]
    return W, M


@pytest.mark.parametrize("sign", [1.0, -1.0])
@pytest.mark.parametrize("M0", [False, True])
@pytest.mark.parametrize("C", [1, 8, 37])
def test_closed_form_equals_sequential(sign, M0, C):
    """Proposition 3.1 per matrix reproduces the per-token recursion at every
    chunk end, ragged last chunk included."""
    H, T, D, Dh = 2, 37, 6, 8
    g = synth.gen_e2(H, T, D, 23)
    k, v = g["k"].double().numpy(), g["v"].double().numpy()
    eta, beta, gamma = (g[n].double().numpy() for n in ("eta", "beta", "gamma"))
    eta = eta * 1e-2
    W, M = _state(np.random.default_rng(15), H, D, Dh, M0)
    Ws, Ms = G.e2_gelu_sequential(k, v, eta, beta, gamma, W, M, C, sign)
    Wc, Mc = G.e2_gelu_closed_form(k, v, eta, beta, gamma, W, M, C, sign)
    for h in range(H):
        for m in G.MATS:
            assert np.max(np.abs(Wc[h][m] - Ws[h][m])) <= 1e-11 * np.max(np.abs(Ws[h][m]))
            assert np.max(np.abs(Mc[h][m] - Ms[h][m])) <= 1e-11 * np.max(np.abs(Ms[h][m]))


def test_zero_output_matrix_gives_identity_and_no_first_layer_gradient():
    """W2 = 0: LN(0) = 0, so f(x) = x, and no gradient reaches W1."""
    rng = np.random.default_rng(16)
    W = _W(rng, 5, 8, w2_scale=0.0)
    k, v = rng.normal(size=(4, 5)), rng.normal(size=(4, 5))
    f, _ = G.fw_forward(W, k)
    assert np.array_equal(f, k)
    g = G._grads(W, k, v)
    assert np.max(np.abs(g["w1"][0])) == 0.0
    assert np.max(np.abs(g["w2"][0])) > 0.0


def test_mixer_without_learning_keeps_state_and_outputs_f_W0():
    """eta_base = 0: gamma = 1, no gradient enters, M0 = 0 stays 0, so the
    state is unchanged and every output is f_W0(q_t)."""
    H, T, D, dm, C, Dh = 2, 100, 64, 128, 32, 64
    g = synth.gen_e2_mixer(H, T, D, dm, 18)
    W, M = _state(np.random.default_rng(17), H, D, Dh, False)
    x, wqkv, bias = g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy()
    out, Wn, Mn = G.e2_gelu_mixer(x, wqkv, bias, 0.0, 0.5, 4.0, W, M, H, D, C)
    q = G._mlp.mixer_inputs(x, wqkv, bias, 0.0, 0.5, 4.0, H, D)[0]
    for h in range(H):
        for m in G.MATS:
            assert np.array_equal(Wn[h][m], W[h][m])
            assert np.array_equal(Mn[h][m], M[h][m])
        f, _ = G.fw_forward(W[h], q[h])
        assert np.max(np.abs(out[:, h] - f)) < 1e-12


def test_outputs_use_the_chunk_start_state():
    """Outputs of chunk r equal f under the state after chunks 0..r-1."""
    H, T, D, dm, C, Dh = 1, 96, 64, 128, 32, 64
    g = synth.gen_e2_mixer(H, T, D, dm, 19)
    W, M = _state(np.random.default_rng(18), H, D, Dh, False)
    x, wqkv, bias = g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy()
    out, _, _ = G.e2_gelu_mixer(x, wqkv, bias, 1e-3, 0.5, 4.0, W, M, H, D, C)
    q, k, v, eta, beta, gamma = G._mlp.mixer_inputs(x, wqkv, bias, 1e-3, 0.5, 4.0, H, D)
    W2, _ = G.e2_gelu_closed_form(k[:, :64], v[:, :64], eta[:, :64], beta[:, :64], gamma[:, :64], W, M, C)
    f, _ = G.fw_forward(W2[0], q[0, 64:])
    assert np.max(np.abs(out[64:, 0] - f)) < 1e-12
