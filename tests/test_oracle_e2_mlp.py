"""Pins of the SwiGLU fast-weight E2-TTT oracle (CPU only): the per-token
gradients against finite differences of the loss, the layer normalisation
against the library's, the chunk-end closed form against the per-token
recursion, and the special cases the formula fixes."""
import numpy as np
import pytest
import torch

import synth
from oracle import e2ttt_mlp as X


def _W(rng, D, Dh, w3_scale=None):
    s3 = 1.0 / np.sqrt(Dh) if w3_scale is None else w3_scale
    return {"w1": rng.normal(size=(Dh, D)), "w2": rng.normal(size=(Dh, D)), "w3": rng.normal(size=(D, Dh)) * s3}


def _fd(W, k, v, m, eps=1e-6):
    fd = np.zeros_like(W[m])
    for i in range(W[m].shape[0]):
        for j in range(W[m].shape[1]):
            Wp = {a: b.copy() for a, b in W.items()}
            Wm = {a: b.copy() for a, b in W.items()}
            Wp[m][i, j] += eps
            Wm[m][i, j] -= eps
            fd[i, j] = (X.fw_loss(Wp, k, v) - X.fw_loss(Wm, k, v)) / (2 * eps)
    return fd


@pytest.mark.parametrize("m", X.MATS)
def test_gradients_match_finite_differences(m):
    rng = np.random.default_rng(3)
    W = _W(rng, 4, 6)
    k, v = rng.normal(size=(5, 4)), rng.normal(size=(5, 4))
    l, r = X._grads(W, k, v)[m]
    fd = _fd(W, k, v, m)
    assert np.max(np.abs(l.T @ r - fd)) <= 1e-7 * np.max(np.abs(fd))


def test_planted_mistake_in_swiglu_derivative_fails_the_pin(monkeypatch):
    """Dropping the SiLU derivative's second term (a plausible slip) breaks
    the finite-difference agreement of grad_{w1}."""
    def wrong(W, k, v):
        f, (a1, a2, s, h, z, r) = X.fw_forward(W, k)
        dy = X.layer_norm_bwd(f - v, z, r)
        dh = dy @ W["w3"]
        return dy, h, dh * a2 * s, dh * a1 * s
    rng = np.random.default_rng(3)
    W = _W(rng, 4, 6)
    k, v = rng.normal(size=(5, 4)), rng.normal(size=(5, 4))
    monkeypatch.setattr(X, "fw_grad_factors", wrong)
    l, r = X._grads(W, k, v)["w1"]
    fd = _fd(W, k, v, "w1")
    assert np.max(np.abs(l.T @ r - fd)) > 1e-3 * np.max(np.abs(fd))


def test_layer_norm_matches_library():
    rng = np.random.default_rng(4)
    y = rng.normal(size=(7, 16)) * 3 + 1
    z, r = X.layer_norm(y)
    zt = torch.nn.functional.layer_norm(torch.from_numpy(y), (16,), eps=X.EPS).numpy()
    assert np.max(np.abs(z - zt)) < 1e-12
    # its backward against the library's autograd
    yt = torch.from_numpy(y).requires_grad_(True)
    dz = rng.normal(size=y.shape)
    torch.nn.functional.layer_norm(yt, (16,), eps=X.EPS).backward(torch.from_numpy(dz))
    assert np.max(np.abs(X.layer_norm_bwd(dz, z, r) - yt.grad.numpy())) < 1e-12


def _state(rng, H, D, Dh, M0):
    W = [_W(rng, D, Dh) for _ in range(H)]
    M = [{m: (rng.normal(size=W[0][m].shape) * 0.01 if M0 else np.zeros(W[0][m].shape)) for m in X.MATS}
         for _ in range(H)]
    return W, M


@pytest.mark.parametrize("sign", [1.0, -1.0])
@pytest.mark.parametrize("M0", [False, True])
@pytest.mark.parametrize("C", [1, 8, 13, 37])
def test_closed_form_equals_sequential(sign, M0, C):
    """Proposition 3.1 per matrix reproduces the per-token recursion at every
    chunk end (gradients at the chunk-start weights), ragged last chunk
    included; C = 1 is per-token online SGD with momentum and decay."""
    H, T, D, Dh = 2, 37, 6, 8
    g = synth.gen_e2(H, T, D, 21)
    k, v = g["k"].double().numpy(), g["v"].double().numpy()
    eta, beta, gamma = (g[n].double().numpy() for n in ("eta", "beta", "gamma"))
    eta = eta * 1e-2
    W, M = _state(np.random.default_rng(5), H, D, Dh, M0)
    Ws, Ms = X.e2_mlp_sequential(k, v, eta, beta, gamma, W, M, C, sign)
    Wc, Mc = X.e2_mlp_closed_form(k, v, eta, beta, gamma, W, M, C, sign)
    for h in range(H):
        for m in X.MATS:
            assert np.max(np.abs(Wc[h][m] - Ws[h][m])) <= 1e-11 * np.max(np.abs(Ws[h][m]))
            assert np.max(np.abs(Mc[h][m] - Ms[h][m])) <= 1e-11 * np.max(np.abs(Ms[h][m]))


def test_zero_output_matrix_gives_identity_and_no_first_layer_gradient():
    """W3 = 0: LN(0) = 0, so f(x) = x, and no gradient reaches W1, W2."""
    rng = np.random.default_rng(6)
    W = _W(rng, 5, 8, w3_scale=0.0)
    k, v = rng.normal(size=(4, 5)), rng.normal(size=(4, 5))
    f, _ = X.fw_forward(W, k)
    assert np.array_equal(f, k)
    G = X._grads(W, k, v)
    for m in ("w1", "w2"):
        assert np.max(np.abs(G[m][0])) == 0.0
    assert np.max(np.abs(G["w3"][0])) > 0.0


def test_mixer_without_learning_keeps_state_and_outputs_f_W0():
    """eta_base = 0: gamma = 1, no gradient enters, M0 = 0 stays 0, so the
    state is unchanged and every output is f_W0(q_t)."""
    H, T, D, dm, C, Dh = 2, 100, 64, 128, 32, 64
    g = synth.gen_e2_mixer(H, T, D, dm, 8)
    W, M = _state(np.random.default_rng(7), H, D, Dh, False)
    x, wqkv, bias = g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy()
    out, Wn, Mn = X.e2_mlp_mixer(x, wqkv, bias, 0.0, 0.5, 4.0, W, M, H, D, C)
    q = X.mixer_inputs(x, wqkv, bias, 0.0, 0.5, 4.0, H, D)[0]
    for h in range(H):
        for m in X.MATS:
            assert np.array_equal(Wn[h][m], W[h][m])
            assert np.array_equal(Mn[h][m], M[h][m])
        f, _ = X.fw_forward(W[h], q[h])
        assert np.max(np.abs(out[:, h] - f)) < 1e-12


def test_outputs_use_the_chunk_start_state():
    """Outputs of chunk r equal f under the state after chunks 0..r-1 (the
    closed form applied to the earlier tokens)."""
    H, T, D, dm, C, Dh = 1, 96, 64, 128, 32, 64
    g = synth.gen_e2_mixer(H, T, D, dm, 9)
    W, M = _state(np.random.default_rng(8), H, D, Dh, False)
    x, wqkv, bias = g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy()
    out, _, _ = X.e2_mlp_mixer(x, wqkv, bias, 1e-3, 0.5, 4.0, W, M, H, D, C)
    q, k, v, eta, beta, gamma = X.mixer_inputs(x, wqkv, bias, 1e-3, 0.5, 4.0, H, D)
    W2, _ = X.e2_mlp_closed_form(k[:, :64], v[:, :64], eta[:, :64], beta[:, :64], gamma[:, :64], W, M, C)
    f, _ = X.fw_forward(W2[0], q[0, 64:])
    assert np.max(np.abs(out[64:, 0] - f)) < 1e-12
