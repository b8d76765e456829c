"""Pins of the oracle's step functions against textbook definitions, library
routines and invariants (CPU only)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import ttt_e2e as O

rng = np.random.default_rng(0)


def t64(a, grad=False):
    return torch.tensor(a, dtype=torch.float64, requires_grad=grad)


def test_rmsnorm_matches_library_and_unit_rms():
    x = rng.standard_normal((7, 32))
    g = rng.standard_normal(32)
    y, r = O.rmsnorm(x, g, 1e-5)
    ref = Fn.rms_norm(t64(x), (32,), weight=t64(g), eps=1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    y1, _ = O.rmsnorm(x, np.ones(32), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y1 ** 2, axis=1)), 1.0, rtol=1e-13)


def test_rmsnorm_bwd_matches_autograd():
    x = rng.standard_normal((5, 24))
    g = rng.standard_normal(24)
    dy = rng.standard_normal((5, 24))
    _, r = O.rmsnorm(x, g, 1e-5)
    dx = O.rmsnorm_bwd(dy, x, g, r)
    xt = t64(x, True)
    y = Fn.rms_norm(xt, (24,), weight=t64(g), eps=1e-5)
    (y * t64(dy)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_swiglu_fwd_bwd_match_autograd():
    u = rng.standard_normal((6, 16))
    w1, w2 = rng.standard_normal((40, 16)), rng.standard_normal((40, 16))
    w3 = rng.standard_normal((16, 40))
    dy = rng.standard_normal((6, 16))
    y, cache = O.swiglu(u, w1, w2, w3)
    du, g1, g2, g3 = O.swiglu_bwd(dy, cache, w1, w2, w3)
    ts = [t64(a, True) for a in (u, w1, w2, w3)]
    yt = (Fn.silu(ts[0] @ ts[1].T) * (ts[0] @ ts[2].T)) @ ts[3].T
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12)
    (yt * t64(dy)).sum().backward()
    for mine, ref in zip((du, g1, g2, g3), ts):
        np.testing.assert_allclose(mine, ref.grad.numpy(), rtol=1e-11, atol=1e-11)


def test_rope_identities():
    dh = 16
    x = rng.standard_normal((9, 3, dh))
    pos = np.arange(9) * 1000 + 3
    y = O.rope(x, pos, 10000.0)
    # position 0 is the identity
    np.testing.assert_allclose(O.rope(x[:1], np.array([0]), 10000.0), x[:1], rtol=0, atol=0)
    # rotations preserve the norm of every head vector
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # the inverse rotation undoes it
    np.testing.assert_allclose(O.rope(y, pos, 10000.0, inverse=True), x, rtol=1e-12, atol=1e-12)
    # closed form: pairs (x_j, x_{j+dh/2}) form the complex number x_j + i x_{j+dh/2},
    # multiplied by exp(i pos theta^(-2j/dh))
    z = (x[..., : dh // 2] + 1j * x[..., dh // 2:]) * np.exp(
        1j * pos[:, None, None] * (10000.0 ** (-2.0 * np.arange(dh // 2) / dh)))
    np.testing.assert_allclose(y[..., : dh // 2], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[..., dh // 2:], z.imag, rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    dh = 32
    q = rng.standard_normal((1, 1, dh))
    k = rng.standard_normal((1, 1, dh))
    def score(i, j):
        return float(np.sum(O.rope(q, np.array([i]), 10000.0) * O.rope(k, np.array([j]), 10000.0)))
    assert score(7, 3) == pytest.approx(score(1007, 1003), rel=1e-10)
    assert score(131071, 131000) == pytest.approx(score(71, 0), rel=1e-9)


def _sdpa_ref(q, K, V, qpos, kpos, window, grad=False):
    """Library attention with an explicit boolean mask (GQA by repetition)."""
    n, H, dh = q.shape
    g = H // K.shape[1]
    qt = t64(q, grad)
    Kt = t64(K, grad)
    Vt = t64(V, grad)
    Kr = Kt.repeat_interleave(g, dim=1)
    Vr = Vt.repeat_interleave(g, dim=1)
    m = torch.tensor((kpos[None, :] <= qpos[:, None]) & (kpos[None, :] > qpos[:, None] - window))
    o = Fn.scaled_dot_product_attention(qt.transpose(0, 1), Kr.transpose(0, 1), Vr.transpose(0, 1),
                                        attn_mask=m)
    return o.transpose(0, 1), (qt, Kt, Vt)


@pytest.mark.parametrize("H,Hk", [(4, 4), (6, 2)])
def test_swa_full_window_is_causal_softmax_attention(H, Hk):
    T, dh = 20, 8
    q = rng.standard_normal((T, H, dh))
    K = rng.standard_normal((T, Hk, dh))
    V = rng.standard_normal((T, Hk, dh))
    pos = np.arange(T)
    o, _ = O.swa_attention(q, pos, K, V, pos, window=T)
    qt = t64(q).transpose(0, 1)
    Kr = t64(K).repeat_interleave(H // Hk, 1).transpose(0, 1)
    Vr = t64(V).repeat_interleave(H // Hk, 1).transpose(0, 1)
    ref = Fn.scaled_dot_product_attention(qt, Kr, Vr, is_causal=True).transpose(0, 1).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_swa_window_one_returns_own_value_and_window_masks():
    T, H, dh = 12, 2, 4
    q = rng.standard_normal((T, H, dh))
    K = rng.standard_normal((T, H, dh))
    V = rng.standard_normal((T, H, dh))
    pos = np.arange(T)
    o, _ = O.swa_attention(q, pos, K, V, pos, window=1)
    np.testing.assert_allclose(o, V, rtol=0, atol=1e-15)
    o5, _ = O.swa_attention(q, pos, K, V, pos, window=5)
    ref, _ = _sdpa_ref(q, K, V, pos, pos, 5)
    np.testing.assert_allclose(o5, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_swa_bwd_matches_autograd_with_constant_keys():
    n, m, H, Hk, dh, win = 6, 14, 4, 2, 8, 10
    qpos = np.arange(8, 14)
    kpos = np.arange(0, 14)
    q = rng.standard_normal((n, H, dh))
    K = rng.standard_normal((m, Hk, dh))
    V = rng.standard_normal((m, Hk, dh))
    do = rng.standard_normal((n, H, dh))
    o, P = O.swa_attention(q, qpos, K, V, kpos, win)
    grad_keys = kpos >= 8
    dq, dK, dV = O.swa_attention_bwd(do, q, K, V, P, grad_keys)
    ref, (qt, Kt, Vt) = _sdpa_ref(q, K, V, qpos, kpos, win, grad=True)
    np.testing.assert_allclose(o, ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    (ref * t64(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dK[grad_keys], Kt.grad.numpy()[grad_keys], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dV[grad_keys], Vt.grad.numpy()[grad_keys], rtol=1e-11, atol=1e-11)
    assert np.all(dK[~grad_keys] == 0) and np.all(dV[~grad_keys] == 0)


def test_cross_entropy_matches_library_and_grad_rows_sum_to_zero():
    z = rng.standard_normal((9, 50)) * 3
    lab = rng.integers(0, 50, 9)
    loss, p = O.cross_entropy(z, lab)
    ref = Fn.cross_entropy(t64(z), torch.tensor(lab), reduction="none").numpy()
    np.testing.assert_allclose(loss, ref, rtol=1e-13)
    dz = p.copy()
    dz[np.arange(9), lab] -= 1
    np.testing.assert_allclose(dz.sum(1), 0.0, atol=1e-14)
    zt = t64(z, True)
    Fn.cross_entropy(zt, torch.tensor(lab), reduction="sum").backward()
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=1e-12, atol=1e-14)
