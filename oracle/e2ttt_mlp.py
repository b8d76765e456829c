"""E2-TTT with a SwiGLU fast-weight network (test infrastructure only).

Source: [P3] "Rethinking Expressivity and Efficiency in Test-Time Training",
section 方法细节: 快速权重网络实例化 (the SwiGLU fast-weight net with a
residual connection and layer normalisation,
    f_W(x) = x + LN(W3 (SiLU(W1 x) * (W2 x))) ),
Proposition 3.1 and Algorithm 1 (each chunk's outputs under the chunk-start
state; the chunk-end state of every fast-weight matrix aggregated from the
per-token gradients taken at the chunk-start W0 with the shared scalar
kernels K^W_t, K^M_t), and section 附录细节 (the chain rule: the gradient of
L_t with respect to any matrix is a Jacobian that depends only on (W0, k_t)
applied to g_t = dL_t / df, so one backward serves both aggregations).

Readings where the pages are silent:
  * LN is a layer normalisation over the D features without affine
    parameters, eps = 1e-5.
  * The per-token loss is 1/2 ||f_W0(k_t) - v_t||^2, as for the linear fast
    weight, so g_t = f_W0(k_t) - v_t.
  * Each of W1, W2, W3 carries its own momentum and follows the recursion
    M_t = beta_t M_{t-1} + eta_t G_t, W_t = gamma_t W_{t-1} + M_t with the
    same scalars; G_t = sign * grad_W L_t at W0 (sign -1: descent).
Everything is float64.
"""
from __future__ import annotations

import numpy as np

from oracle.e2ttt import chunk_scalars, mixer_inputs

EPS = 1e-5
MATS = ("w1", "w2", "w3")


def layer_norm(y):
    """(y - mean) / sqrt(var + eps) over the last axis; returns (z, rstd)."""
    mu = y.mean(axis=-1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + EPS)
    return (y - mu) * r, r


def layer_norm_bwd(dz, z, r):
    """Gradient through layer_norm: rstd (dz - mean(dz) - z mean(dz z))."""
    return r * (dz - dz.mean(axis=-1, keepdims=True) - z * (dz * z).mean(axis=-1, keepdims=True))


def fw_forward(W, x):
    """f_W(x) for rows x [n, D]; W = dict(w1 [Dh, D], w2 [Dh, D], w3 [D, Dh]).
    Returns (f [n, D], cache)."""
    a1 = x @ W["w1"].T
    a2 = x @ W["w2"].T
    s = 1.0 / (1.0 + np.exp(-a1))
    h = a1 * s * a2
    y = h @ W["w3"].T
    z, r = layer_norm(y)
    return x + z, (a1, a2, s, h, z, r)


def fw_grad_factors(W, k, v):
    """Per-token gradient factors of L_t = 1/2 ||f_W(k_t) - v_t||^2:
    grad_{w3} L_t = dy_t h_t^T, grad_{w1} L_t = da1_t k_t^T,
    grad_{w2} L_t = da2_t k_t^T. Returns (dy, h, da1, da2)."""
    f, (a1, a2, s, h, z, r) = fw_forward(W, k)
    g = f - v
    dy = layer_norm_bwd(g, z, r)
    dh = dy @ W["w3"]
    da1 = dh * a2 * s * (1.0 + a1 * (1.0 - s))
    da2 = dh * a1 * s
    return dy, h, da1, da2


def fw_loss(W, k, v):
    """Sum over the rows of 1/2 ||f_W(k_t) - v_t||^2."""
    f, _ = fw_forward(W, k)
    return 0.5 * float(np.sum((f - v) ** 2))


def _grads(W0, k, v):
    """Per-token gradients as (left factor [n, rows], right factor [n, cols])
    per matrix: grad_t = outer(left_t, right_t)."""
    dy, h, da1, da2 = fw_grad_factors(W0, k, v)
    return dict(w1=(da1, k), w2=(da2, k), w3=(dy, h))


class Net:
    """A fast-weight net for the E2 machinery below: its matrix names, its
    forward f_W(x) -> (f, cache) and its per-token gradient factors
    grads(W0, k, v) -> {name: (left [n, rows], right [n, cols])}. The
    functions are looked up by name in their module at call time."""

    def __init__(self, module, mats):
        self.module, self.mats = module, mats

    def forward(self, W, x):
        return self.module.fw_forward(W, x)

    def grads(self, W0, k, v):
        return self.module._grads(W0, k, v)


def _copy(Ws, mats=MATS):
    return [{m: np.array(w[m], np.float64) for m in mats} for w in Ws]


def _net(net):
    import sys
    return net if net is not None else Net(sys.modules[__name__], MATS)


def e2_mlp_sequential(k, v, eta, beta, gamma, W, M, C, sign=-1.0, net=None):
    """Per-token recursion chunk by chunk with G_t = sign grad_W L_t at the
    chunk-start W0, for every matrix. k, v [H, T, D]; eta, beta, gamma
    [H, T]; W, M: lists (per head) of dicts of matrices; net: the
    fast-weight net (default: this module's SwiGLU net). Returns (W, M)."""
    net = _net(net)
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    eta, beta, gamma = (np.asarray(x, np.float64) for x in (eta, beta, gamma))
    W, M = _copy(W, net.mats), _copy(M, net.mats)
    H, T, _ = k.shape
    for h in range(H):
        for a in range(0, T, C):
            e = min(T, a + C)
            G = net.grads(_copy([W[h]], net.mats)[0], k[h, a:e], v[h, a:e])
            for t in range(e - a):
                for m in net.mats:
                    l, r = G[m]
                    M[h][m] = beta[h, a + t] * M[h][m] + eta[h, a + t] * sign * np.outer(l[t], r[t])
                    W[h][m] = gamma[h, a + t] * W[h][m] + M[h][m]
    return W, M


def e2_mlp_chunk(k, v, eta, beta, gamma, W0, M0, sign=-1.0, net=None):
    """Proposition 3.1 for one head and one chunk, every matrix with the
    same scalars: W_C = gamma~_0 W0 + beta~_0 R_1 M0 + sum_t K^W_t G_t,
    M_C = beta~_0 M0 + sum_t K^M_t G_t."""
    net = _net(net)
    bt, gt, R, KM, KW = chunk_scalars(eta, beta, gamma)
    G = net.grads(W0, k, v)
    W, M = {}, {}
    for m in net.mats:
        l, r = G[m]
        W[m] = gt[0] * W0[m] + bt[0] * R[1] * M0[m] + sign * (l * KW[:, None]).T @ r
        M[m] = bt[0] * M0[m] + sign * (l * KM[:, None]).T @ r
    return W, M


def e2_mlp_closed_form(k, v, eta, beta, gamma, W, M, C, sign=-1.0, net=None):
    """e2_mlp_chunk applied chunk by chunk to every head."""
    net = _net(net)
    k, v = np.asarray(k, np.float64), np.asarray(v, np.float64)
    eta, beta, gamma = (np.asarray(x, np.float64) for x in (eta, beta, gamma))
    W, M = _copy(W, net.mats), _copy(M, net.mats)
    H, T, _ = k.shape
    for h in range(H):
        for a in range(0, T, C):
            e = min(T, a + C)
            W[h], M[h] = e2_mlp_chunk(k[h, a:e], v[h, a:e], eta[h, a:e], beta[h, a:e], gamma[h, a:e],
                                      W[h], M[h], sign, net)
    return W, M


def e2_mlp_mixer(x, wqkv, bias, eta_base, alpha_base, tau, W, M, H, D, C, sign=-1.0, net=None):
    """The E2-TTT token mixer's TTT path with the SwiGLU fast-weight net,
    chunk by chunk ([P3] Algorithm 1): outputs o_t = f_W0(q_t) under the
    state at the start of t's chunk, then the chunk-end state of every
    matrix by Proposition 3.1 (descent). Inputs from mixer_inputs (bf16
    q, k, v; float32 scalars). W, M: lists (per head) of dicts. Returns
    (outputs [T, H, D], W, M)."""
    net = _net(net)
    q, k, v, eta, beta, gamma = mixer_inputs(x, wqkv, bias, eta_base, alpha_base, tau, H, D)
    T = q.shape[1]
    W, M = _copy(W, net.mats), _copy(M, net.mats)
    out = np.zeros((T, H, D))
    for a in range(0, T, C):
        e = min(T, a + C)
        for h in range(H):
            out[a:e, h], _ = net.forward(W[h], q[h, a:e])
            W[h], M[h] = e2_mlp_chunk(k[h, a:e], v[h, a:e], eta[h, a:e], beta[h, a:e], gamma[h, a:e],
                                      W[h], M[h], sign, net)
    return out, W, M
