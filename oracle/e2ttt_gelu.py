"""E2-TTT with a GELU fast-weight network (test infrastructure only).

Source: [P3] "Rethinking Expressivity and Efficiency in Test-Time Training",
section 方法细节: 快速权重网络实例化 (the GELU MLP fast-weight net with a
residual connection and layer normalisation,
    f_W(x) = x + LN(W2 GELU(W1 x)) ),
with Proposition 3.1 and Algorithm 1 applied as for the SwiGLU net
(oracle/e2ttt_mlp.py, whose chunk-end machinery this module reuses).

Readings where the pages are silent (besides those of oracle/e2ttt_mlp.py:
LN without affine parameters, eps 1e-5; per-token loss 1/2 ||f - v||^2;
each matrix with its own momentum under the shared scalars):
  * GELU is the exact one, u Phi(u) with Phi the standard normal CDF.
  * W1 is [Dh, D] and W2 [D, Dh].
Everything is float64.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from oracle import e2ttt_mlp as _mlp
from oracle.e2ttt_mlp import layer_norm, layer_norm_bwd

MATS = ("w1", "w2")


def gelu(u):
    """u Phi(u) = u (1 + erf(u / sqrt 2)) / 2."""
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def gelu_grad(u):
    """d GELU / du = Phi(u) + u phi(u)."""
    return 0.5 * (1.0 + erf(u / math.sqrt(2.0))) + u * np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def fw_forward(W, x):
    """f_W(x) for rows x [n, D]; W = dict(w1 [Dh, D], w2 [D, Dh]).
    Returns (f [n, D], cache)."""
    u = x @ W["w1"].T
    a = gelu(u)
    y = a @ W["w2"].T
    z, r = layer_norm(y)
    return x + z, (u, a, z, r)


def fw_grad_factors(W, k, v):
    """Per-token gradient factors of L_t = 1/2 ||f_W(k_t) - v_t||^2:
    grad_{w2} L_t = dy_t a_t^T, grad_{w1} L_t = du_t k_t^T.
    Returns (dy, a, du)."""
    f, (u, a, z, r) = fw_forward(W, k)
    dy = layer_norm_bwd(f - v, z, r)
    du = (dy @ W["w2"]) * gelu_grad(u)
    return dy, a, du


def fw_loss(W, k, v):
    """Sum over the rows of 1/2 ||f_W(k_t) - v_t||^2."""
    f, _ = fw_forward(W, k)
    return 0.5 * float(np.sum((f - v) ** 2))


def _grads(W0, k, v):
    """Per-token gradients as (left factor, right factor) per matrix."""
    dy, a, du = fw_grad_factors(W0, k, v)
    return dict(w1=(du, k), w2=(dy, a))


def _net():
    import sys
    return _mlp.Net(sys.modules[__name__], MATS)


def e2_gelu_sequential(k, v, eta, beta, gamma, W, M, C, sign=-1.0):
    """The per-token recursion (e2_mlp_sequential) with the GELU net."""
    return _mlp.e2_mlp_sequential(k, v, eta, beta, gamma, W, M, C, sign, _net())


def e2_gelu_closed_form(k, v, eta, beta, gamma, W, M, C, sign=-1.0):
    """Proposition 3.1 chunk by chunk (e2_mlp_closed_form) with the GELU net."""
    return _mlp.e2_mlp_closed_form(k, v, eta, beta, gamma, W, M, C, sign, _net())


def e2_gelu_mixer(x, wqkv, bias, eta_base, alpha_base, tau, W, M, H, D, C, sign=-1.0):
    """The E2-TTT token mixer's TTT path (e2_mlp_mixer) with the GELU net:
    outputs o_t = f_W0(q_t) under each chunk's start state, then the
    chunk-end state of W1, W2. Returns (outputs [T, H, D], W, M)."""
    return _mlp.e2_mlp_mixer(x, wqkv, bias, eta_base, alpha_base, tau, W, M, H, D, C, sign, _net())
