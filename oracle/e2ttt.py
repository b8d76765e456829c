"""E2-TTT chunk-end state: per-token recursion and its closed form
(test infrastructure only).

Source: [P3] "Rethinking Expressivity and Efficiency in Test-Time Training"
(papercache digest of E2-TTT), section 方法细节: the target per-token recursion
with coupled momentum and decay, the unrolled closed form, the suffix products
and ratio sum, Proposition 3.1 (chunk-end W_C, M_C); section 附录细节: the
unrolled derivation and the near-unit-retention limit R_t -> C - t + 1.

The fast weight is linear, f_W(k) = W k, and (as the workload states) the
per-token gradient is taken at the chunk-start W0:
    G_t = (W0 k_t - v_t) k_t^T
(the gradient of 1/2 ||W0 k_t - v_t||^2; the page's G_t is its negative and
the identity is linear in G, so both signs are exercised by the pins).
Everything here is float64 on the bf16-valued k, v and fp32-valued scalars.

The chunk-wise baseline the page compares against (section 背景知识, LaCT's
large-chunk rule, and the "chunk-averaged" ablation of 实验结果) is
lact_chunked: one update direction per chunk from the eta-weighted gradients
at the chunk-start W0, a chunk-level momentum factor equal to the mean of the
chunk's beta_t, and no decay.
"""
from __future__ import annotations

import numpy as np


def _grad_terms(W0, k, v, sign):
    """Rows e_t = W0 k_t - v_t ([C, D]) so that G_t = sign * e_t k_t^T."""
    return sign * (k @ W0.T - v)


def e2_sequential(k, v, eta, beta, gamma, W, M, C, sign=1.0):
    """Per-token recursion, chunk by chunk:
         M_t = beta_t M_{t-1} + eta_t G_t,   W_t = gamma_t W_{t-1} + M_t,
    with G_t evaluated at the chunk-start W0. k, v [H, T, D]; eta, beta, gamma
    [H, T]; W, M [H, D, D]. Returns final (W, M)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    eta, beta, gamma = (np.asarray(x, np.float64) for x in (eta, beta, gamma))
    W = np.array(W, np.float64)
    M = np.array(M, np.float64)
    H, T, D = k.shape
    for h in range(H):
        for a in range(0, T, C):
            e = min(T, a + C)
            W0 = W[h].copy()
            E = _grad_terms(W0, k[h, a:e], v[h, a:e], sign)
            for t in range(e - a):
                G = np.outer(E[t], k[h, a + t])
                M[h] = beta[h, a + t] * M[h] + eta[h, a + t] * G
                W[h] = gamma[h, a + t] * W[h] + M[h]
    return W, M


def chunk_scalars(eta, beta, gamma):
    """Suffix products and ratio sum of one chunk (t = 1..C, stored 0-based):
         beta~_t = prod_{i=t+1}^{C} beta_i,  gamma~_t likewise  (t = 0..C),
         R_t = sum_{i=t}^{C} gamma~_i / beta~_i,
         K^M_t = eta_t beta~_t,  K^W_t = eta_t beta~_t R_t.
    Returns (bt [C+1], gt [C+1], R [C+1] with R[0] unused, KM [C], KW [C])."""
    C = len(eta)
    bt = np.ones(C + 1)
    gt = np.ones(C + 1)
    for t in range(C - 1, -1, -1):           # bt[t] = beta_{t+1} * bt[t+1]
        bt[t] = beta[t] * bt[t + 1]
        gt[t] = gamma[t] * gt[t + 1]
    R = np.zeros(C + 2)
    for t in range(C, 0, -1):
        R[t] = gt[t] / bt[t] + R[t + 1]
    KM = eta * bt[1:]
    KW = eta * bt[1:] * R[1:C + 1]
    return bt, gt, R[:C + 1], KM, KW


def e2_closed_form(k, v, eta, beta, gamma, W, M, C, sign=1.0):
    """Proposition 3.1 applied chunk by chunk:
         M_C = beta~_0 M_0 + sum_t K^M_t G_t,
         W_C = gamma~_0 W_0 + beta~_0 R_1 M_0 + sum_t K^W_t G_t.
    The aggregations are sum_t K_t e_t k_t^T = (diag(K) E)^T K."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    eta, beta, gamma = (np.asarray(x, np.float64) for x in (eta, beta, gamma))
    W = np.array(W, np.float64)
    M = np.array(M, np.float64)
    H, T, D = k.shape
    for h in range(H):
        for a in range(0, T, C):
            e = min(T, a + C)
            W0, M0 = W[h].copy(), M[h].copy()
            bt, gt, R, KM, KW = chunk_scalars(eta[h, a:e], beta[h, a:e], gamma[h, a:e])
            E = _grad_terms(W0, k[h, a:e], v[h, a:e], sign)
            dW = (E * KW[:, None]).T @ k[h, a:e]
            dM = (E * KM[:, None]).T @ k[h, a:e]
            W[h] = gt[0] * W0 + bt[0] * R[1] * M0 + dW
            M[h] = bt[0] * M0 + dM
    return W, M


def lact_chunked(k, v, eta, beta, W, M, C, sign=1.0):
    """LaCT's chunk-wise update, chunk by chunk ([P3] 背景知识):
         G = sum_t eta_t G_t   (G_t = sign (W0 k_t - v_t) k_t^T at the chunk-start W0),
         M <- mean_t(beta_t) M + G,   W <- W + M.
    k, v [H, T, D]; eta, beta [H, T]; W, M [H, D, D]. Returns final (W, M)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    eta, beta = (np.asarray(x, np.float64) for x in (eta, beta))
    W = np.array(W, np.float64)
    M = np.array(M, np.float64)
    H, T, D = k.shape
    for h in range(H):
        for a in range(0, T, C):
            e = min(T, a + C)
            E = _grad_terms(W[h], k[h, a:e], v[h, a:e], sign)
            G = (E * eta[h, a:e, None]).T @ k[h, a:e]
            M[h] = np.mean(beta[h, a:e]) * M[h] + G
            W[h] = W[h] + M[h]
    return W, M
