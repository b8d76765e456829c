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


def _bf16(a):
    """Round to bfloat16 (round to nearest even, through float32) and back to
    float64: the storage precision of the chunk computation's k, v, q."""
    import torch
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def mixer_inputs(x, wqkv, bias, eta_base, alpha_base, tau, H, D):
    """The E2-TTT token mixer's per-token inputs from the layer input x [T, dm]
    ([P3] 方法细节, 混合模型架构设计 and 依赖于输入的动态参数化): one
    projection x wqkv^T gives shared queries, keys and values (H heads of D)
    and three scalar logits per head (rows of wqkv in that order, plus bias);
    the TTT path takes q, k through SiLU and L2 normalisation over each head;
      eta_t = eta_base sigma(z_eta),  beta_t = sigma(z_beta)^(1 / tau),
      alpha_t = alpha_base sigma(z_alpha),  gamma_t = 1 - eta_t alpha_t.
    Returns q, k, v [H, T, D] (bfloat16 values, the chunk computation's input
    precision) and eta, beta, gamma [H, T] (float32 values)."""
    x = np.asarray(x, np.float64)
    P = x @ np.asarray(wqkv, np.float64).T
    T = x.shape[0]
    HD = H * D

    def heads(a):
        return a.reshape(T, H, D).transpose(1, 0, 2)

    def silu_l2(a):
        a = a / (1.0 + np.exp(-a))
        return a / np.linalg.norm(a, axis=-1, keepdims=True)
    q = silu_l2(heads(P[:, :HD]))
    k = silu_l2(heads(P[:, HD:2 * HD]))
    v = heads(P[:, 2 * HD:3 * HD])
    z = P[:, 3 * HD:3 * HD + 3 * H] + np.asarray(bias, np.float64)
    sig = 1.0 / (1.0 + np.exp(-z))
    eta = eta_base * sig[:, :H]
    beta = sig[:, H:2 * H] ** (1.0 / tau)
    alpha = alpha_base * sig[:, 2 * H:]
    gamma = 1.0 - eta * alpha
    f32 = lambda a: np.asarray(a.T, np.float32).astype(np.float64)
    return _bf16(q), _bf16(k), _bf16(v), f32(eta), f32(beta), f32(gamma)


def e2_mixer(x, wqkv, bias, eta_base, alpha_base, tau, W, M, H, D, C, sign=-1.0):
    """The E2-TTT token mixer's TTT path with a linear fast weight, chunk by
    chunk ([P3] Algorithm 1): outputs o_t = W q_t with W the state at the
    start of t's chunk (line 1), then the chunk-end state by Proposition 3.1
    (lines 2-7), with the page's G_t, the negative gradient of
    1/2 ||W0 k_t - v_t||^2 (sign = -1; descent). Returns (outputs [T, H, D],
    final W, final M)."""
    q, k, v, eta, beta, gamma = mixer_inputs(x, wqkv, bias, eta_base, alpha_base, tau, H, D)
    T = q.shape[1]
    W = np.array(W, np.float64)
    M = np.array(M, np.float64)
    out = np.zeros((T, H, D))
    for a in range(0, T, C):
        e = min(T, a + C)
        for h in range(H):
            out[a:e, h] = q[h, a:e] @ W[h].T
        W, M = e2_closed_form(k[:, a:e], v[:, a:e], eta[:, a:e], beta[:, a:e], gamma[:, a:e], W, M, e - a, sign)
    return out, W, M
