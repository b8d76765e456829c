"""Independent re-implementation of the TTT-E2E inner loop with torch autograd
(test infrastructure only).

Written separately from ``ttt_e2e`` (its own forward, no shared helpers) and
differentiated by torch.autograd in float64 on the CPU, so that it pins the
hand-derived backward of ``ttt_e2e`` and its mini-batch bookkeeping. With
b = 1 it is per-token online SGD, the special case the method reduces to
when every token is its own step ([P1] "TTT-E2E：端到端测试时训练的长上下文语言建模",
section 持续学习框架: W_t = W_{t-1} - alpha grad l_t).

Semantics (same readings as the oracle): causal window i - k < t <= i;
K/V of each position computed once under its own mini-batch's fast weights
and then detached; position i predicts x_{i+1}; MEAN or SUM per mini-batch.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _t(a):
    return torch.as_tensor(np.asarray(a), dtype=torch.float64)


def ttt_loop_autograd(cfg: dict, weights, tokens, b=None, alpha=None, reduction=None):
    L = cfg["n_layers"]
    nd = cfg.get("n_dynamic", 0) or (L - (3 * L) // 4)
    s0 = L - nd
    H, Hk, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    k_win = cfg["window"]
    eps = cfg["rms_eps"]
    theta = cfg["rope_theta"]
    b = cfg["minibatch"] if b is None else b
    alpha = cfg["alpha"] if alpha is None else alpha
    reduction = cfg.get("reduction", "mean") if reduction is None else reduction

    E = _t(weights["embed"])
    LM = _t(weights["lm_head"])
    gf = _t(weights["final_norm"])
    lay = [{k: _t(v) for k, v in x.items()} for x in weights["layers"]]
    dnorm = [_t(x["norm"]) for x in weights["dyn"]]
    fast = [[_t(x["w1"]).clone(), _t(x["w2"]).clone(), _t(x["w3"]).clone()] for x in weights["dyn"]]
    tok = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
    T = tok.numel()

    j = torch.arange(dh // 2, dtype=torch.float64)
    inv = theta ** (-(2.0 * j) / dh)

    def rot(x, p):  # x [n, heads, dh]
        ang = p.to(torch.float64)[:, None] * inv[None, :]
        c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        x1, x2 = x[..., : dh // 2], x[..., dh // 2:]
        return torch.cat([x1 * c - x2 * s, x1 * s + x2 * c], -1)

    def nrm(x, g):
        return g * x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps)

    def mlp(u, w1, w2, w3):
        return (torch.nn.functional.silu(u @ w1.T) * (u @ w2.T)) @ w3.T

    Ks = [torch.zeros(T, Hk, dh, dtype=torch.float64) for _ in range(L)]
    Vs = [torch.zeros(T, Hk, dh, dtype=torch.float64) for _ in range(L)]
    losses = torch.zeros(T - 1, dtype=torch.float64)
    for a in range(0, T, b):
        e = min(a + b, T)
        p = torch.arange(a, e)
        params = [w for blk in fast for w in blk]
        for w in params:
            w.requires_grad_(True)
        x = E[tok[a:e]]
        for l in range(L):
            lw = lay[l]
            u = nrm(x, lw["attn_norm"])
            q = rot((u @ lw["wq"].T).view(-1, H, dh), p)
            kk = rot((u @ lw["wk"].T).view(-1, Hk, dh), p)
            vv = (u @ lw["wv"].T).view(-1, Hk, dh)
            lo = max(0, a - k_win + 1)
            Kc = torch.cat([Ks[l][lo:a], kk], 0)
            Vc = torch.cat([Vs[l][lo:a], vv], 0)
            kp = torch.arange(lo, e)
            vis = (kp[None, :] <= p[:, None]) & (kp[None, :] > p[:, None] - k_win)
            outs = []
            for hh in range(H):
                g = hh // (H // Hk)
                sc = (q[:, hh] @ Kc[:, g].T) / math.sqrt(dh)
                sc = sc.masked_fill(~vis, float("-inf"))
                outs.append(torch.softmax(sc, -1) @ Vc[:, g])
            x = x + torch.cat(outs, -1) @ lw["wo"].T
            x = x + mlp(nrm(x, lw["mlp_norm"]), lw["w1"], lw["w2"], lw["w3"])
            if l >= s0:
                w1, w2, w3 = fast[l - s0]
                x = x + mlp(nrm(x, dnorm[l - s0]), w1, w2, w3)
            Ks[l][a:e] = kk.detach()
            Vs[l][a:e] = vv.detach()
        z = nrm(x, gf) @ LM.T
        nt = min(e, T - 1) - a
        if nt <= 0:
            continue
        li = torch.nn.functional.cross_entropy(z[:nt], tok[a + 1: a + 1 + nt], reduction="none")
        losses[a: a + nt] = li.detach()
        lm = li.mean() if reduction == "mean" else li.sum()
        grads = torch.autograd.grad(lm, params)
        with torch.no_grad():
            new = [w - alpha * g for w, g in zip(params, grads)]
        fast = [new[3 * i: 3 * i + 3] for i in range(nd)]
    dyn = [dict(w1=f[0].detach().numpy(), w2=f[1].detach().numpy(), w3=f[2].detach().numpy())
           for f in fast]
    return dict(loss=losses.numpy(), dyn=dyn)


def online_sgd(cfg: dict, weights, tokens, alpha=None):
    """Per-token online SGD: one gradient step per target token."""
    return ttt_loop_autograd(cfg, weights, tokens, b=1, alpha=alpha)
