"""TTT-E2E inner loop: plain CPU oracle (test infrastructure only).

Sources (web pages on the method):
  [P1] "TTT-E2E：端到端测试时训练的长上下文语言建模" (metaphor-xennon encyclopedia
       article): sections "持续学习框架" (the prequential objective and the SGD
       step), "内层循环：测试时训练" (chunked inner loop), "架构设计" and
       "完整PyTorch实现" (SWA transformer, RoPE with base 10000 and half-split
       rotation, last quarter of blocks updated, tied lm_head), "关键设计参数"
       (window k >= chunk b).
  [P2] "NVIDIA开源TTT-E2E：128K上下文快2.7倍" (longzhangge digest): sections
       "另辟蹊径" (loss is a sum of next-token CE terms; only MLPs updated;
       embeddings, norms and attention frozen; mini-batches + SWA) and
       "学会如何持续学习" (k = 8K, b = 1K, last 1/4 of blocks, a static MLP
       added beside the dynamic one in updated blocks).

Readings where the pages are silent or inconsistent (each also listed in the
design notes):
  * causal window: key t is visible to query i iff i - k < t <= i;
  * K/V of a position are computed once, under the fast weights of its own
    mini-batch, and are constants afterwards (a key/value store spans
    mini-batches);
  * position i always predicts token i+1, across mini-batch boundaries;
    mini-batches tile [0, T): P_m = [m b, min((m+1) b, T));
  * per mini-batch loss is the MEAN over its targets (SUM as an option);
  * updated blocks run attention -> static SwiGLU MLP -> dynamic SwiGLU MLP,
    each a pre-RMSNorm residual sublayer; no gate;
  * RMSNorm (eps 1e-5, no bias), SwiGLU h + W3(silu(W1 u) * (W2 u)), no
    biases, 1/sqrt(dh) attention scale, RoPE at absolute positions with
    angles computed in float64, GQA by contiguous head groups.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np


# ----------------------------------------------------------------------------
# Configuration
# ----------------------------------------------------------------------------
@dataclass
class Cfg:
    L: int
    d: int
    H: int
    Hk: int
    dh: int
    F: int
    Fd: int
    V: int
    window: int
    b: int
    nd: int
    alpha: float
    eps: float
    theta: float
    reduction: str

    @property
    def s(self) -> int:
        """First updated block: the last quarter of the blocks are updated
        ([P1] 架构设计: start layer = 3 L // 4)."""
        return self.L - self.nd

    @staticmethod
    def from_dict(c: dict) -> "Cfg":
        L = c["n_layers"]
        nd = c.get("n_dynamic", 0) or (L - (3 * L) // 4)
        return Cfg(L=L, d=c["d_model"], H=c["n_heads"], Hk=c["n_kv_heads"], dh=c["head_dim"],
                   F=c["ffn_hidden"], Fd=c["dyn_ffn_hidden"], V=c["vocab"], window=c["window"],
                   b=c["minibatch"], nd=nd, alpha=float(c["alpha"]), eps=float(c["rms_eps"]),
                   theta=float(c["rope_theta"]), reduction=c.get("reduction", "mean"))


# ----------------------------------------------------------------------------
# Step functions (forward and hand-derived backward)
# ----------------------------------------------------------------------------
def rmsnorm(x, g, eps):
    """y = g * x / sqrt(mean(x^2) + eps); returns (y, r) with r the inverse rms."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return (x * r) * g, r


def rmsnorm_bwd(dy, x, g, r):
    """dx for y = g * x * r(x):  dx = r (g dy) - x r^3 mean((g dy) x)."""
    gd = dy * g
    return r * gd - x * (r ** 3) * np.mean(gd * x, axis=-1, keepdims=True)


def silu(a):
    return a / (1.0 + np.exp(-a))


def swiglu(u, w1, w2, w3):
    """W3 (silu(W1 u) * (W2 u)); returns (y, cache)."""
    a = u @ w1.T
    c = u @ w2.T
    m = silu(a) * c
    return m @ w3.T, (u, a, c, m)


def swiglu_bwd(dy, cache, w1, w2, w3, want_w=True):
    """Backward of swiglu: returns (du, dW1, dW2, dW3)."""
    u, a, c, m = cache
    dm = dy @ w3
    sg = 1.0 / (1.0 + np.exp(-a))
    da = dm * c * sg * (1.0 + a * (1.0 - sg))
    dc = dm * (a * sg)
    du = da @ w1 + dc @ w2
    if not want_w:
        return du, None, None, None
    return du, da.T @ u, dc.T @ u, dy.T @ m


def rope_angles(pos, dh, theta):
    """pos * theta^(-2j/dh), j < dh/2, in float64 ([P1] RoPE: inv_freq =
    1 / base^(arange(0, dim, 2) / dim))."""
    j = np.arange(dh // 2, dtype=np.float64)
    inv = 1.0 / (theta ** (2.0 * j / dh))
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, pos, theta, inverse=False):
    """Half-split rotation of each head vector: (x1, x2) -> (x1 c - x2 s, x1 s + x2 c).
    x: [n, heads, dh]; inverse=True rotates by the negative angle (its
    transpose, used by the backward)."""
    dh = x.shape[-1]
    ang = rope_angles(pos, dh, theta)
    c = np.cos(ang).astype(x.dtype)[:, None, :]
    s = np.sin(ang).astype(x.dtype)[:, None, :]
    if inverse:
        s = -s
    x1, x2 = x[..., : dh // 2], x[..., dh // 2:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def swa_attention(q, qpos, K, V, kpos, window):
    """Causal sliding-window attention.

    q [n, H, dh] at positions qpos; K, V [m, Hk, dh] at positions kpos.
    Key t is visible to query i iff i - window < t <= i. Query head j reads
    KV head j // (H / Hk). Returns (o [n, H, dh], P [H, n, m])."""
    n, H, dh = q.shape
    Hk = K.shape[1]
    g = H // Hk
    dq = np.asarray(qpos)[:, None]
    dk = np.asarray(kpos)[None, :]
    mask = (dk <= dq) & (dk > dq - window)
    scale = 1.0 / math.sqrt(dh)
    o = np.zeros_like(q)
    P = np.zeros((H, n, K.shape[0]), dtype=q.dtype)
    for h in range(H):
        kh = h // g
        s = (q[:, h, :] @ K[:, kh, :].T) * scale
        s = np.where(mask, s, -np.inf)
        mx = np.max(s, axis=1, keepdims=True)
        p = np.exp(s - mx)
        p = p / np.sum(p, axis=1, keepdims=True)
        P[h] = p
        o[:, h, :] = p @ V[:, kh, :]
    return o, P


def swa_attention_bwd(do, q, K, V, P, grad_keys):
    """Backward of swa_attention given its probabilities P.

    Returns dq [n, H, dh] and (dK, dV) [m, Hk, dh] restricted to the key rows
    selected by the boolean mask grad_keys (other rows are constants: zeros)."""
    n, H, dh = q.shape
    Hk = K.shape[1]
    g = H // Hk
    scale = 1.0 / math.sqrt(dh)
    dq = np.zeros_like(q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for h in range(H):
        kh = h // g
        p = P[h]
        dp = do[:, h, :] @ V[:, kh, :].T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dq[:, h, :] = (ds @ K[:, kh, :]) * scale
        dK[:, kh, :] += (ds.T @ q[:, h, :]) * scale
        dV[:, kh, :] += p.T @ do[:, h, :]
    dK[~grad_keys] = 0
    dV[~grad_keys] = 0
    return dq, dK, dV


def cross_entropy(z, labels):
    """Per-row natural-log CE: loss_i = logsumexp(z_i) - z_i[label_i]; also
    returns softmax(z)."""
    mx = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - mx)
    se = np.sum(e, axis=1, keepdims=True)
    lse = (mx + np.log(se))[:, 0]
    loss = lse - z[np.arange(z.shape[0]), labels]
    return loss, e / se


# ----------------------------------------------------------------------------
# Model state
# ----------------------------------------------------------------------------
class KVStore:
    """Keys (post-RoPE) and values of every processed position, per layer."""

    def __init__(self, cfg: Cfg, cap: int, dtype):
        self.K = [np.zeros((cap, cfg.Hk, cfg.dh), dtype=dtype) for _ in range(cfg.L)]
        self.V = [np.zeros((cap, cfg.Hk, cfg.dh), dtype=dtype) for _ in range(cfg.L)]
        self.n = 0


def _cast_weights(w, dtype):
    def cv(a):
        return np.asarray(a, dtype=dtype)
    out = {"embed": cv(w["embed"]), "final_norm": cv(w["final_norm"])}
    out["lm_head"] = cv(w["lm_head"])
    out["layers"] = [{k: cv(v) for k, v in lyr.items()} for lyr in w["layers"]]
    out["dyn"] = [{k: cv(v) for k, v in b.items()} for b in w["dyn"]]
    return out


def forward_positions(cfg: Cfg, w, dyn, store: KVStore, tokens, a: int, e: int, keep=True):
    """Forward of positions [a, e) (all earlier positions already in store).

    Writes K/V of [a, e) into the store. Returns (logits [e-a, V], caches)."""
    pos = np.arange(a, e)
    h = w["embed"][np.asarray(tokens[a:e])]
    lo = max(0, a - cfg.window + 1)
    kpos = np.arange(lo, e)
    caches = []
    for l in range(cfg.L):
        lw = w["layers"][l]
        c = {}
        # attention sublayer
        c["h_att"] = h
        u, r = rmsnorm(h, lw["attn_norm"], cfg.eps)
        c["u_att"], c["r_att"] = u, r
        q = (u @ lw["wq"].T).reshape(-1, cfg.H, cfg.dh)
        k = (u @ lw["wk"].T).reshape(-1, cfg.Hk, cfg.dh)
        v = (u @ lw["wv"].T).reshape(-1, cfg.Hk, cfg.dh)
        q = rope(q, pos, cfg.theta)
        k = rope(k, pos, cfg.theta)
        store.K[l][a:e] = k
        store.V[l][a:e] = v
        Kw, Vw = store.K[l][lo:e], store.V[l][lo:e]
        o, P = swa_attention(q, pos, Kw, Vw, kpos, cfg.window)
        c["q"], c["Kw"], c["Vw"], c["P"], c["o"] = q, Kw, Vw, P, o
        h = h + o.reshape(-1, cfg.H * cfg.dh) @ lw["wo"].T
        # static MLP sublayer
        c["h_mlp"] = h
        u, r = rmsnorm(h, lw["mlp_norm"], cfg.eps)
        c["r_mlp"] = r
        y, c["mlp"] = swiglu(u, lw["w1"], lw["w2"], lw["w3"])
        h = h + y
        # dynamic MLP sublayer (updated blocks only)
        if l >= cfg.s:
            dw = dyn[l - cfg.s]
            c["h_dyn"] = h
            u, r = rmsnorm(h, w["dyn"][l - cfg.s]["norm"], cfg.eps)
            c["r_dyn"] = r
            y, c["dynmlp"] = swiglu(u, dw["w1"], dw["w2"], dw["w3"])
            h = h + y
        caches.append(c if (keep and l >= cfg.s) else None)
    store.n = e
    u, r = rmsnorm(h, w["final_norm"], cfg.eps)
    z = u @ w["lm_head"].T
    return z, dict(layers=caches, h_f=h, r_f=r, pos=pos, lo=lo, a=a, e=e)


def backward_minibatch(cfg: Cfg, w, dyn, cache, dz):
    """Gradient of the mini-batch loss w.r.t. the dynamic MLP weights.

    dz [n, V] is dLoss/dlogits. Cached K/V of earlier mini-batches and all
    frozen parameters are constants. Returns a list (per updated block) of
    dicts {w1, w2, w3}."""
    a, e, lo = cache["a"], cache["e"], cache["lo"]
    grads = [None] * cfg.nd
    dh = rmsnorm_bwd(dz @ w["lm_head"], cache["h_f"], w["final_norm"], cache["r_f"])
    inbatch = np.arange(lo, e) >= a
    for l in range(cfg.L - 1, cfg.s - 1, -1):
        lw = w["layers"][l]
        c = cache["layers"][l]
        dw = dyn[l - cfg.s]
        du, g1, g2, g3 = swiglu_bwd(dh, c["dynmlp"], dw["w1"], dw["w2"], dw["w3"])
        grads[l - cfg.s] = dict(w1=g1, w2=g2, w3=g3)
        if l == cfg.s:
            break
        dh = dh + rmsnorm_bwd(du, c["h_dyn"], w["dyn"][l - cfg.s]["norm"], c["r_dyn"])
        du, _, _, _ = swiglu_bwd(dh, c["mlp"], lw["w1"], lw["w2"], lw["w3"], want_w=False)
        dh = dh + rmsnorm_bwd(du, c["h_mlp"], lw["mlp_norm"], c["r_mlp"])
        do = (dh @ lw["wo"]).reshape(-1, cfg.H, cfg.dh)
        dq, dK, dV = swa_attention_bwd(do, c["q"], c["Kw"], c["Vw"], c["P"], inbatch)
        pos = cache["pos"]
        dq = rope(dq, pos, cfg.theta, inverse=True)
        dk = rope(dK[inbatch], pos, cfg.theta, inverse=True)
        dv = dV[inbatch]
        n = e - a
        dx = (dq.reshape(n, -1) @ lw["wq"] + dk.reshape(n, -1) @ lw["wk"]
              + dv.reshape(n, -1) @ lw["wv"])
        dh = dh + rmsnorm_bwd(dx, c["h_att"], lw["attn_norm"], c["r_att"])
    return grads


# ----------------------------------------------------------------------------
# Public oracle functions
# ----------------------------------------------------------------------------
def _dyn_init(w, dtype):
    return [{k: np.array(b[k], dtype=dtype) for k in ("w1", "w2", "w3")} for b in w["dyn"]]


def minibatch_step(cfg: Cfg, w, dyn, store: KVStore, tokens, a: int, e: int, alpha: float, reduction: str,
                   loss):
    """One mini-batch P = [a, e) of the inner loop, in place: forward under
    the fast weights dyn (earlier positions' K/V from the store, this
    mini-batch's added to it), loss[i] = l_i for the positions with a target
    (i <= T-2, T = len(tokens)), then, if there is one, the SGD step
    dyn <- dyn - alpha dL/d(dyn) with L the MEAN (or SUM) of those l_i.
    Returns the logits [e-a, V]."""
    T = len(tokens)
    dtype = dyn[0]["w1"].dtype.type if cfg.nd else w["embed"].dtype.type
    z, cache = forward_positions(cfg, w, dyn, store, tokens, a, e)
    nt = min(e, T - 1) - a          # positions with a target
    if nt <= 0:
        return z
    lab = tokens[a + 1: a + 1 + nt]
    li, p = cross_entropy(z[:nt], lab)
    loss[a: a + nt] = li
    scale = (1.0 / nt) if reduction == "mean" else 1.0
    dz = np.zeros_like(z)
    dz[:nt] = p
    dz[np.arange(nt), lab] -= 1.0
    dz *= scale
    grads = backward_minibatch(cfg, w, dyn, cache, dz)
    for i in range(cfg.nd):
        for k in ("w1", "w2", "w3"):
            dyn[i][k] = dyn[i][k] - dtype(alpha) * grads[i][k]
    return z


def ttt_inner_loop(cfg_d: dict, weights, tokens, alpha=None, b=None, reduction=None,
                   dtype=np.float64, keep_state=False):
    """The mini-batch TTT inner loop ([P1] 内层循环 and 持续学习框架; [P2] 另辟蹊径).

    For each mini-batch P_m = [m b, min((m+1) b, T)):
      1. forward P_m under the current fast weights W^(m) (earlier K/V from
         the store);
      2. L_m = sum (MEAN: mean) of l_i = CE(z_i, x_{i+1}) over i in P_m, i <= T-2;
      3. G_m = dL_m / dW^(m) over the dynamic MLPs of the last quarter of blocks;
      4. W^(m+1) = W^(m) - alpha G_m   (plain SGD, no momentum/decay/clipping).
    A mini-batch without targets (only position T-1) is forward only.

    Returns dict(loss [T-1] (each l_i under its own mini-batch's weights),
    dyn (final fast weights), and, if keep_state, store/last_logits)."""
    cfg = Cfg.from_dict(cfg_d)
    alpha = cfg.alpha if alpha is None else float(alpha)
    b = cfg.b if b is None else int(b)
    reduction = cfg.reduction if reduction is None else reduction
    w = _cast_weights(weights, dtype)
    dyn = _dyn_init(w, dtype)
    tokens = np.asarray(tokens, dtype=np.int64)
    T = len(tokens)
    store = KVStore(cfg, T + 1, dtype)
    loss = np.zeros(T - 1, dtype=dtype)
    last_logits = None
    for a in range(0, T, b):
        e = min(a + b, T)
        z = minibatch_step(cfg, w, dyn, store, tokens, a, e, alpha, reduction, loss)
        if e == T:
            last_logits = z[-1].copy()
    out = dict(loss=loss, dyn=dyn)
    if keep_state:
        # trained: positions below it have been used (with their targets) for
        # an update; T - 1 has no target yet
        out.update(store=store, weights=w, cfg=cfg, last_logits=last_logits, tokens=list(tokens),
                   trained=T - 1, alpha=alpha, reduction=reduction)
    return out


def decode_step(state: dict, token: int):
    """Forward of one new position p = store.n under the current fast weights,
    continuing a loop state (keep_state=True). No update. Returns logits [V]."""
    cfg, w, store = state["cfg"], state["weights"], state["store"]
    p = store.n
    if p >= store.K[0].shape[0]:
        for l in range(cfg.L):
            store.K[l] = np.concatenate([store.K[l], np.zeros_like(store.K[l])])
            store.V[l] = np.concatenate([store.V[l], np.zeros_like(store.V[l])])
    toks = np.zeros(p + 1, dtype=np.int64)
    toks[p] = token
    if "tokens" in state:
        state["tokens"].append(int(token))
    z, _ = forward_positions(cfg, w, state["dyn"], store, toks, p, p + 1, keep=False)
    return z[0]


def decode_step_update(state: dict, token: int):
    """Decode with test-time training continuing into generation ([P2]
    "NVIDIA开源TTT-E2E：128K上下文快2.7倍", section 效果惊人: the model keeps
    learning from the tokens it reads after the context). Reading adopted:
    the positions consumed since the last update are trained in groups of b:
    when the token x_p arrives and the b positions [u, u + b) before p = u + b
    have all their targets (the last one is x_p), the inner-loop step runs on
    them (forward under the current fast weights, their keys/values stored
    again, loss, backward, SGD) before position p is decoded under the new
    weights. Continues a state of ttt_inner_loop(keep_state=True), after
    which u = T - 1.
    Returns (logits [V] for position p, the b losses of an update made
    before it or None)."""
    cfg, w, store = state["cfg"], state["weights"], state["store"]
    p = store.n
    while p + 1 > store.K[0].shape[0]:
        for l in range(cfg.L):
            store.K[l] = np.concatenate([store.K[l], np.zeros_like(store.K[l])])
            store.V[l] = np.concatenate([store.V[l], np.zeros_like(store.V[l])])
    state["tokens"].append(int(token))
    toks = np.asarray(state["tokens"], dtype=np.int64)
    u = state["trained"]
    losses = None
    if p - u >= cfg.b:
        loss = np.zeros(p, dtype=store.K[0].dtype)
        minibatch_step(cfg, w, state["dyn"], store, toks, u, u + cfg.b, state["alpha"], state["reduction"], loss)
        losses = loss[u:u + cfg.b].copy()
        state["trained"] = u + cfg.b
    z, _ = forward_positions(cfg, w, state["dyn"], store, toks, p, p + 1, keep=False)
    return z[0], losses


def plain_forward(cfg_d: dict, weights, tokens, dtype=np.float64, return_logits=False):
    """The model without test-time training ([P1] 完整PyTorch实现, outer_loop_loss
    with use_ttt=False): every position at once under W0 with a dense causal
    window mask. Returns per-token losses [T-1] (and logits)."""
    cfg = Cfg.from_dict(cfg_d)
    w = _cast_weights(weights, dtype)
    tokens = np.asarray(tokens, dtype=np.int64)
    T = len(tokens)
    pos = np.arange(T)
    h = w["embed"][tokens]
    for l in range(cfg.L):
        lw = w["layers"][l]
        u, _ = rmsnorm(h, lw["attn_norm"], cfg.eps)
        q = rope((u @ lw["wq"].T).reshape(T, cfg.H, cfg.dh), pos, cfg.theta)
        k = rope((u @ lw["wk"].T).reshape(T, cfg.Hk, cfg.dh), pos, cfg.theta)
        v = (u @ lw["wv"].T).reshape(T, cfg.Hk, cfg.dh)
        o = np.zeros_like(q)
        blk = 512
        for a in range(0, T, blk):
            e = min(T, a + blk)
            lo = max(0, a - cfg.window + 1)
            o[a:e], _ = swa_attention(q[a:e], pos[a:e], k[lo:e], v[lo:e], pos[lo:e], cfg.window)
        h = h + o.reshape(T, -1) @ lw["wo"].T
        u, _ = rmsnorm(h, lw["mlp_norm"], cfg.eps)
        h = h + swiglu(u, lw["w1"], lw["w2"], lw["w3"])[0]
        if l >= cfg.s:
            dw = w["dyn"][l - cfg.s]
            u, _ = rmsnorm(h, dw["norm"], cfg.eps)
            h = h + swiglu(u, dw["w1"], dw["w2"], dw["w3"])[0]
    u, _ = rmsnorm(h, w["final_norm"], cfg.eps)
    z = u @ w["lm_head"].T
    loss, _ = cross_entropy(z[:-1], tokens[1:])
    return (loss, z) if return_logits else loss


def minibatch_loss(cfg_d: dict, weights, dyn, tokens, a, e, reduction="mean", dtype=np.float64):
    """L_m of one mini-batch [a, e) as a function of the fast weights `dyn`,
    with every earlier position's K/V computed under W0 (used by the
    finite-difference pin; for a = 0 the store is empty)."""
    cfg = Cfg.from_dict(cfg_d)
    w = _cast_weights(weights, dtype)
    w0dyn = _dyn_init(w, dtype)
    tokens = np.asarray(tokens, dtype=np.int64)
    T = len(tokens)
    store = KVStore(cfg, T + 1, dtype)
    if a > 0:
        forward_positions(cfg, w, w0dyn, store, tokens, 0, a, keep=False)
    z, _ = forward_positions(cfg, w, dyn, store, tokens, a, e, keep=False)
    nt = min(e, T - 1) - a
    li, _ = cross_entropy(z[:nt], tokens[a + 1: a + 1 + nt])
    return li.mean() if reduction == "mean" else li.sum()


def minibatch_grad(cfg_d: dict, weights, tokens, a, e, reduction="mean", dtype=np.float64):
    """Hand-derived gradient of minibatch_loss at W0 (same store semantics)."""
    cfg = Cfg.from_dict(cfg_d)
    w = _cast_weights(weights, dtype)
    dyn = _dyn_init(w, dtype)
    tokens = np.asarray(tokens, dtype=np.int64)
    T = len(tokens)
    store = KVStore(cfg, T + 1, dtype)
    if a > 0:
        forward_positions(cfg, w, dyn, store, tokens, 0, a, keep=False)
    z, cache = forward_positions(cfg, w, dyn, store, tokens, a, e)
    nt = min(e, T - 1) - a
    lab = tokens[a + 1: a + 1 + nt]
    _, p = cross_entropy(z[:nt], lab)
    dz = np.zeros_like(z)
    dz[:nt] = p
    dz[np.arange(nt), lab] -= 1.0
    if reduction == "mean":
        dz /= nt
    return backward_minibatch(cfg, w, dyn, cache, dz)
