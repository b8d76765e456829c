"""E2-TTT hybrid token-mixer block: sliding-window attention beside the TTT
path, fused by a data-dependent gate (test infrastructure only).

Source: [P3] "Rethinking Expressivity and Efficiency in Test-Time Training",
section 方法细节, 混合模型架构设计 and Figure 2: the input is projected once to
shared queries, keys and values that feed two parallel branches -- the
E2-TTT path (SiLU and L2 normalisation of q and k, input-dependent scalars)
for non-local dependencies and sliding-window attention (SWA) for local
ones -- and the two outputs are interpolated element-wise by a gate that
depends on the data; the macro design follows Llama.

Readings where the pages are silent:
  * the gate is g = sigmoid(x Wg^T + bg), one value per output feature
    (H D), and out = g * o_SWA + (1 - g) * o_TTT;
  * the SWA branch takes the projections before the TTT path's SiLU and L2
    normalisation, stored in bf16 as the kernels store them, with RoPE
    (Llama: half-split rotation, base rope_theta) on q and k, scale
    1/sqrt(D), causal window w (key t visible to query i iff i - w < t <=
    i), one key head per query head;
  * the output projection after the mix is a plain product and is left to
    the caller.
Everything is float64.
"""
from __future__ import annotations

import numpy as np

from oracle.e2ttt import _bf16, e2_mixer
from oracle.e2ttt_gelu import e2_gelu_mixer
from oracle.e2ttt_mlp import e2_mlp_mixer
from oracle.ttt_e2e import rope, swa_attention


def swa_branch(x, wqkv, H, D, rope_theta, window, block=512):
    """SWA over the shared projections; evaluated one block of queries at a
    time against the keys that block can see (each query's own window)."""
    x = np.asarray(x, np.float64)
    P = x @ np.asarray(wqkv, np.float64).T
    T = x.shape[0]
    HD = H * D
    q = _bf16(P[:, :HD]).reshape(T, H, D)
    k = _bf16(P[:, HD:2 * HD]).reshape(T, H, D)
    v = _bf16(P[:, 2 * HD:3 * HD]).reshape(T, H, D)
    pos = np.arange(T)
    qr = rope(q, pos, rope_theta)
    kr = rope(k, pos, rope_theta)
    out = np.zeros((T, H, D))
    for a in range(0, T, block):
        e = min(T, a + block)
        lo = max(0, a - window + 1)
        out[a:e], _ = swa_attention(qr[a:e], pos[a:e], kr[lo:e], v[lo:e], pos[lo:e], window)
    return out


def gate(x, wgate, bgate):
    """sigmoid(x Wg^T + bg): [T, H D]."""
    z = np.asarray(x, np.float64) @ np.asarray(wgate, np.float64).T + np.asarray(bgate, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def hybrid_mixer(x, wqkv, bias, wgate, bgate, eta_base, alpha_base, tau, rope_theta, window, state, H, D, C):
    """The hybrid block: TTT path (state = (W, M) arrays for the linear fast
    weight, or (W, M) lists of per-head dicts for the SwiGLU net, keys w1,
    w2, w3, or the GELU net, keys w1, w2), SWA branch, gate. Returns
    (out [T, H, D], W, M)."""
    W, M = state
    if isinstance(W, list) and "w3" not in W[0]:
        o_ttt, W, M = e2_gelu_mixer(x, wqkv, bias, eta_base, alpha_base, tau, W, M, H, D, C)
    elif isinstance(W, list):
        o_ttt, W, M = e2_mlp_mixer(x, wqkv, bias, eta_base, alpha_base, tau, W, M, H, D, C)
    else:
        o_ttt, W, M = e2_mixer(x, wqkv, bias, eta_base, alpha_base, tau, W, M, H, D, C)
    o_swa = swa_branch(x, wqkv, H, D, rope_theta, window)
    g = gate(x, wgate, bgate).reshape(o_ttt.shape)
    return g * o_swa + (1.0 - g) * o_ttt, W, M
