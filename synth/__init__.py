"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds the five workload descriptions and a counter-based random
generator. It contains none of the method's arithmetic: it only draws token
streams, weight matrices and the per-token scalars of the E2-TTT chunk scan.
Both the HIP path and the CPU oracle receive exactly these values.

Generator (one published construction, restated here):
  * a 32-bit integer mixer (the "lowbias32" xor-shift-multiply finaliser) is
    applied to (counter XOR stream key); the stream key is itself a mix of
    (seed, tensor id). Multiplication mod 2**32 is split into 16-bit halves
    so that int64 arithmetic never overflows;
  * a uniform in (0, 1) is (h + 0.5) / 2**32 in float64;
  * a normal is Box-Muller's cosine branch in float64 from two uniforms.
Everything is integer arithmetic except Box-Muller's log/cos/sqrt, so CPU and
GPU evaluations agree bit for bit on the integers and uniforms and to within
an ulp of float64 on normals (a bf16 rounding flip needs a float64 value
within ~1e-16 relative of a bf16 tie point).
Token ids follow a truncated Zipf(1.1) law on ranks 1..V (id = rank - 1),
drawn by inverse CDF with a float64 table built on the host; this stands in
for the natural-text corpora on which the method is evaluated, which are not
available here.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

M32 = 0xFFFFFFFF

# ----------------------------------------------------------------------------
# Workloads. Field names follow the config record of the method's reference
# sketch (vocab, d_model, heads, layers, window k, chunk b, lr alpha).
# ----------------------------------------------------------------------------
CONFIGS: Dict[str, dict] = {
    # Tiny fp32 correctness workload.
    "tiny": dict(n_layers=2, d_model=64, n_heads=4, n_kv_heads=4, head_dim=16,
                 ffn_hidden=256, dyn_ffn_hidden=256, vocab=256, window=16,
                 minibatch=16, n_dynamic=1, alpha=0.1, rms_eps=1e-5,
                 rope_theta=10000.0, dtype="f32", reduction="mean",
                 seq=256, tokens="uniform", seed=1),
    # 125M-shape, bf16 compute + fp32 fast-weight master.
    "125m": dict(n_layers=12, d_model=768, n_heads=12, n_kv_heads=12, head_dim=64,
                 ffn_hidden=2048, dyn_ffn_hidden=2048, vocab=32000, window=1024,
                 minibatch=1024, n_dynamic=3, alpha=0.01, rms_eps=1e-5,
                 rope_theta=10000.0, dtype="bf16", reduction="mean",
                 seq=8192, tokens="zipf", seed=2),
    # 1B-shape.
    "1b": dict(n_layers=24, d_model=2048, n_heads=16, n_kv_heads=16, head_dim=128,
               ffn_hidden=5632, dyn_ffn_hidden=5632, vocab=32000, window=8192,
               minibatch=1024, n_dynamic=6, alpha=0.01, rms_eps=1e-5,
               rope_theta=10000.0, dtype="bf16", reduction="mean",
               seq=32768, tokens="zipf", seed=3),
    # 3B-shape headline: 24 query / 8 KV heads, 128K context.
    "3b": dict(n_layers=28, d_model=3072, n_heads=24, n_kv_heads=8, head_dim=128,
               ffn_hidden=8192, dyn_ffn_hidden=8192, vocab=128256, window=8192,
               minibatch=1024, n_dynamic=7, alpha=0.005, rms_eps=1e-5,
               rope_theta=10000.0, dtype="bf16", reduction="mean",
               seq=131072, tokens="zipf", seed=4),
}

# E2-TTT chunk-end workload.
E2_CONFIG = dict(heads=16, seq=32768, dim=128, chunk=2048, seed=5)

# E2-TTT token-mixer workload: the same heads and length, layer width
# 16 x 128, the pages' training chunk of 512, and scalar rates that keep the
# chunked dynamics bounded on synthetic inputs (SiLU + L2-normalised keys are
# strongly correlated, so the per-chunk gradients add up coherently).
E2_MIXER_CONFIG = dict(heads=16, seq=32768, dim=128, d_model=2048, chunk=512, eta_base=1e-4, alpha_base=0.5,
                       tau=4.0, seed=6)
# the same mixer with a SwiGLU fast-weight net of `hidden` units per head
E2_MLP_CONFIG = dict(heads=16, seq=32768, dim=128, hidden=256, d_model=2048, chunk=512, eta_base=3e-4,
                     alpha_base=0.5, tau=4.0, seed=7)
# the same token mixer with the GELU fast-weight net (same shapes)
E2_GELU_CONFIG = dict(E2_MLP_CONFIG, seed=10)
# the hybrid block (SWA beside the SwiGLU TTT path, gated)
E2_HYBRID_CONFIG = dict(E2_MLP_CONFIG, window=1024, rope_theta=10000.0, seed=8)


def config(name: str, **overrides) -> dict:
    c = dict(CONFIGS[name])
    c.update(overrides)
    return c


# ----------------------------------------------------------------------------
# Counter-based generator
# ----------------------------------------------------------------------------
def _mul32(x: torch.Tensor, m: int) -> torch.Tensor:
    lo, hi = m & 0xFFFF, (m >> 16) & 0xFFFF
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _key(seed: int, stream: int) -> int:
    t = torch.tensor([(seed * 0x9E3779B1 + stream * 0x85EBCA77 + 0x27D4EB2F) & M32],
                     dtype=torch.int64)
    return int(_mix32(_mix32(t))[0])


def _hash(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    k = _key(seed, stream)
    return _mix32(_mix32((idx & M32) ^ k) ^ ((k * 7 + 0x165667B1) & M32))


def uniform(seed: int, stream: int, n: int, device="cpu", offset: int = 0) -> torch.Tensor:
    """float64 uniforms in (0, 1), element i from counter offset + i."""
    idx = torch.arange(offset, offset + n, dtype=torch.int64, device=device)
    return (_hash(seed, stream, idx).to(torch.float64) + 0.5) * (1.0 / 4294967296.0)


def normal(seed: int, stream: int, n: int, device="cpu", offset: int = 0) -> torch.Tensor:
    """float64 standard normals (Box-Muller, cosine branch)."""
    idx = torch.arange(offset, offset + n, dtype=torch.int64, device=device)
    u1 = (_hash(seed, stream, 2 * idx).to(torch.float64) + 0.5) * (1.0 / 4294967296.0)
    u2 = (_hash(seed, stream, 2 * idx + 1).to(torch.float64) + 0.5) * (1.0 / 4294967296.0)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def _normal_tensor(seed, stream, shape, std, dtype, device, chunk=1 << 24):
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=dtype, device=device)
    for a in range(0, n, chunk):
        e = min(n, a + chunk)
        out[a:e] = (normal(seed, stream, e - a, device, offset=a) * std).to(dtype)
    return out.view(*shape)


# ----------------------------------------------------------------------------
# Token streams
# ----------------------------------------------------------------------------
def zipf_cdf(vocab: int, s: float = 1.1) -> torch.Tensor:
    r = np.arange(1, vocab + 1, dtype=np.float64)
    p = r ** (-s)
    c = np.cumsum(p)
    c = c / c[-1]
    c[-1] = 1.0
    return torch.from_numpy(c)


def gen_tokens(cfg: dict, n: Optional[int] = None, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """int32 token ids [n] (default n = cfg['seq'])."""
    n = cfg["seq"] if n is None else n
    seed = cfg["seed"] if seed is None else seed
    u = uniform(seed, 1, n, device)
    V = cfg["vocab"]
    if cfg["tokens"] == "uniform":
        ids = torch.clamp((u * V).floor().to(torch.int64), max=V - 1)
    else:
        cdf = zipf_cdf(V).to(device)
        ids = torch.clamp(torch.searchsorted(cdf, u, right=True), max=V - 1)
    return ids.to(torch.int32)


# ----------------------------------------------------------------------------
# Model weights: nn.Linear layout [out, in]; matrices N(0, 0.02^2), gains 1.
# ----------------------------------------------------------------------------
def torch_dtype(cfg: dict):
    return torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16


def gen_weights(cfg: dict, device="cpu", seed: Optional[int] = None, std: float = 0.02) -> dict:
    """Weights as a nested dict of tensors in the workload's storage dtype.

    Draw order (stream ids): embed, then per layer wq, wk, wv, wo, w1, w2, w3,
    then per dynamic block w1, w2, w3. lm_head is tied to embed.
    """
    seed = cfg["seed"] if seed is None else seed
    dt = torch_dtype(cfg)
    L, d, H, Hk, dh = cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    F, Fd, V = cfg["ffn_hidden"], cfg["dyn_ffn_hidden"], cfg["vocab"]
    nd = cfg["n_dynamic"] or (L - (3 * L) // 4)
    sid = [100]

    def mat(*shape):
        sid[0] += 1
        return _normal_tensor(seed, sid[0], shape, std, dt, device)

    def ones(n):
        return torch.ones(n, dtype=dt, device=device)

    w = {"embed": mat(V, d)}
    w["lm_head"] = w["embed"]
    w["final_norm"] = ones(d)
    layers = []
    for _ in range(L):
        layers.append(dict(attn_norm=ones(d), wq=mat(H * dh, d), wk=mat(Hk * dh, d),
                           wv=mat(Hk * dh, d), wo=mat(d, H * dh), mlp_norm=ones(d),
                           w1=mat(F, d), w2=mat(F, d), w3=mat(d, F)))
    w["layers"] = layers
    dyn = []
    for _ in range(nd):
        dyn.append(dict(norm=ones(d), w1=mat(Fd, d), w2=mat(Fd, d), w3=mat(d, Fd)))
    w["dyn"] = dyn
    return w


def weights_to_numpy(w: dict, np_dtype=np.float64) -> dict:
    """Host copy of a weight dict as numpy arrays (exact: bf16 -> f32/f64 is exact)."""
    def cv(t):
        return t.detach().to("cpu", torch.float32).numpy().astype(np_dtype)
    out = {"embed": cv(w["embed"]), "final_norm": cv(w["final_norm"])}
    out["lm_head"] = out["embed"] if w["lm_head"] is w["embed"] else cv(w["lm_head"])
    out["layers"] = [{k: cv(v) for k, v in lyr.items()} for lyr in w["layers"]]
    out["dyn"] = [{k: cv(v) for k, v in b.items()} for b in w["dyn"]]
    return out


# ----------------------------------------------------------------------------
# E2-TTT chunk-scan inputs
# ----------------------------------------------------------------------------
def gen_e2(heads: int, seq: int, dim: int, seed: int, device="cpu") -> dict:
    """k, v ~ N(0,1)/sqrt(dim) rounded to bf16, [H, T, D]; eta ~ U(0, 0.1),
    beta, gamma ~ U(0.9, 1) in fp32, [H, T]; W ~ N(0, 0.02^2) fp32 [H, D, D];
    M = 0."""
    n = heads * seq * dim
    s = 1.0 / math.sqrt(dim)
    k = (normal(seed, 1, n, device) * s).to(torch.bfloat16).view(heads, seq, dim)
    v = (normal(seed, 2, n, device) * s).to(torch.bfloat16).view(heads, seq, dim)
    eta = (uniform(seed, 3, heads * seq, device) * 0.1).to(torch.float32).view(heads, seq)
    beta = (0.9 + 0.1 * uniform(seed, 4, heads * seq, device)).to(torch.float32).view(heads, seq)
    gamma = (0.9 + 0.1 * uniform(seed, 5, heads * seq, device)).to(torch.float32).view(heads, seq)
    W = (normal(seed, 6, heads * dim * dim, device) * 0.02).to(torch.float32).view(heads, dim, dim)
    M = torch.zeros(heads, dim, dim, dtype=torch.float32, device=device)
    return dict(k=k, v=v, eta=eta, beta=beta, gamma=gamma, W=W, M=M)


def gen_e2_mixer(heads: int, seq: int, dim: int, d_model: int, seed: int, device="cpu") -> dict:
    """x ~ N(0, 1) [T, d_model] and wqkv [3 H D + 3 H, d_model] (rows Wq, Wk ~
    N(0, 1/d_model); Wv ~ N(0, 1/(d_model D)), so values have about unit norm
    as in the chunk-end workload; the eta, beta, alpha logit rows ~ N(0,
    1/d_model)), both rounded to bf16; bias [3 H] float = (0, 3, 0) per
    group (beta starts near 1); W ~ N(0, 0.02^2) float [H, D, D]; M = 0."""
    H, D, dm = heads, dim, d_model
    x = normal(seed, 1, seq * dm, device).to(torch.bfloat16).view(seq, dm)
    rows = 3 * H * D + 3 * H
    std = torch.full((rows, 1), 1.0 / math.sqrt(dm), dtype=torch.float64, device=device)
    std[2 * H * D:3 * H * D] /= math.sqrt(D)
    wqkv = (normal(seed, 2, rows * dm, device).view(rows, dm) * std).to(torch.bfloat16)
    bias = torch.cat([torch.zeros(H), torch.full((H,), 3.0), torch.zeros(H)]).to(torch.float32).to(device)
    W = (normal(seed, 3, H * D * D, device) * 0.02).to(torch.float32).view(H, D, D)
    M = torch.zeros(H, D, D, dtype=torch.float32, device=device)
    return dict(x=x, wqkv=wqkv, bias=bias, W=W, M=M)


def gen_e2_mlp_state(heads: int, dim: int, hidden: int, seed: int, device="cpu") -> dict:
    """Initial SwiGLU fast-weight state per head: w1, w2 ~ N(0, 1) [H, hidden,
    dim] (unit-norm keys give pre-activations of about unit size), w3 ~ N(0,
    1/hidden) [H, dim, hidden], float32; momenta m1, m2, m3 = 0."""
    H, D, Dh = heads, dim, hidden
    w1 = normal(seed, 11, H * Dh * D, device).to(torch.float32).view(H, Dh, D)
    w2 = normal(seed, 12, H * Dh * D, device).to(torch.float32).view(H, Dh, D)
    w3 = (normal(seed, 13, H * D * Dh, device) / math.sqrt(Dh)).to(torch.float32).view(H, D, Dh)
    z = lambda t: torch.zeros_like(t)
    return dict(w1=w1, w2=w2, w3=w3, m1=z(w1), m2=z(w2), m3=z(w3))


def gen_e2_gelu_state(heads: int, dim: int, hidden: int, seed: int, device="cpu") -> dict:
    """Initial GELU fast-weight state per head: w1 ~ N(0, 1) [H, hidden, dim],
    w2 ~ N(0, 1/hidden) [H, dim, hidden], float32; momenta m1, m2 = 0."""
    H, D, Dh = heads, dim, hidden
    w1 = normal(seed, 31, H * Dh * D, device).to(torch.float32).view(H, Dh, D)
    w2 = (normal(seed, 32, H * D * Dh, device) / math.sqrt(Dh)).to(torch.float32).view(H, D, Dh)
    z = lambda t: torch.zeros_like(t)
    return dict(w1=w1, w2=w2, m1=z(w1), m2=z(w2))


def gen_gate(heads: int, dim: int, d_model: int, seed: int, device="cpu") -> dict:
    """Gate projection of the hybrid block: wgate ~ N(0, 1/d_model) [H dim,
    d_model] rounded to bf16, bgate = 0 float [H dim]."""
    n = heads * dim
    wg = (normal(seed, 21, n * d_model, device).view(n, d_model) / math.sqrt(d_model)).to(torch.bfloat16)
    return dict(wgate=wg, bgate=torch.zeros(n, dtype=torch.float32, device=device))
