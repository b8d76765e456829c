"""Pins of the hybrid token-mixer oracle (CPU only): the blocked SWA branch
against dense causal attention from the library and against the unblocked
window definition, its window-1 case, and the gate's limits."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import e2ttt_hybrid as Y
from oracle.e2ttt import _bf16
from oracle.ttt_e2e import rope, swa_attention


def _proj(T=70, H=2, D=64, dm=64, seed=12):
    g = synth.gen_e2_mixer(H, T, D, dm, seed)
    return g["x"].double().numpy(), g["wqkv"].double().numpy(), g["bias"].numpy()


def _qkv(x, wqkv, H, D, theta):
    P = x @ wqkv.T
    T = x.shape[0]
    q, k, v = (_bf16(P[:, i * H * D:(i + 1) * H * D]).reshape(T, H, D) for i in range(3))
    pos = np.arange(T)
    return rope(q, pos, theta), rope(k, pos, theta), v


def test_swa_branch_with_window_over_the_stream_is_causal_attention():
    H, D = 2, 64
    x, wqkv, _ = _proj(H=H, D=D)
    T = x.shape[0]
    o = Y.swa_branch(x, wqkv, H, D, 10000.0, window=10 * T, block=16)
    q, k, v = _qkv(x, wqkv, H, D, 10000.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a).permute(1, 0, 2) for a in (q, k, v)), is_causal=True).permute(1, 0, 2).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


@pytest.mark.parametrize("window", [1, 5, 33])
def test_swa_branch_blocked_equals_the_window_definition(window):
    H, D = 2, 64
    x, wqkv, _ = _proj(H=H, D=D)
    T = x.shape[0]
    o = Y.swa_branch(x, wqkv, H, D, 500.0, window=window, block=16)
    q, k, v = _qkv(x, wqkv, H, D, 500.0)
    pos = np.arange(T)
    ref, _ = swa_attention(q, pos, k, v, pos, window)
    assert np.max(np.abs(o - ref)) < 1e-12
    if window == 1:
        assert np.max(np.abs(o - v)) < 1e-12


def test_gate_limits_select_one_branch():
    H, D, dm, C = 2, 64, 64, 32
    x, wqkv, bias = _proj(H=H, D=D, dm=dm)
    T = x.shape[0]
    rng = np.random.default_rng(3)
    wg = rng.normal(size=(H * D, dm)) / math.sqrt(dm)
    W = rng.normal(size=(H, D, D)) * 0.02
    M = np.zeros_like(W)
    args = (x, wqkv, bias, wg)
    tail = (1e-4, 0.5, 4.0, 10000.0, 16, (W, M), H, D, C)
    o_on, _, _ = Y.hybrid_mixer(*args, np.full(H * D, 1e3), *tail)
    o_off, W2, M2 = Y.hybrid_mixer(*args, np.full(H * D, -1e3), *tail)
    swa = Y.swa_branch(x, wqkv, H, D, 10000.0, 16)
    from oracle.e2ttt import e2_mixer
    ttt, W3, M3 = e2_mixer(x, wqkv, bias, 1e-4, 0.5, 4.0, W, M, H, D, C)
    assert np.max(np.abs(o_on - swa)) < 1e-12
    assert np.max(np.abs(o_off - ttt)) < 1e-12
    assert np.array_equal(W2, W3) and np.array_equal(M2, M3)
    # gate 1/2: the mean of the branches
    o_half, _, _ = Y.hybrid_mixer(x, wqkv, bias, np.zeros_like(wg), np.zeros(H * D), *tail)
    assert np.max(np.abs(o_half - 0.5 * (swa + ttt))) < 1e-12
