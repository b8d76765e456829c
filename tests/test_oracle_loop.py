"""Pins of the oracle's TTT loop (CPU only): finite differences, the alpha = 0
and b = 1 special cases, an independent autograd implementation, the
single-step case and the loss magnitude at initialisation."""
import math

import numpy as np
import pytest

import synth
from oracle import ttt_e2e as O
from oracle import autograd_ref as A


def tiny(**kw):
    c = synth.config("tiny", **kw)
    w = synth.weights_to_numpy(synth.gen_weights(c))
    return c, w


def _fd_check(c, w, a, e, reduction, ncoord=70, h=1e-6, seed=0):
    tok = synth.gen_tokens(c).numpy()
    g = O.minibatch_grad(c, w, tok, a, e, reduction)
    r = np.random.default_rng(seed)
    worst = 0.0
    for i, blk in enumerate(w["dyn"]):
        for name in ("w1", "w2", "w3"):
            W = blk[name]
            G = g[i][name]
            scale = np.max(np.abs(G))
            for _ in range(ncoord):
                idx = tuple(r.integers(0, s) for s in W.shape)
                dyn_p = [{k: np.array(b[k]) for k in ("w1", "w2", "w3")} for b in w["dyn"]]
                dyn_m = [{k: np.array(b[k]) for k in ("w1", "w2", "w3")} for b in w["dyn"]]
                dyn_p[i][name][idx] += h
                dyn_m[i][name][idx] -= h
                fd = (O.minibatch_loss(c, w, dyn_p, tok, a, e, reduction)
                      - O.minibatch_loss(c, w, dyn_m, tok, a, e, reduction)) / (2 * h)
                worst = max(worst, abs(fd - G[idx]) / scale)
    return worst


@pytest.mark.parametrize("a,e,red", [(0, 16, "mean"), (32, 48, "mean"), (16, 32, "sum")])
def test_gradient_matches_central_finite_differences(a, e, red):
    c, w = tiny()
    # several coordinates of each matrix; error relative to the matrix's max |G|
    assert _fd_check(c, w, a, e, red) < 1e-6


def test_gradient_fd_with_gqa_and_two_updated_blocks():
    c, w = tiny(n_layers=4, n_heads=4, n_kv_heads=2, n_dynamic=2, window=8)
    assert _fd_check(c, w, 8, 16, "mean", ncoord=25) < 1e-6


def test_alpha_zero_equals_plain_forward():
    c, w = tiny()
    tok = synth.gen_tokens(c).numpy()
    out = O.ttt_inner_loop(c, w, tok, alpha=0.0)
    ref = O.plain_forward(c, w, tok)
    np.testing.assert_allclose(out["loss"], ref, rtol=1e-12, atol=1e-12)
    for blk, orig in zip(out["dyn"], w["dyn"]):
        for k in ("w1", "w2", "w3"):
            assert np.array_equal(blk[k], orig[k])


def test_alpha_zero_equals_plain_forward_ragged_and_gqa():
    c, w = tiny(n_layers=4, n_kv_heads=2, n_dynamic=1, window=12, minibatch=7)
    w = synth.weights_to_numpy(synth.gen_weights(c))
    tok = synth.gen_tokens(c, n=61).numpy()
    out = O.ttt_inner_loop(c, w, tok, alpha=0.0)
    np.testing.assert_allclose(out["loss"], O.plain_forward(c, w, tok), rtol=1e-12, atol=1e-12)


def test_b1_equals_per_token_online_sgd():
    c, w = tiny()
    tok = synth.gen_tokens(c, n=40).numpy()
    mine = O.ttt_inner_loop(c, w, tok, b=1)
    ref = A.online_sgd(c, w, tok)
    np.testing.assert_allclose(mine["loss"], ref["loss"], rtol=1e-11, atol=1e-12)
    for x, y in zip(mine["dyn"], ref["dyn"]):
        for k in ("w1", "w2", "w3"):
            np.testing.assert_allclose(x[k], y[k], rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("b,T,red", [(16, 80, "mean"), (5, 37, "mean"), (7, 30, "sum")])
def test_loop_matches_independent_autograd_loop(b, T, red):
    c, w = tiny()
    tok = synth.gen_tokens(c, n=T).numpy()
    mine = O.ttt_inner_loop(c, w, tok, b=b, reduction=red)
    ref = A.ttt_loop_autograd(c, w, tok, b=b, reduction=red)
    np.testing.assert_allclose(mine["loss"], ref["loss"], rtol=1e-11, atol=1e-12)
    for x, y in zip(mine["dyn"], ref["dyn"]):
        for k in ("w1", "w2", "w3"):
            dw = np.max(np.abs(y[k] - 0))
            np.testing.assert_allclose(x[k], y[k], rtol=0, atol=1e-11 * max(dw, 1))


def test_single_minibatch_is_one_step_with_plain_forward_gradient():
    """T = b + 1: one update, whose gradient is that of the plain forward's
    mean loss over positions 0..b-1 (finite differences of plain_forward)."""
    c, w = tiny()
    b = c["minibatch"]
    tok = synth.gen_tokens(c, n=b + 1).numpy()
    out = O.ttt_inner_loop(c, w, tok)
    alpha = c["alpha"]
    r = np.random.default_rng(3)
    h = 1e-6
    for name in ("w1", "w2", "w3"):
        W0 = w["dyn"][0][name]
        step = (W0 - out["dyn"][0][name]) / alpha
        for _ in range(30):
            idx = tuple(r.integers(0, s) for s in W0.shape)
            wp = synth.weights_to_numpy(synth.gen_weights(c))
            wm = synth.weights_to_numpy(synth.gen_weights(c))
            wp["dyn"][0][name][idx] += h
            wm["dyn"][0][name][idx] -= h
            fd = (O.plain_forward(c, wp, tok)[:b].mean() - O.plain_forward(c, wm, tok)[:b].mean()) / (2 * h)
            assert abs(fd - step[idx]) < 1e-7 * max(1.0, np.max(np.abs(step)))


def test_decode_alpha_zero_equals_plain_forward_logits():
    c, w = tiny()
    tok = synth.gen_tokens(c, n=45).numpy()
    st = O.ttt_inner_loop(c, w, tok[:40], alpha=0.0, keep_state=True)
    _, z = O.plain_forward(c, w, tok, return_logits=True)
    np.testing.assert_allclose(st["last_logits"], z[39], rtol=1e-12, atol=1e-12)
    for p in range(40, 45):
        lg = O.decode_step(st, int(tok[p]))
        np.testing.assert_allclose(lg, z[p], rtol=1e-12, atol=1e-12)


def test_loss_at_init_is_near_log_vocab():
    c, w = tiny()
    tok = synth.gen_tokens(c).numpy()
    out = O.ttt_inner_loop(c, w, tok)
    assert abs(out["loss"].mean() - math.log(c["vocab"])) < 0.05
    # the updates move the fast weights
    assert np.max(np.abs(out["dyn"][0]["w1"] - w["dyn"][0]["w1"])) > 0


def test_sgd_step_decreases_the_minibatch_loss():
    c, w = tiny()
    tok = synth.gen_tokens(c).numpy()
    b = c["minibatch"]
    g = O.minibatch_grad(c, w, tok, 0, b)
    dyn0 = [{k: np.array(x[k]) for k in ("w1", "w2", "w3")} for x in w["dyn"]]
    dyn1 = [{k: dyn0[i][k] - 1e-2 * g[i][k] for k in ("w1", "w2", "w3")} for i in range(len(dyn0))]
    assert O.minibatch_loss(c, w, dyn1, tok, 0, b) < O.minibatch_loss(c, w, dyn0, tok, 0, b)


# ---------------------------------------------------------------------------
# Sensitivity: a plausible mistake planted in the oracle (on the CPU) must make
# one of the pins above fail.
# ---------------------------------------------------------------------------
def _mut_rope_bwd_sign(orig):
    def f(x, pos, theta, inverse=False):
        return orig(x, pos, theta, inverse=False)
    return f


def _mut_rms_bwd_drop(orig):
    def f(dy, x, g, r):
        return r * dy * g
    return f


def _mut_attn_no_rowsum(orig):
    # dS = P * dP without the "- rowsum(P * dP)" term
    def f(do, q, K, V, P, grad_keys):
        dq, dK, dV = orig(do, q, K, V, P, grad_keys)
        H, dh = q.shape[1], q.shape[2]
        g = H // K.shape[1]
        for h in range(H):
            p = P[h]
            dp = do[:, h, :] @ V[:, h // g, :].T
            dq[:, h, :] += (p * np.sum(p * dp, axis=1, keepdims=True)) @ K[:, h // g, :] / np.sqrt(dh)
        return dq, dK, dV
    return f


def _mut_swiglu_dc(orig):
    def f(dy, cache, w1, w2, w3, want_w=True):
        u, a, c, m = cache
        return orig(dy, (u, a, -c, m), w1, w2, w3, want_w)
    return f


@pytest.mark.parametrize("target,mut", [("rope", _mut_rope_bwd_sign),
                                        ("rmsnorm_bwd", _mut_rms_bwd_drop),
                                        ("swa_attention_bwd", _mut_attn_no_rowsum),
                                        ("swiglu_bwd", _mut_swiglu_dc)])
def test_planted_mistakes_are_caught(monkeypatch, target, mut):
    c, w = tiny(n_layers=3, n_dynamic=2, window=8)
    tok = synth.gen_tokens(c, n=24).numpy()
    orig = getattr(O, target)
    if target == "rope":
        # only the backward's inverse rotation is broken
        bad = mut(orig)
        monkeypatch.setattr(O, "backward_minibatch", _wrap_bwd_rope(O.backward_minibatch, bad, orig))
    else:
        monkeypatch.setattr(O, target, mut(orig))
    mine = O.ttt_inner_loop(c, w, tok, b=8)
    ref = A.ttt_loop_autograd(c, w, tok, b=8)
    err = max(np.max(np.abs(x[k] - y[k])) for x, y in zip(mine["dyn"], ref["dyn"]) for k in ("w1", "w2", "w3"))
    assert err > 1e-9


def _wrap_bwd_rope(bwd, bad, orig):
    def f(*a, **k):
        O.rope = bad
        try:
            return bwd(*a, **k)
        finally:
            O.rope = orig
    return f


# ------------------------------------------------------- decode with updates
def _tiny(**over):
    c = synth.config("tiny", **over)
    w = synth.weights_to_numpy(synth.gen_weights(c))
    return c, w


@pytest.mark.parametrize("over", [dict(), dict(n_layers=3, n_kv_heads=2, n_dynamic=2, window=24)])
def test_decode_with_updates_equals_prefill_of_the_longer_stream(over):
    """After a prefill of T = 2b + 1 tokens, decoding with updates through
    position N - 1 = 4b trains the two mini-batches [2b, 3b) and [3b, 4b) at
    positions 3b and 4b: the fast weights, the losses of those positions and
    the last logits equal a prefill of the N = 4b + 1 tokens."""
    c, w = _tiny(**over)
    b = c["minibatch"]
    T, N = 2 * b + 1, 4 * b + 1
    tok = synth.gen_tokens(c, n=N).numpy()
    st = O.ttt_inner_loop(c, w, tok[:T], keep_state=True)
    losses = {}
    for p in range(T, N):
        z, l = O.decode_step_update(st, int(tok[p]))
        if l is not None:
            losses[p] = l
    assert sorted(losses) == [3 * b, 4 * b]
    ref = O.ttt_inner_loop(c, w, tok, keep_state=True)
    for i in range(len(w["dyn"])):
        for k in ("w1", "w2", "w3"):
            np.testing.assert_allclose(st["dyn"][i][k], ref["dyn"][i][k], rtol=0, atol=1e-13)
    np.testing.assert_allclose(losses[3 * b], ref["loss"][2 * b:3 * b], rtol=1e-12)
    np.testing.assert_allclose(losses[4 * b], ref["loss"][3 * b:4 * b], rtol=1e-12)
    np.testing.assert_allclose(z, ref["last_logits"], rtol=1e-11, atol=1e-13)


def test_decode_with_updates_at_alpha_zero_is_the_plain_model():
    """alpha = 0 and a prefill length that does not end a mini-batch: the
    updates change nothing, so every decode logit and every loss of the
    trained positions equal the plain forward of the whole stream."""
    c, w = _tiny(alpha=0.0)
    b = c["minibatch"]
    T, N = b + 7, 3 * b + 12
    tok = synth.gen_tokens(c, n=N).numpy()
    st = O.ttt_inner_loop(c, w, tok[:T], keep_state=True)
    _, zref = O.plain_forward(c, w, tok, return_logits=True)
    lref = O.plain_forward(c, w, tok)
    n_upd = 0
    for p in range(T, N):
        z, l = O.decode_step_update(st, int(tok[p]))
        np.testing.assert_allclose(z, zref[p], rtol=1e-12, atol=1e-13)
        if l is not None:
            np.testing.assert_allclose(l, lref[p - b:p], rtol=1e-12)
            n_upd += 1
    # training groups start at T - 1 (the first position without a target)
    assert n_upd == (N - 1 - (T - 1)) // b
