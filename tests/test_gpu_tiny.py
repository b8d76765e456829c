"""GPU parity of the whole inner loop on the tiny fp32 workload (and small
variants: GQA, ragged tails, SUM, b = 1), against the float64 oracle.
Tolerance: 1e-5 relative on per-token loss and on the final fast weights
(update-normalised: max |W - W_ref| / max |W_ref - W0|)."""
import numpy as np
import pytest
import torch

import synth
from oracle import ttt_e2e as O
from tests.util import dw_err, rel_loss_err, say, to_device

pytestmark = pytest.mark.gpu

TOL = 1e-5


def run_gpu(c, w_cpu, tok_cpu, max_seq=None):
    import test_long_context_amd as tla
    w = to_device(w_cpu)
    tok = tok_cpu.cuda()
    m = tla.TTT(c, w, max_seq=max_seq or len(tok_cpu))
    loss = m.prefill(tok)
    m.sync()
    fw = [tuple(x.cpu().numpy() for x in m.fast_weights(i)) for i in range(len(w_cpu["dyn"]))]
    loss = loss.cpu().numpy()
    m.close()
    return loss, fw


def check(c, T=None, alpha=None, b=None, reduction=None, tol=TOL):
    if alpha is not None:
        c = dict(c, alpha=alpha)
    if b is not None:
        c = dict(c, minibatch=b)
    if reduction is not None:
        c = dict(c, reduction=reduction)
    say(f"case: {dict((k, c[k]) for k in ('n_layers', 'n_heads', 'n_kv_heads', 'window', 'minibatch', 'alpha', 'reduction'))} T={T}")
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c, n=T)
    loss, fw = run_gpu(c, w, tok)
    wn = synth.weights_to_numpy(w)
    ref = O.ttt_inner_loop(c, wn, tok.numpy())
    le = rel_loss_err(loss, ref["loss"])
    errs = []
    for i, (g1, g2, g3) in enumerate(fw):
        for name, g in (("w1", g1), ("w2", g2), ("w3", g3)):
            errs.append(dw_err(g, ref["dyn"][i][name], wn["dyn"][i][name]))
    say(f"  loss rel err {le:.3e}  max dW err {max(errs):.3e}")
    assert le < tol
    assert max(errs) < tol
    return loss, fw, ref, wn


def test_tiny_full_sequence():
    check(synth.config("tiny"))


def test_tiny_alpha_zero_keeps_weights_and_matches_plain_forward():
    c = synth.config("tiny", alpha=0.0)
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c)
    loss, fw = run_gpu(c, w, tok)
    wn = synth.weights_to_numpy(w)
    ref = O.plain_forward(c, wn, tok.numpy())
    assert rel_loss_err(loss, ref) < TOL
    for i, (g1, g2, g3) in enumerate(fw):
        assert np.array_equal(g1, wn["dyn"][i]["w1"].astype(np.float32))
        assert np.array_equal(g2, wn["dyn"][i]["w2"].astype(np.float32))
        assert np.array_equal(g3, wn["dyn"][i]["w3"].astype(np.float32))


def test_tiny_b1_is_online_sgd():
    check(synth.config("tiny"), T=48, b=1)


def test_tiny_ragged_tail_gqa_two_dynamic_blocks():
    c = synth.config("tiny", n_layers=4, n_kv_heads=2, n_dynamic=2, window=24, minibatch=16)
    check(c, T=150)


def test_tiny_sum_reduction_and_last_minibatch_forward_only():
    # SUM scales each step by the mini-batch size; alpha / b keeps the update
    # the size of the MEAN case, so the update-normalised metric stays above
    # the fp32 rounding floor of W itself.
    c = synth.config("tiny", reduction="sum", alpha=0.1 / 16)
    check(c, T=16 * 5 + 1)


def test_tiny_dh64_window_spanning_many_tiles():
    c = synth.config("tiny", d_model=128, n_heads=2, n_kv_heads=1, head_dim=64, window=100,
                     minibatch=40, ffn_hidden=128, dyn_ffn_hidden=96)
    check(c, T=230)


# Edge cases of the loop's tiling and the block split (fp32, float64 oracle):
# the shortest stream (one target), a stream shorter than one mini-batch, a
# window equal to the mini-batch, every block dynamic (nothing hoisted but
# block 0's attention and static MLP), and a single-layer model.
EDGE = [
    ("T=2", dict(), 2),
    ("T<b", dict(minibatch=16), 11),
    ("window=b", dict(window=16, minibatch=16), 70),
    ("all blocks dynamic", dict(n_layers=2, n_dynamic=2), 60),
    ("one layer", dict(n_layers=1, n_dynamic=1), 50),
]


@pytest.mark.parametrize("name,over,T", EDGE, ids=[e[0] for e in EDGE])
def test_tiny_edge_cases(name, over, T):
    check(synth.config("tiny", **over), T=T)


def test_tiny_reset_and_repeat_is_bitwise_identical():
    """ttt_reset restores W0, clears the store and the position: a second
    prefill of the same stream gives the same losses and fast weights, bit
    for bit (no atomics or order-dependent sums on the path)."""
    import test_long_context_amd as tla
    c = synth.config("tiny", n_layers=3, n_kv_heads=2, n_dynamic=2, window=24, minibatch=16)
    w = to_device(synth.gen_weights(c))
    tok = synth.gen_tokens(c, n=120).cuda()
    m = tla.TTT(c, w, max_seq=120)
    runs = []
    for _ in range(2):
        m.reset()
        loss = m.prefill(tok)
        m.sync()
        runs.append((loss.cpu().numpy(), [tuple(x.cpu().numpy() for x in m.fast_weights(i)) for i in range(2)]))
    m.close()
    assert np.array_equal(runs[0][0], runs[1][0])
    for a, b in zip(runs[0][1], runs[1][1]):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
