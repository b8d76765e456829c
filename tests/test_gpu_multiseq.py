"""GPU parity of the multi-sequence prefill (ttt_config.n_seq = B > 1).

B independent token streams run side by side, each with its own fast
weights, key/value window and losses: the products with frozen weights see
the B mini-batches as one block of B b rows, the products with fast weights
run as one batched launch, and the position-dependent kernels run per
sequence. Each sequence must match the oracle's single-sequence inner loop
on its own tokens at the usual tolerances: fp32 1e-5 (float64 oracle); bf16
2e-2 on losses and 5e-2 of the update on fast weights (float32 oracle on the
same bf16 values); last-position logits max |z - z_ref| / max |z_ref|.
B identical streams give bit-identical results (every kernel treats the
sequences alike), and the 3B shape's second sequence matches the stored
oracle values of its stream."""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import ttt_e2e as O
from tests.util import dw_err, rel_loss_err, say, to_device

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def streams(c, B, T):
    return torch.stack([synth.gen_tokens(c, n=T, seed=c["seed"] + 100 * j) for j in range(B)])


def gpu_multi(c, w, toks):
    import test_long_context_amd as tla
    B, T = toks.shape
    m = tla.TTT(dict(c, n_seq=B), to_device(w), max_seq=T + 1)
    last = torch.empty(B, c["vocab"], dtype=torch.float32, device="cuda")
    loss = m.prefill(toks.cuda(), last_logits=last)
    m.sync()
    nd = len(w["dyn"])
    fw = [[tuple(x.cpu().numpy() for x in m.fast_weights(i, seq=j)) for i in range(nd)] for j in range(B)]
    out = loss.cpu().numpy(), last.cpu().numpy(), fw
    m.close()
    return out


def check(c, B, T, loss_tol, w_tol, z_tol, dtype):
    say(f"multi-sequence case: B={B} L={c['n_layers']} d={c['d_model']} H={c['n_heads']}/{c['n_kv_heads']}"
        f"x{c['head_dim']} k={c['window']} b={c['minibatch']} slab={c.get('prefix_slab', 0)} "
        f"dtype={c['dtype']} T={T}")
    w = synth.gen_weights(c)
    toks = streams(c, B, T)
    loss, last, fw = gpu_multi(c, w, toks)
    assert loss.shape == (B, T - 1) and last.shape == (B, c["vocab"])
    wn = synth.weights_to_numpy(w, dtype)
    for j in range(B):
        ref = O.ttt_inner_loop(c, wn, toks[j].numpy(), dtype=dtype, keep_state=True)
        le = rel_loss_err(loss[j], ref["loss"])
        errs = [dw_err(g, ref["dyn"][i][k], wn["dyn"][i][k])
                for i, gs in enumerate(fw[j]) for k, g in zip(("w1", "w2", "w3"), gs)]
        zr = ref["last_logits"]
        ze = float(np.abs(last[j] - zr).max() / np.abs(zr).max())
        say(f"  sequence {j}: loss rel err {le:.3e}  max dW err {max(errs):.3e}  last logits {ze:.3e}")
        assert np.all(np.isfinite(loss[j]))
        assert le < loss_tol
        assert max(errs) < w_tol
        assert ze < z_tol


def test_tiny_fp32_three_sequences_ragged():
    # 150 = 9 mini-batches of 16 + 6: the ragged last mini-batch in every sequence
    check(synth.config("tiny"), B=3, T=150, loss_tol=1e-5, w_tol=1e-5, z_tol=1e-5, dtype=np.float64)


def test_tiny_fp32_gqa_two_dynamic_blocks_ring_reused():
    c = synth.config("tiny", n_layers=4, n_kv_heads=2, n_dynamic=2, window=24, minibatch=16, prefix_slab=16)
    check(c, B=2, T=150, loss_tol=1e-5, w_tol=1e-5, z_tol=1e-5, dtype=np.float64)


def test_bf16_small_gqa_dh128_two_sequences():
    c = synth.config("125m", n_layers=4, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128,
                     ffn_hidden=512, dyn_ffn_hidden=512, vocab=4096, window=256, minibatch=128,
                     n_dynamic=2, alpha=0.01)
    check(c, B=2, T=300, loss_tol=2e-2, w_tol=5e-2, z_tol=2e-2, dtype=np.float32)


def test_bf16_identical_sequences_bitwise_equal():
    import test_long_context_amd as tla
    c = synth.config("125m", n_layers=4, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128,
                     ffn_hidden=512, dyn_ffn_hidden=512, vocab=4096, window=256, minibatch=128,
                     n_dynamic=2, alpha=0.01)
    w = synth.gen_weights(c)
    t = synth.gen_tokens(c, n=400)
    loss, last, fw = gpu_multi(c, w, torch.stack([t, t, t]))
    for j in (1, 2):
        assert np.array_equal(loss[j], loss[0])
        assert np.array_equal(last[j], last[0])
        for a, b in zip(fw[j], fw[0]):
            for x, y in zip(a, b):
                assert np.array_equal(x, y)
    say(f"  3 identical sequences: losses, logits and fast weights bit-identical (mean loss {loss[0].mean():.4f})")


def test_bf16_3b_shape_two_sequences_second_against_stored_oracle_values():
    """3B shapes, B = 2: sequence 1 is the 128K workload's first 8193 tokens
    (8 mini-batches), checked against the oracle values stored for them;
    sequence 0 is another stream, checked against a single-sequence run of
    the same library on it (the products it shares a launch with see twice
    the rows)."""
    import test_long_context_amd as tla
    from tests.test_gpu_bf16 import LOSS_TOL, W_TOL, check_fast_weights
    fname = os.path.join(HERE, "golden", "ttt_3b_8minibatches.npz")
    if not os.path.exists(fname):
        pytest.skip("golden values not generated")
    g = np.load(fname, allow_pickle=False)
    c = synth.config("3b")
    T = len(g["tokens"])
    w = synth.gen_weights(c, device="cuda")
    t1 = synth.gen_tokens(c, n=T, device="cuda")
    assert np.array_equal(t1.cpu().numpy(), g["tokens"])
    t0 = synth.gen_tokens(c, n=T, device="cuda", seed=c["seed"] + 100)
    say(f"  3b two sequences: T={T}")
    m = tla.TTT(dict(c, n_seq=2), w, max_seq=T + 1)
    loss = m.prefill(torch.stack([t0, t1]))
    m.sync()
    nd = c["n_dynamic"] or (c["n_layers"] - (3 * c["n_layers"]) // 4)
    le = rel_loss_err(loss[1].cpu().numpy(), g["loss"])
    errs, ext = check_fast_weights(m, g, nd, w, seq=1)
    fw0 = [m.fast_weights(i, seq=0) for i in range(nd)]
    l0 = loss[0].cpu().numpy()
    m.close()
    del m
    m1 = tla.TTT(c, w, max_seq=T + 1)
    l0s = m1.prefill(t0).cpu().numpy()
    fws = [m1.fast_weights(i) for i in range(nd)]
    m1.sync()
    e0 = rel_loss_err(l0, l0s)
    d0 = max(float((a - b).abs().max() / (b - w["dyn"][i][k].float()).abs().max())
             for i in range(nd) for k, a, b in zip(("w1", "w2", "w3"), fw0[i], fws[i]))
    m1.close()
    say(f"  sequence 1 vs stored oracle: loss rel err {le:.3e}  sampled W_T err {max(errs):.3e}"
        + (f"  row/col max err {max(ext):.3e}" if ext else ""))
    say(f"  sequence 0 vs single-sequence run: loss rel err {e0:.3e}  W_T err {d0:.3e}")
    assert le < LOSS_TOL
    assert max(errs) < W_TOL
    assert not ext or max(ext) < W_TOL
    assert np.all(np.isfinite(l0))
    assert e0 < LOSS_TOL and d0 < W_TOL


def test_decode_refused_on_multi_sequence_context():
    import test_long_context_amd as tla
    c = synth.config("tiny")
    w = synth.gen_weights(c)
    m = tla.TTT(dict(c, n_seq=2), to_device(w), max_seq=64)
    m.prefill(streams(c, 2, 40).cuda())
    with pytest.raises(tla.TTTError) as ei:
        m.decode_step(torch.zeros(1, dtype=torch.int32, device="cuda"))
    assert ei.value.code == -2  # TTT_ERR_UNSUPPORTED
    m.close()
