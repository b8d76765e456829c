"""GPU parity of the bf16 path (bf16 storage, fp32 accumulation, fp32
fast-weight master) against the float32 oracle on the same bf16-valued
inputs. Tolerances: 2e-2 relative on per-token loss, 5e-2 on the final fast
weights measured against the update (max |W - W_ref| / max |W_ref - W0|)."""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import ttt_e2e as O
from tests.util import dw_err, rel_loss_err, ring_capacity, say, to_device

pytestmark = pytest.mark.gpu

LOSS_TOL = 2e-2
W_TOL = 5e-2
HERE = os.path.dirname(os.path.abspath(__file__))


def run_gpu(c, w, tok, max_seq=None):
    import test_long_context_amd as tla
    m = tla.TTT(c, w, max_seq=max_seq or tok.numel())
    loss = m.prefill(tok)
    m.sync()
    fw = [tuple(x.cpu().numpy() for x in m.fast_weights(i)) for i in range(len(w["dyn"]))]
    loss = loss.cpu().numpy()
    m.close()
    return loss, fw


def check(c, T):
    say(f"case: bf16 L={c['n_layers']} d={c['d_model']} H={c['n_heads']}/{c['n_kv_heads']}x{c['head_dim']} "
        f"F={c['ffn_hidden']} V={c['vocab']} k={c['window']} b={c['minibatch']} T={T}")
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c, n=T)
    loss, fw = run_gpu(c, to_device(w), tok.cuda())
    wn = synth.weights_to_numpy(w, np.float32)
    ref = O.ttt_inner_loop(c, wn, tok.numpy(), dtype=np.float32)
    le = rel_loss_err(loss, ref["loss"])
    errs = [dw_err(g, ref["dyn"][i][k], wn["dyn"][i][k])
            for i, gs in enumerate(fw) for k, g in zip(("w1", "w2", "w3"), gs)]
    say(f"  loss rel err {le:.3e}  max dW err {max(errs):.3e}  mean loss {loss.mean():.4f}")
    assert np.all(np.isfinite(loss))
    assert le < LOSS_TOL
    assert max(errs) < W_TOL


def test_bf16_small_gqa_dh128():
    c = synth.config("125m", n_layers=4, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128,
                     ffn_hidden=512, dyn_ffn_hidden=512, vocab=4096, window=256, minibatch=128,
                     n_dynamic=2, alpha=0.01)
    check(c, T=700)


def test_bf16_125m_full_sequence():
    check(synth.config("125m"), T=8192)


def test_bf16_1b_prefix_two_minibatches():
    check(synth.config("1b"), T=2 * 1024 + 1)


def test_generator_cpu_gpu_identical():
    """The counter-based generator gives the same bf16 weights on either device."""
    a = synth._normal_tensor(4, 101, (1 << 22,), 0.02, torch.bfloat16, "cpu")
    b = synth._normal_tensor(4, 101, (1 << 22,), 0.02, torch.bfloat16, "cuda").cpu()
    diff = int((a.view(torch.int16) != b.view(torch.int16)).sum())
    say(f"  generator bf16 mismatches: {diff} of {1 << 22}")
    assert diff <= 2
    ta = synth.gen_tokens(synth.config("3b"), n=1 << 16)
    tb = synth.gen_tokens(synth.config("3b"), n=1 << 16, device="cuda").cpu()
    assert torch.equal(ta, tb)


def check_fast_weights(m, g, nd, w, seq=0):
    """Fast weights after the last update against the stored oracle record:
    4096 sampled coordinates per matrix and, where stored, the maximum of
    |W_T - W0| over every row and every column (a wrong row or column moves
    its maximum whichever entries the samples hit). Errors are normalised by
    max |W_T - W0| over the matrix; |max|a| - max|b|| <= max|a - b|, so the
    extrema errors never exceed the full-matrix error."""
    errs, ext = [], []
    for i in range(nd):
        ws = m.fast_weights(i, seq=seq)
        for k, W in zip(("w1", "w2", "w3"), ws):
            den = float(g[f"d{i}_{k}_den"])
            idx = torch.from_numpy(g[f"d{i}_{k}_idx"]).cuda()
            got = W.reshape(-1)[idx].cpu().numpy().astype(np.float64)
            errs.append(float(np.max(np.abs(got - g[f"d{i}_{k}_val"]))) / den)
            if f"d{i}_{k}_rowmax" in g:
                w0 = w["dyn"][i][k]
                dW = (W.double() - w0.double()).abs()
                rmax = dW.amax(dim=1).cpu().numpy()
                cmax = dW.amax(dim=0).cpu().numpy()
                ext.append(max(float(np.max(np.abs(rmax - g[f"d{i}_{k}_rowmax"]))),
                               float(np.max(np.abs(cmax - g[f"d{i}_{k}_colmax"])))) / den)
        del ws
    return errs, ext


def check_stored(fname, workload, ntok, label, prefix_slab=0):
    """GPU prefill of the workload's first ntok tokens against values written
    by tests/golden/make_golden.py (oracle only): losses of every position and
    4096 sampled coordinates of every fast-weight matrix after the last
    update, normalised by max |W_T - W0| over the matrix (and the row and
    column maxima of the update where the file holds them); then any decode
    steps the file holds."""
    import test_long_context_amd as tla
    g = np.load(os.path.join(HERE, "golden", fname), allow_pickle=False)
    c = synth.config(workload, prefix_slab=prefix_slab)
    ndec = len(g["tokens"]) - int(g["prefill_len"]) if "prefill_len" in g else 0
    T = len(g["tokens"]) - ndec
    assert T == ntok(c)
    w = synth.gen_weights(c, device="cuda")
    tok = synth.gen_tokens(c, n=T + ndec, device="cuda")
    assert np.array_equal(tok.cpu().numpy(), g["tokens"])
    assert np.array_equal(w["embed"][:4, :8].float().cpu().numpy(), g["embed_head"])
    max_seq = c["seq"] + 1024 if not prefix_slab else T + ndec + 1
    cap = ring_capacity(c, max_seq)
    say(f"  {label}: ring of {cap} slots for {T + ndec} positions")
    m = tla.TTT(c, w, max_seq=max_seq)
    loss = m.prefill(tok[:T])
    m.sync()
    le = rel_loss_err(loss.cpu().numpy(), g["loss"])
    nd = c["n_dynamic"] or (c["n_layers"] - (3 * c["n_layers"]) // 4)
    errs, ext = check_fast_weights(m, g, nd, w)
    say(f"  {label}: loss rel err {le:.3e}  sampled W_T err {max(errs):.3e}"
        + (f"  row/col max err {max(ext):.3e}" if ext else ""))
    zerr = []
    for j in range(ndec):
        z = m.decode_step(tok[T + j:T + j + 1]).cpu().numpy().astype(np.float64)
        den = float(g[f"z{j}_absmax"])
        e_s = float(np.max(np.abs(z[g[f"z{j}_idx"]] - g[f"z{j}_val"]))) / den
        e_t = float(np.max(np.abs(z[g[f"z{j}_top_idx"]] - g[f"z{j}_top_val"]))) / den
        say(f"  {label} decode step {j} (slot {(T + j) % cap}): sampled logit err {e_s:.3e}  top-16 err {e_t:.3e}")
        assert np.all(np.isfinite(z))
        zerr.append((e_s, e_t, int(np.argmax(z)) in set(g[f"z{j}_top_idx"].tolist())))
    m.close()
    assert le < LOSS_TOL
    assert max(errs) < W_TOL
    assert not ext or max(ext) < W_TOL
    for e_s, e_t, top_ok in zerr:
        assert e_s < 2e-2 and e_t < 2e-2 and top_ok
    return cap


def _stored(fname):
    return pytest.mark.skipif(not os.path.exists(os.path.join(HERE, "golden", fname)),
                              reason="golden values not generated")


@_stored("ttt_3b_minibatch0.npz")
def test_bf16_3b_full_shape_first_minibatch_against_stored_oracle_values():
    """Full 3B shapes (bench launch configuration): mini-batch 0 of the 128K
    stream (1024 positions, one update) and the forward-only position 1024."""
    check_stored("ttt_3b_minibatch0.npz", "3b", lambda c: c["minibatch"] + 1, "3b mini-batch 0")


@_stored("ttt_3b_8minibatches.npz")
def test_bf16_3b_full_shape_eight_minibatches_against_stored_oracle_values():
    """Full 3B shapes: the first 8 mini-batches of the stream and their
    updates (each mini-batch under the previous one's fast weights)."""
    check_stored("ttt_3b_8minibatches.npz", "3b", lambda c: 8 * c["minibatch"] + 1, "3b 8 mini-batches")


@_stored("ttt_3b_16minibatches.npz")
def test_bf16_3b_full_shape_sixteen_minibatches_ring_reused_against_stored_oracle_values():
    """Full 3B shapes over the first 16 mini-batches: 8 that fill the
    8192-key window, then 8 with the window sliding across mini-batch edges
    (every query sees 8192 keys), the forward-only position 16384 and 3
    decode steps. A prefix slab of 1024 gives a 16384-slot ring, so position
    16384 and the decode steps reuse slots of positions 0..3 while the
    window reads across the wrap."""
    cap = check_stored("ttt_3b_16minibatches.npz", "3b", lambda c: 16 * c["minibatch"] + 1,
                       "3b 16 mini-batches", prefix_slab=1024)
    assert cap == 16384


@_stored("ttt_1b_full.npz")
def test_bf16_1b_full_sequence_against_stored_oracle_values():
    """The whole 1B-shape workload: 32768 tokens, 32 mini-batches and their
    updates."""
    check_stored("ttt_1b_full.npz", "1b", lambda c: c["seq"], "1b full sequence")


@_stored("ttt_3b_decode8k.npz")
def test_bf16_3b_decode_full_window_against_stored_oracle_values():
    """The decode workload's shape: after a TTT prefill of 8192 tokens of the
    3B stream (8 updates), decode steps over the full 8192-key window
    (captured graph, as timed). Sampled logits and the oracle's 16 largest
    logits within 2e-2 of max |z|; the GPU's top token is among the oracle's
    16 largest."""
    import test_long_context_amd as tla
    g = np.load(os.path.join(HERE, "golden", "ttt_3b_decode8k.npz"), allow_pickle=False)
    c = synth.config("3b")
    T = int(g["prefill_len"])
    ndec = len(g["tokens"]) - T
    w = synth.gen_weights(c, device="cuda")
    tok = synth.gen_tokens(c, n=T + ndec, device="cuda")
    assert np.array_equal(tok.cpu().numpy(), g["tokens"])
    assert np.array_equal(w["embed"][:4, :8].float().cpu().numpy(), g["embed_head"])
    m = tla.TTT(c, w, max_seq=T + ndec + 1)
    m.prefill(tok[:T])
    for j in range(ndec):
        z = m.decode_step(tok[T + j:T + j + 1]).cpu().numpy().astype(np.float64)
        den = float(g[f"z{j}_absmax"])
        e_s = float(np.max(np.abs(z[g[f"z{j}_idx"]] - g[f"z{j}_val"]))) / den
        e_t = float(np.max(np.abs(z[g[f"z{j}_top_idx"]] - g[f"z{j}_top_val"]))) / den
        say(f"  3b decode step {j}: sampled logit err {e_s:.3e}  top-16 err {e_t:.3e}")
        assert np.all(np.isfinite(z))
        assert e_s < 2e-2 and e_t < 2e-2
        assert int(np.argmax(z)) in set(g[f"z{j}_top_idx"].tolist())
    m.close()


def test_bf16_3b_shape_two_minibatches_repeat_bitwise():
    """Two prefills of the same 2049 tokens at the full 3B shapes (bench
    launch configuration: side streams, split-K partials, key-split
    attention) after ttt_reset give identical losses and fast weights, bit
    for bit: every sum on the path is taken in a fixed order."""
    import test_long_context_amd as tla
    c = synth.config("3b")
    T = 2 * c["minibatch"] + 1
    say(f"case: 3b shape, {T} tokens, two prefills")
    w = synth.gen_weights(c, device="cuda")
    tok = synth.gen_tokens(c, n=T, device="cuda")
    m = tla.TTT(c, w, max_seq=c["seq"] + 1024)
    runs = []
    for _ in range(2):
        m.reset()
        loss = m.prefill(tok)
        m.sync()
        runs.append((loss.clone(), [tuple(x.clone() for x in m.fast_weights(i)) for i in range(c["n_dynamic"])]))
    m.close()
    assert bool(torch.isfinite(runs[0][0]).all())
    assert torch.equal(runs[0][0], runs[1][0])
    for a, b in zip(runs[0][1], runs[1][1]):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_bf16_fused_update_kernel_option():
    """TTT_UPDATE_KERNEL=fused (one persistent launch for both update
    products of a block) against the oracle, with K = b = 1024 (update waves
    one tile behind the MFMA waves) and a ragged last mini-batch."""
    c = synth.config("125m", n_layers=4, d_model=512, n_heads=4, n_kv_heads=2, head_dim=128,
                     ffn_hidden=1024, dyn_ffn_hidden=1024, vocab=4096, window=1024, minibatch=1024,
                     n_dynamic=2, alpha=0.01)
    os.environ["TTT_UPDATE_KERNEL"] = "fused"
    os.environ["TTT_WEIGHT_ROUNDING"] = "nearest"  # the fused kernel writes the two-term copy
    try:
        check(c, T=2600)
    finally:
        del os.environ["TTT_UPDATE_KERNEL"]
        del os.environ["TTT_WEIGHT_ROUNDING"]


@pytest.mark.parametrize("workload", ["small", "1b"])
def test_bf16_two_term_working_copy_option(workload):
    """TTT_WEIGHT_ROUNDING=nearest: the working copy rounded to nearest plus a
    low term, both in the forward products (instead of one stochastically
    rounded copy)."""
    if workload == "small":
        c = synth.config("125m", n_layers=4, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128,
                         ffn_hidden=512, dyn_ffn_hidden=512, vocab=4096, window=256, minibatch=128,
                         n_dynamic=2, alpha=0.01)
        T = 700
    else:
        c, T = synth.config("1b"), 2 * 1024 + 1
    os.environ["TTT_WEIGHT_ROUNDING"] = "nearest"
    try:
        check(c, T=T)
    finally:
        del os.environ["TTT_WEIGHT_ROUNDING"]
