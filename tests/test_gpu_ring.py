"""GPU parity with each layer's key/value ring reused several times within
one prefill, and decode continuing across the reuse.

The ring holds cap positions (slot = position mod cap); a small prefix slab
(ttt_config.prefix_slab) gives a small ring, so a short stream already
overwrites every slot several times: the RoPE/key scatter, the transposed
value store, the attention reads across the wrap and the decode's fused
projection-and-store all run on reused slots, as in the 128K workload.
Tolerances as in the other parity tests: fp32 1e-5 (float64 oracle), bf16
2e-2 on loss and 5e-2 of the update on fast weights (float32 oracle on the
same bf16 values); decode logits max |z - z_ref| / max |z_ref|."""
import numpy as np
import pytest

import synth
from oracle import ttt_e2e as O
from tests.util import dw_err, rel_loss_err, ring_capacity, say, to_device

pytestmark = pytest.mark.gpu


def prefill_and_decode(c, w, tok, T, ndec):
    import test_long_context_amd as tla
    m = tla.TTT(c, to_device(w), max_seq=T + ndec + 1)
    loss = m.prefill(tok[:T].cuda())
    zs = [m.decode_step(tok[T + j:T + j + 1].cuda()) for j in range(ndec)]
    m.sync()
    fw = [tuple(x.cpu().numpy() for x in m.fast_weights(i)) for i in range(len(w["dyn"]))]
    out = loss.cpu().numpy(), fw, [z.cpu().numpy() for z in zs]
    m.close()
    return out


def check(c, T, ndec, loss_tol, w_tol, z_tol, dtype, min_wraps):
    cap = ring_capacity(c, T + ndec + 1)
    wraps = (T + ndec) / cap
    say(f"ring case: L={c['n_layers']} d={c['d_model']} H={c['n_heads']}/{c['n_kv_heads']}x{c['head_dim']} "
        f"k={c['window']} b={c['minibatch']} slab={c['prefix_slab']} dtype={c['dtype']} T={T} "
        f"decode={ndec} cap={cap} wraps={wraps:.2f}")
    assert T >= min_wraps * cap, "the stream must reuse every ring slot"
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c, n=T + ndec)
    loss, fw, zs = prefill_and_decode(c, w, tok, T, ndec)
    wn = synth.weights_to_numpy(w, dtype)
    ref = O.ttt_inner_loop(c, wn, tok[:T].numpy(), dtype=dtype, keep_state=True)
    le = rel_loss_err(loss, ref["loss"])
    errs = [dw_err(g, ref["dyn"][i][k], wn["dyn"][i][k])
            for i, gs in enumerate(fw) for k, g in zip(("w1", "w2", "w3"), gs)]
    say(f"  loss rel err {le:.3e}  max dW err {max(errs):.3e}")
    assert np.all(np.isfinite(loss))
    assert le < loss_tol
    assert max(errs) < w_tol
    for j in range(ndec):
        r = O.decode_step(ref, int(tok[T + j]))
        e = float(np.abs(zs[j] - r).max() / np.abs(r).max())
        say(f"  decode step {j} (position {T + j}, slot {(T + j) % cap}): logit rel err {e:.3e}")
        assert np.all(np.isfinite(zs[j]))
        assert e < z_tol, (j, e)


def test_tiny_fp32_ring_reused_four_times():
    # cap = 128 for T = 512: every slot written four times
    c = synth.config("tiny", prefix_slab=16)
    check(c, T=512, ndec=5, loss_tol=1e-5, w_tol=1e-5, z_tol=1e-5, dtype=np.float64, min_wraps=3)


def test_tiny_fp32_gqa_ragged_ring_reused_three_times():
    # slab and mini-batch not multiples of the 64-position key tiles, a
    # ragged last mini-batch, two dynamic blocks and GQA
    c = synth.config("tiny", n_layers=4, n_kv_heads=2, n_dynamic=2, window=40, minibatch=24,
                     prefix_slab=40)
    check(c, T=410, ndec=4, loss_tol=1e-5, w_tol=1e-5, z_tol=1e-5, dtype=np.float64, min_wraps=3)


def test_bf16_gqa_dh128_ring_reused_twice():
    # the bf16 kernels (MFMA attention over the transposed value store);
    # slab 160 and b = 96 are not multiples of 64; cap = 512 for T = 1300
    c = synth.config("125m", n_layers=4, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128,
                     ffn_hidden=512, dyn_ffn_hidden=512, vocab=4096, window=256, minibatch=96,
                     n_dynamic=2, alpha=0.01, prefix_slab=160)
    check(c, T=1300, ndec=4, loss_tol=2e-2, w_tol=5e-2, z_tol=2e-2, dtype=np.float32, min_wraps=2)


def test_bf16_dh64_window_equal_minibatch_ring_reused_twice():
    # dh 64 kernels; window = b, so a query's keys span two mini-batches
    c = synth.config("125m", n_layers=3, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
                     ffn_hidden=512, dyn_ffn_hidden=256, vocab=2048, window=128, minibatch=128,
                     n_dynamic=1, alpha=0.01, prefix_slab=128)
    check(c, T=900, ndec=3, loss_tol=2e-2, w_tol=5e-2, z_tol=2e-2, dtype=np.float32, min_wraps=2)
