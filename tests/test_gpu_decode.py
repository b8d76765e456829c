"""GPU parity of ttt_decode_step: after a TTT prefill of T tokens, each
decode step is the forward of one new position under the adapted fast
weights, with the window's keys/values from the store, and no update. The
reference is the oracle's decode on its own prefill state (float64 for the
fp32 workload, float32 on the same bf16 values for bf16). Logit error is
max |z - z_ref| / max |z_ref| per step: 1e-5 (fp32), 2e-2 (bf16)."""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import ttt_e2e as O
from tests.util import say, to_device

pytestmark = pytest.mark.gpu


def gpu_decode(c, w, tok, T, ndec):
    import test_long_context_amd as tla
    m = tla.TTT(c, to_device(w), max_seq=T + ndec + 1)
    m.prefill(tok[:T].cuda())
    out = []
    for j in range(ndec):
        out.append(m.decode_step(tok[T + j:T + j + 1].cuda()).cpu().numpy())
    m.sync()
    m.close()
    return out


def oracle_decode(c, w, tok, T, ndec, dtype):
    wn = synth.weights_to_numpy(w, dtype)
    st = O.ttt_inner_loop(c, wn, tok[:T].numpy(), dtype=dtype, keep_state=True)
    return [O.decode_step(st, int(tok[T + j])) for j in range(ndec)]


def check(c, T, ndec, tol, dtype):
    say(f"decode case: L={c['n_layers']} d={c['d_model']} H={c['n_heads']}/{c['n_kv_heads']}x{c['head_dim']} "
        f"k={c['window']} b={c['minibatch']} dtype={c['dtype']} T={T} steps={ndec}")
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c, n=T + ndec)
    got = gpu_decode(c, w, tok, T, ndec)
    ref = oracle_decode(c, w, tok, T, ndec, dtype)
    for j, (g, r) in enumerate(zip(got, ref)):
        e = float(np.abs(g - r).max() / np.abs(r).max())
        say(f"  step {j}: logit rel err {e:.3e}")
        assert np.all(np.isfinite(g))
        assert e < tol, (j, e)
    return got


def test_decode_tiny_fp32():
    check(synth.config("tiny"), T=64, ndec=6, tol=1e-5, dtype=np.float64)


def test_decode_tiny_ragged_gqa_two_dynamic_blocks():
    c = synth.config("tiny", n_layers=4, n_kv_heads=2, n_dynamic=2, window=24, minibatch=16)
    check(c, T=150, ndec=4, tol=1e-5, dtype=np.float64)


def test_decode_graph_replays_match_eager():
    """The captured launch sequence, replayed step after step, gives the same
    logits as launching it eagerly."""
    c = synth.config("tiny", n_layers=3, n_kv_heads=2, n_dynamic=1, window=32, minibatch=16)
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c, n=100)
    a = gpu_decode(c, w, tok, 90, 8)
    os.environ["TTT_DECODE_GRAPH"] = "0"
    try:
        b = gpu_decode(c, w, tok, 90, 8)
    finally:
        del os.environ["TTT_DECODE_GRAPH"]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_decode_bf16_small_gqa_dh128():
    c = synth.config("125m", n_layers=4, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128,
                     ffn_hidden=512, dyn_ffn_hidden=512, vocab=4096, window=256, minibatch=128,
                     n_dynamic=2, alpha=0.01)
    check(c, T=700, ndec=3, tol=2e-2, dtype=np.float32)


def test_decode_bf16_125m():
    check(synth.config("125m"), T=1500, ndec=2, tol=2e-2, dtype=np.float32)


def test_decode_needs_prefill():
    import test_long_context_amd as tla
    c = synth.config("tiny")
    w = synth.gen_weights(c)
    m = tla.TTT(c, to_device(w), max_seq=64)
    with pytest.raises(tla.TTTError) as ei:
        m.decode_step(torch.zeros(1, dtype=torch.int32, device="cuda"))
    assert ei.value.code == -5  # TTT_ERR_STATE
    m.close()


# ------------------------------------------------------- decode with updates
def check_updates(c, T, N, tol_z, tol_l, tol_w, dtype):
    """Prefill T tokens, then decode with updates through position N - 1,
    against the oracle's decode_step_update on its own prefill state: logits
    of every step, the losses of every update, and the final fast weights
    (update-normalised)."""
    import test_long_context_amd as tla
    from tests.util import dw_err
    say(f"decode-update case: L={c['n_layers']} d={c['d_model']} H={c['n_heads']}/{c['n_kv_heads']}x{c['head_dim']} "
        f"b={c['minibatch']} dtype={c['dtype']} T={T} N={N}")
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c, n=N)
    m = tla.TTT(c, to_device(w), max_seq=N + 1)
    m.prefill(tok[:T].cuda())
    got = []
    for p in range(T, N):
        z, l = m.decode_step_update(tok[p:p + 1].cuda())
        got.append((z.cpu().numpy(), None if l is None else l.cpu().numpy()))
    m.sync()
    fw = [tuple(x.cpu().numpy() for x in m.fast_weights(i)) for i in range(len(w["dyn"]))]
    m.close()
    wn = synth.weights_to_numpy(w, dtype)
    st = O.ttt_inner_loop(c, wn, tok[:T].numpy(), dtype=dtype, keep_state=True)
    n_upd = 0
    for j, p in enumerate(range(T, N)):
        zr, lr = O.decode_step_update(st, int(tok[p]))
        zg, lg = got[j]
        e = float(np.abs(zg - zr).max() / np.abs(zr).max())
        assert np.all(np.isfinite(zg))
        assert (lg is None) == (lr is None), p
        if lr is not None:
            el = float(np.max(np.abs(lg - lr) / np.abs(lr)))
            say(f"  update before position {p}: loss rel err {el:.3e}; logit rel err {e:.3e}")
            assert el < tol_l
            n_upd += 1
        assert e < tol_z, (p, e)
    errs = [dw_err(g, st["dyn"][i][k], wn["dyn"][i][k])
            for i, gs in enumerate(fw) for k, g in zip(("w1", "w2", "w3"), gs)]
    say(f"  {n_upd} updates; final fast weights err {max(errs):.3e}")
    assert n_upd >= 2
    assert max(errs) < tol_w


def test_decode_updates_tiny_fp32():
    # T = 2b + 1: the decode-time mini-batches continue the prefill's tiling
    c = synth.config("tiny")
    check_updates(c, T=33, N=81, tol_z=1e-5, tol_l=1e-5, tol_w=1e-5, dtype=np.float64)


def test_decode_updates_tiny_fp32_gqa_off_grid():
    # a prefill length that does not end a mini-batch; GQA, two dynamic blocks
    c = synth.config("tiny", n_layers=4, n_kv_heads=2, n_dynamic=2, window=24, minibatch=16)
    check_updates(c, T=50, N=99, tol_z=1e-5, tol_l=1e-5, tol_w=1e-5, dtype=np.float64)


def test_decode_updates_bf16_small_gqa_dh128():
    c = synth.config("125m", n_layers=4, d_model=256, n_heads=4, n_kv_heads=2, head_dim=128,
                     ffn_hidden=512, dyn_ffn_hidden=512, vocab=4096, window=256, minibatch=128,
                     n_dynamic=2, alpha=0.01)
    check_updates(c, T=300, N=560, tol_z=2e-2, tol_l=2e-2, tol_w=5e-2, dtype=np.float32)
