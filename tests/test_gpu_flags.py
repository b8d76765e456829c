"""Device-detected conditions reported by ttt_sync (include/ttt.h): a token
id outside [0, vocab) raises TTT_ERR_TOKEN_RANGE, a non-finite loss raises
TTT_ERR_NONFINITE. The kernels that read token ids bound-check them (a bad
input row is zeroed, a bad label gives a NaN loss and no one-hot term), so
these inputs never lead to an out-of-range access; the flags are cleared by
the sync that reports them."""
import numpy as np
import pytest
import torch

import synth
from tests.util import say, to_device

pytestmark = pytest.mark.gpu

TOKEN_RANGE, NONFINITE = -6, -7


def _ctx(c, w, max_seq):
    import test_long_context_amd as tla
    return tla, tla.TTT(c, to_device(w), max_seq=max_seq)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bad", [-1, "vocab"])
def test_out_of_range_token_in_prefill_is_reported(dtype, bad):
    if dtype == "f32":
        c = synth.config("tiny")
    else:
        c = synth.config("125m", n_layers=2, d_model=256, n_heads=2, n_kv_heads=2, head_dim=128,
                         ffn_hidden=256, dyn_ffn_hidden=256, vocab=1024, window=64, minibatch=64,
                         n_dynamic=1)
    T = 100
    bad_id = c["vocab"] if bad == "vocab" else bad
    say(f"flag case: {dtype} token {bad_id} at position 37 of {T}")
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c, n=T)
    tok[37] = bad_id
    tla, m = _ctx(c, w, T + 4)
    loss = m.prefill(tok.cuda())
    with pytest.raises(tla.TTTError) as ei:
        m.sync()
    assert ei.value.code == TOKEN_RANGE
    m.sync()   # reported once, then cleared
    lc = loss.cpu().numpy()
    # position 36 predicts the bad id: no loss is defined there
    assert np.isnan(lc[36])
    keep = np.ones(T - 1, bool)
    keep[36] = False
    assert np.all(np.isfinite(lc[keep]))
    for i in range(len(w["dyn"])):
        assert all(bool(torch.isfinite(x).all()) for x in m.fast_weights(i))
    # a decode step with a bad id is reported the same way
    m.decode_step(torch.tensor([bad_id], dtype=torch.int32, device="cuda"))
    with pytest.raises(tla.TTTError) as ei:
        m.sync()
    assert ei.value.code == TOKEN_RANGE
    m.decode_step(tok[T - 1:T].cuda())
    m.sync()
    m.close()


def test_nonfinite_loss_is_reported():
    """An infinite embedding row turns every later activation of that
    position into NaN (RMSNorm of an infinite row), so its loss is not
    finite."""
    c = synth.config("tiny")
    T = 48
    w = synth.gen_weights(c)
    tok = synth.gen_tokens(c, n=T)
    w["embed"][int(tok[T - 2])] = float("inf")
    tla, m = _ctx(c, w, T)
    m.prefill(tok.cuda())
    with pytest.raises(tla.TTTError) as ei:
        m.sync()
    assert ei.value.code == NONFINITE
    m.sync()
    m.close()
